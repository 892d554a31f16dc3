"""The fp64 oracle against its pins (closed forms, special cases, invariants,
finite differences and PyTorch's CPU fp64 attention).  CPU only."""

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_rejects_zero_keys():
    q = np.zeros((1, 1, 3, 2))
    k = np.zeros((1, 1, 0, 2))
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, k, k, 1.0, False)


def test_visible_mask_top_left():
    m = oracle.visible_mask(3, 5, True)
    assert m.tolist() == [[True, False, False, False, False],
                          [True, True, False, False, False],
                          [True, True, True, False, False]]
    assert oracle.visible_mask(2, 2, False).all()
