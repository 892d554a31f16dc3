"""Helpers for the GPU parity tests: device transfer, error metrics and the
tolerances the kernels must meet against the fp64 oracle.

Tolerances (bf16 inputs, fp32 accumulation): max |dO| <= 1e-2 and mean
|dO| <= 1e-3 over all compared elements, max |d lse| <= 1e-3, and for
gradients max |dX - dX_ref| / max |dX_ref| <= 2e-2.  fp32 path: max |d| /
max |ref| <= 1e-5 for every output.
"""

import sys

import numpy as np
import pytest
import torch

from workloads import to_f64

BF16_O_MAX = 1e-2
BF16_O_MEAN = 1e-3
BF16_LSE_MAX = 1e-3
BF16_GRAD_REL = 2e-2
F32_REL = 1e-5


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda", 0)


def announce(msg):
    """Name the case on the real stderr before a GPU step (survives capture)."""
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def to_dev(*ts):
    dev = device()
    return tuple(t.to(dev).contiguous() for t in ts)


def fwd_errors(O, lse, O_ref, lse_ref):
    O = np.asarray(O, np.float64)
    d = np.abs(O - O_ref)
    return dict(o_max=float(d.max()) if d.size else 0.0,
                o_mean=float(d.mean()) if d.size else 0.0,
                lse_max=float(np.abs(np.asarray(lse, np.float64) - lse_ref).max()) if d.size else 0.0)


def assert_bf16_fwd(errs, what):
    assert errs["o_max"] <= BF16_O_MAX, f"{what}: max|dO| {errs}"
    assert errs["o_mean"] <= BF16_O_MEAN, f"{what}: mean|dO| {errs}"
    assert errs["lse_max"] <= BF16_LSE_MAX, f"{what}: max|dlse| {errs}"


def rel_to_max(x, ref, floor=1e-9):
    """max |x - ref| / max |ref|.  A reference that is zero up to fp64
    round-off (below ``floor``, e.g. dQ with a single key) is compared in
    absolute terms instead: the quotient would only measure round-off."""
    x = np.asarray(x, np.float64)
    m = np.abs(ref).max() if np.size(ref) else 0.0
    d = np.abs(x - ref).max() if np.size(ref) else 0.0
    return float(d / m) if m > floor else float(d)


def f64(t):
    return to_f64(t)
