"""The blockwise recurrence the method runs is exact: an fp64 model of it,
over random key-block splits, equals the oracle's plain definition.

The recurrence follows the annotated-code page "How Flash Attention Improves
Transformer Memory Efficiency ...", section "The Three Running Statistics":
per query row a running max m, a running sum l rescaled by exp(m_old - m_new)
and an unnormalised output rescaled the same way, divided by l at the end;
lse = m + log l.  The first block of a row may be fully masked (m still
-inf); that case takes the rescale factor as 0 instead of exp(-inf + inf).
CPU only.
"""

import numpy as np
import pytest

import oracle


def _blockwise_head(q, k, v, scale, causal, cuts):
    Lq, Lk = q.shape[0], k.shape[0]
    m = np.full(Lq, -np.inf)
    l = np.zeros(Lq)
    acc = np.zeros((Lq, v.shape[1]))
    bounds = [0] + sorted(cuts) + [Lk]
    for a, b in zip(bounds[:-1], bounds[1:]):
        if a == b:
            continue
        S = scale * (q @ k[a:b].T)
        if causal:
            S = np.where(np.arange(a, b)[None, :] <= np.arange(Lq)[:, None], S, -np.inf)
        m_new = np.maximum(m, S.max(axis=1))
        base = np.where(np.isfinite(m_new), m_new, 0.0)
        p = np.exp(S - base[:, None])
        alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[a:b]
        m = m_new
    return acc / l[:, None], m + np.log(l)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_blockwise_recurrence_equals_definition(causal, seed):
    rng = np.random.default_rng(seed)
    Lq = int(rng.integers(1, 40))
    Lk = Lq if causal else int(rng.integers(1, 40))
    d = int(rng.integers(1, 9))
    q, k, v = (rng.standard_normal((1, 2, n, d)) * 2 for n in (Lq, Lk, Lk))
    scale = float(rng.uniform(0.1, 1.5))
    O, lse = oracle.attn_fwd(q, k, v, scale, causal)
    for trial in range(4):
        cuts = list(rng.integers(0, Lk + 1, size=int(rng.integers(0, 6))))
        for h in range(2):
            Ob, lb = _blockwise_head(q[0, h], k[0, h], v[0, h], scale, causal, cuts)
            np.testing.assert_allclose(Ob, O[0, h], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lb, lse[0, h], rtol=0, atol=1e-12)


def test_fully_masked_first_block_is_handled():
    # Causal, keys split so that row 0's later blocks are fully masked and
    # the row-max stays -inf until a visible key arrives for late rows.
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((1, 1, 12, 4)) for _ in range(3))
    O, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    Ob, lb = _blockwise_head(q[0, 0][::-1], k[0, 0], v[0, 0], 0.5, False, [3, 7])
    # Reversed query order with a non-causal model is just a row permutation.
    O2, l2 = oracle.attn_fwd(q[:, :, ::-1], k, v, 0.5, False)
    np.testing.assert_allclose(Ob, O2[0, 0], atol=1e-12)
    # And the causal model with every split point agrees with the definition.
    Oc, lc = _blockwise_head(q[0, 0], k[0, 0], v[0, 0], 0.5, True, list(range(1, 12)))
    np.testing.assert_allclose(Oc, O[0, 0], atol=1e-12)
    np.testing.assert_allclose(lc, lse[0, 0], atol=1e-12)
