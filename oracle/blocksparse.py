"""fp64 reference for block-sparse attention.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package: imported by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
product path).

A block mask removes whole (query block, key block) rectangles from the
attention pattern -- the block-sparse extension that the glossary page
("Flash Attention", FAQ on block-sparse extensions) sets apart from the
dense exact computation.  What remains is computed exactly: the plain
definition of attention with the mask

    visible(i, j) = block_mask[i // block, j // block] != 0
                    and (not causal or j <= i)

(the causal rule keeps its top-left meaning), softmax over each row's
visible keys, O = P V.  A row that sees no key has no softmax; its output
row is 0 and its lse -inf, the same convention as a key range that a row
does not see (``splitkv``).  Written plainly: the full score matrix is built
and masked, numpy's exp/log act as single steps.
"""

import numpy as np

from .attention import visible_mask


def block_visible(block_mask, Lq, Lk, block, causal):
    """[Lq, Lk] boolean matrix of visible (query, key) pairs for one slice's
    [ceil(Lq/block), ceil(Lk/block)] block mask."""
    bm = np.asarray(block_mask) != 0
    nqb, nkb = -(-Lq // block), -(-Lk // block)
    if bm.shape != (nqb, nkb):
        raise ValueError(f"block mask must be [{nqb}, {nkb}]")
    rows = np.arange(Lq) // block
    cols = np.arange(Lk) // block
    return bm[rows[:, None], cols[None, :]] & visible_mask(Lq, Lk, causal)


def attn_fwd_blocksparse(q, k, v, scale, causal, block_mask, block=128):
    """Attention over the pairs a block mask keeps.

    q [B,H,Lq,d], k [B,H,Lk,d], v [B,H,Lk,dv]; block_mask [nqb, nkb] shared
    by every slice or [B, H, nqb, nkb].  Returns (O [B,H,Lq,dv],
    lse [B,H,Lq]) in float64; rows with no visible key get O = 0 and
    lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, _ = q.shape
    Lk = k.shape[2]
    bm = np.asarray(block_mask)
    O = np.zeros((B, H, Lq, v.shape[3]))
    lse = np.full((B, H, Lq), -np.inf)
    for b in range(B):
        for h in range(H):
            vis = block_visible(bm if bm.ndim == 2 else bm[b, h], Lq, Lk, block, causal)
            seen = vis.any(axis=1)
            S = np.where(vis, scale * (q[b, h] @ k[b, h].T), -np.inf)[seen]
            m = S.max(axis=1, keepdims=True)
            lse_r = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
            O[b, h][seen] = np.exp(S - lse_r[:, None]) @ v[b, h]
            lse[b, h][seen] = lse_r
    return O, lse


def attn_bwd_blocksparse(q, k, v, dO, scale, causal, block_mask, block=128):
    """Gradients of <dO, O> for block-sparse attention.

    The chain rule through the definition above (the same formulas as the
    dense backward, with P zero outside the kept pairs): D_i = sum_c dO_ic
    O_ic, dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K,
    dK = scale dS^T Q.  A row that sees no key has P = 0 and contributes
    nothing.  Returns (dq, dk, dv) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, H, Lq, _ = q.shape
    Lk = k.shape[2]
    bm = np.asarray(block_mask)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            vis = block_visible(bm if bm.ndim == 2 else bm[b, h], Lq, Lk, block, causal)
            seen = vis.any(axis=1)
            S = np.where(vis, scale * (q[b, h] @ k[b, h].T), -np.inf)
            P = np.zeros((Lq, Lk))
            m = S[seen].max(axis=1, keepdims=True)
            lse = m[:, 0] + np.log(np.exp(S[seen] - m).sum(axis=1))
            P[seen] = np.exp(S[seen] - lse[:, None])
            O = P @ v[b, h]
            D = (dO[b, h] * O).sum(axis=1)
            dv[b, h] = P.T @ dO[b, h]
            dP = dO[b, h] @ v[b, h].T
            dS = P * (dP - D[:, None])
            dq[b, h] = scale * (dS @ k[b, h])
            dk[b, h] = scale * (dS.T @ q[b, h])
    return dq, dk, dv
