"""fp64 reference for attention computed over separate key ranges and merged.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package: imported by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
product path).

The decode shape -- a few query rows against a long key sequence, the phase
the blog page ("What Is FlashAttention? ...", section "What it changes for
you") and the explainer page ("Flash attention explained", section "Why this
pattern keeps recurring") single out as bound by memory traffic rather than
arithmetic -- is parallelised over key ranges.  Two definitions are needed
to check it:

* The result of one key range [k0, k1).  It is the attention of the plain
  definition with every key outside the range treated as masked: the same
  S = scale * Q K^T, the same top-left causal rule on *absolute* key indices
  (key j visible to row i iff j <= i), softmax over what stays visible.  A row
  that sees no key of the range has no softmax; its output row is taken as 0
  and its lse as -inf, the values that give it weight zero below.
* The merge.  The softmax normaliser of the whole key set is the sum of the
  per-range ones, exp(lse) = sum_s exp(lse_s), and the output is the average
  of the per-range outputs weighted by their share of it,
  O = sum_s exp(lse_s - lse) O_s.  This is the running-statistics recurrence
  of the annotated-code page ("How Flash Attention Improves Transformer
  Memory Efficiency ...", section "The Three Running Statistics") applied
  once over finished ranges instead of tile by tile: m is the larger of the
  per-range maxima, l the sum of the l_s rescaled by exp(m_s - m), and
  lse = m + log l.

Both are written plainly: the full score matrix is built and masked, numpy's
exp/log act as single steps.
"""

import numpy as np

from .attention import visible_mask


def attn_fwd_keyrange(q, k, v, scale, causal, k0, k1):
    """Attention of every query row over the keys [k0, k1) only.

    q [B,H,Lq,d], k [B,H,Lk,d], v [B,H,Lk,dv]; 0 <= k0 <= k1 <= Lk.  The causal
    rule compares absolute indices (key j visible to row i iff j <= i).
    Returns (O [B,H,Lq,dv], lse [B,H,Lq]) in float64; rows with no visible
    key in the range get O = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, _ = q.shape
    Lk = k.shape[2]
    if not (0 <= k0 <= k1 <= Lk):
        raise ValueError("key range outside [0, Lk]")
    vis = visible_mask(Lq, Lk, causal)
    in_range = np.zeros(Lk, dtype=bool)
    in_range[k0:k1] = True
    vis = vis & in_range[None, :]
    seen = vis.any(axis=1)                      # rows with at least one key
    O = np.zeros((B, H, Lq, v.shape[3]))
    lse = np.full((B, H, Lq), -np.inf)
    for b in range(B):
        for h in range(H):
            S = np.where(vis, scale * (q[b, h] @ k[b, h].T), -np.inf)[seen]
            m = S.max(axis=1, keepdims=True)
            lse_r = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
            P = np.exp(S - lse_r[:, None])
            O[b, h][seen] = P @ v[b, h]
            lse[b, h][seen] = lse_r
    return O, lse


def merge_partials(O_parts, lse_parts):
    """Combine the results of disjoint key ranges into the whole.

    O_parts [S,B,H,Lq,dv], lse_parts [S,B,H,Lq] (natural log; -inf marks a
    range that a row does not see).  Every row must see at least one range.
    Returns (O [B,H,Lq,dv], lse [B,H,Lq]).
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)                    # largest per-range normaliser
    if not np.all(np.isfinite(m)):
        raise ValueError("a row sees no key in any range")
    l = np.exp(lse_parts - m).sum(axis=0)        # exp(-inf) = 0 drops unseen ranges
    lse = m + np.log(l)
    w = np.exp(lse_parts - lse)                  # each range's share, summing to 1
    O = (w[..., None] * O_parts).sum(axis=0)
    return O, lse
