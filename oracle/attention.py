"""fp64 reference attention (forward and backward) by the plain definition.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What is computed, per (batch, head) slice, with every value in float64:

* Scores.  S = scale * Q K^T, an L_q x L_k matrix ("How Flash Attention
  Improves Transformer Memory Efficiency ...", section "Full Matrix
  Construction"; the scale argument is the one passed next to ``causal`` in
  that page's usage example, section "Basic Flash Attention Forward Pass").
* Mask.  With ``causal`` the query in row i may not see key j > i; such
  entries become -inf so their probability is exactly zero (glossary page,
  FAQ "Does it remove the need for attention masks?" and related term
  "causal mask").  Rows and keys are aligned top-left, so every row sees key 0.
* Softmax.  lse_i = log sum_j exp(S_ij) over the visible keys (natural log),
  P = exp(S - lse) so each row of P sums to one; this is the normaliser that
  the blockwise method's running max m and running sum l reconstruct
  (annotated-code page, section "The Three Running Statistics": O_i is the
  accumulator divided by l_i; lse = m + log l).
* Output.  O = P V ("What Is FlashAttention?", section "The problem it
  solves": multiply the normalised scores by the values).
* Backward, for the loss <dO, O>.  The pages name only the recompute and the
  row statistic D_i (annotated-code page, section "Backward Pass
  Efficiency"); the formulas are the chain rule through the definitions
  above:  D_i = sum_c dO_ic O_ic,  dV = P^T dO,  dP = dO V^T,
  dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.

The matrices S and P are materialised on purpose: this is the "standard
attention" the method must reproduce exactly, not the blockwise method.
Library matrix products and numpy's exp/log are used as single steps; there
is no blocking, fusion or reordering beyond the definition.
"""

import numpy as np


def visible_mask(Lq, Lk, causal):
    """Boolean [Lq, Lk] matrix: True where query row i may attend to key j.

    Non-causal: every key is visible.  Causal: key j is visible to row i iff
    j <= i (the mask removes the keys that come after the query; rows and keys
    are aligned at index 0).
    """
    if not causal:
        return np.ones((Lq, Lk), dtype=bool)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= i


def _scores(q, k, scale):
    """S = scale * q k^T for one head: q [Lq, d], k [Lk, d] -> [Lq, Lk]."""
    return scale * (q @ k.T)


def _apply_mask(S, vis):
    """Masked-out scores become -inf, so exp() of them is exactly 0."""
    return np.where(vis, S, -np.inf)


def _row_logsumexp(S):
    """Natural-log log-sum-exp of every row of S, shifted by the row max.

    Every row must hold at least one finite entry (true for top-left causal
    masks whenever there is at least one key).
    """
    m = S.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(S - m).sum(axis=1))


def _probabilities(S, lse):
    """Row softmax written through the log-sum-exp: P = exp(S - lse)."""
    return np.exp(S - lse[:, None])


def _head_forward(q, k, v, scale, vis):
    """Forward for one (batch, head) slice.  Returns (O, lse, P)."""
    S = _apply_mask(_scores(q, k, scale), vis)
    lse = _row_logsumexp(S)
    P = _probabilities(S, lse)
    return P @ v, lse, P


def _head_backward(q, k, v, dO, scale, vis):
    """Gradients of <dO, O> for one slice.  Returns (dq, dk, dv)."""
    O, _, P = _head_forward(q, k, v, scale, vis)
    D = (dO * O).sum(axis=1)
    dv = P.T @ dO
    dP = dO @ v.T
    dS = P * (dP - D[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return dq, dk, dv


def _check(q, k, v):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    if k.shape[:3] != v.shape[:3] or q.shape[:2] != k.shape[:2]:
        raise ValueError("q, k, v shapes disagree")
    if q.shape[3] != k.shape[3]:
        raise ValueError("q and k need the same head dimension")
    if k.shape[2] == 0:
        raise ValueError("attention over zero keys is undefined")
    return q, k, v


def attn_fwd(q, k, v, scale, causal):
    """Exact attention forward.

    q [B,H,Lq,d], k [B,H,Lk,d], v [B,H,Lk,dv] (anything numpy converts).
    Returns (O [B,H,Lq,dv], lse [B,H,Lq]) in float64; lse is natural-log.
    """
    q, k, v = _check(q, k, v)
    B, H, Lq, _ = q.shape
    Lk = k.shape[2]
    vis = visible_mask(Lq, Lk, causal)
    O = np.empty((B, H, Lq, v.shape[3]))
    lse = np.empty((B, H, Lq))
    for b in range(B):
        for h in range(H):
            O[b, h], lse[b, h], _ = _head_forward(q[b, h], k[b, h], v[b, h], scale, vis)
    return O, lse


def attn_fwd_rows(q, k, v, scale, causal, rows):
    """Forward for selected query rows only.

    ``rows`` is an integer array [B, H, R]: the query rows to compute in each
    slice.  Each selected row is the full fp64 row over all keys it may see,
    identical to the same row of :func:`attn_fwd`.  Returns
    (O [B,H,R,dv], lse [B,H,R]).
    """
    q, k, v = _check(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    B, H, Lq, _ = q.shape
    Lk = k.shape[2]
    if rows.ndim != 3 or rows.shape[:2] != (B, H):
        raise ValueError("rows must be [B, H, R]")
    if rows.size and (rows.min() < 0 or rows.max() >= Lq):
        raise ValueError("row index out of range")
    vis_all = visible_mask(Lq, Lk, causal)
    R = rows.shape[2]
    O = np.empty((B, H, R, v.shape[3]))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            r = rows[b, h]
            O[b, h], lse[b, h], _ = _head_forward(q[b, h][r], k[b, h], v[b, h], scale, vis_all[r])
    return O, lse


def attn_bwd(q, k, v, dO, scale, causal):
    """Exact attention backward for the loss <dO, O>.

    Returns (dq [B,H,Lq,d], dk [B,H,Lk,d], dv [B,H,Lk,dv]) in float64.
    """
    q, k, v = _check(q, k, v)
    dO = np.asarray(dO, dtype=np.float64)
    B, H, Lq, _ = q.shape
    Lk = k.shape[2]
    if dO.shape != (B, H, Lq, v.shape[3]):
        raise ValueError("dO must match the output shape")
    vis = visible_mask(Lq, Lk, causal)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _head_backward(
                q[b, h], k[b, h], v[b, h], dO[b, h], scale, vis)
    return dq, dk, dv


def attn_bwd_heads(q, k, v, dO, scale, causal, heads):
    """Backward for selected (batch, head) slices only.

    ``heads`` is a sequence of (b, h) pairs.  Returns three arrays
    [n, L, d] stacked in the order given; each slice equals the same slice
    of :func:`attn_bwd`.
    """
    q, k, v = _check(q, k, v)
    dO = np.asarray(dO, dtype=np.float64)
    Lq, Lk = q.shape[2], k.shape[2]
    vis = visible_mask(Lq, Lk, causal)
    out = [_head_backward(q[b, h], k[b, h], v[b, h], dO[b, h], scale, vis)
           for (b, h) in heads]
    return (np.stack([o[0] for o in out]), np.stack([o[1] for o in out]),
            np.stack([o[2] for o in out]))
