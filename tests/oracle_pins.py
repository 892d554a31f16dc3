"""Checks that pin the fp64 oracle to facts other than its own code.

Each ``pin_*`` function takes the oracle module and raises AssertionError if
a fact fixed by the mathematics or by the source pages does not hold.  The
same functions run against the real oracle (tests/test_oracle.py, all must
pass) and against copies of it with a planted mistake
(tests/test_oracle_mutants.py, at least one must fail per mistake).

Kinds of pin: hand-derived closed forms (tests/golden/closed_forms.json),
special cases (one key, causal row 0, constant values, zero scale, a key
that wins by a margin of 800), bounds, symmetries (key/value permutation,
shifts), the blockwise merge identity, PyTorch's own CPU fp64 attention and
autograd as an independent library routine, central finite differences, and
gradient invariants (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i).
"""

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B, H, Lq, Lk, d, dv=None):
    r = _rng(seed)
    dv = d if dv is None else dv
    return (r.standard_normal((B, H, Lq, d)), r.standard_normal((B, H, Lk, d)),
            r.standard_normal((B, H, Lk, dv)))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, np.max(np.abs(b)) if b.size else 0.0)
    assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol:.1e} * {scale:.3g}"


# --------------------------------------------------------------------------
# forward pins
# --------------------------------------------------------------------------

def pin_golden_forward(oracle):
    g = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))["forward"]
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for causal, key in ((False, "noncausal"), (True, "causal")):
        O, lse = oracle.attn_fwd(q, k, v, g["scale"], causal)
        _close(O[0, 0], g[key]["O"], 1e-14, f"golden O {key}")
        _close(lse[0, 0], g[key]["lse"], 1e-14, f"golden lse {key}")


def pin_single_key(oracle):
    q, k, v = _qkv(1, 2, 3, 5, 1, 4)
    scale = 0.37
    O, lse = oracle.attn_fwd(q, k, v, scale, False)
    # One key: its probability is exactly 1, so O is exactly that V row.
    assert np.array_equal(O, np.broadcast_to(v, O.shape)), "single key must return its V row"
    want = scale * np.einsum("bhid,bhd->bhi", q, k[:, :, 0, :])
    _close(lse, want, 1e-14, "single-key lse")


def pin_causal_row0(oracle):
    q, k, v = _qkv(2, 2, 2, 9, 9, 5)
    scale = 0.8
    O, lse = oracle.attn_fwd(q, k, v, scale, True)
    assert np.array_equal(O[:, :, 0, :], v[:, :, 0, :]), "causal row 0 must equal V[0]"
    want = scale * np.sum(q[:, :, 0, :] * k[:, :, 0, :], axis=-1)
    _close(lse[:, :, 0], want, 1e-14, "causal row-0 lse")


def pin_identity_values(oracle):
    # V = identity exposes the probability matrix itself: O = P.
    L, d = 7, 3
    q, k, _ = _qkv(3, 1, 2, L, L, d)
    v = np.broadcast_to(np.eye(L), (1, 2, L, L)).copy()
    for causal in (False, True):
        P, _ = oracle.attn_fwd(q, k, v, 0.9, causal)
        _close(P.sum(axis=-1), np.ones(P.shape[:-1]), 1e-14, "softmax rows sum to 1")
        assert np.all(P >= 0), "probabilities must be non-negative"
        iu = np.triu_indices(L, 1)
        upper = P[:, :, iu[0], iu[1]]
        if causal:
            assert np.all(upper == 0), "causal: keys after the query get probability 0"
        else:
            assert np.all(upper > 0), "non-causal: every key gets a positive weight"


def pin_constant_values(oracle):
    q, k, _ = _qkv(4, 2, 2, 6, 8, 4)
    c = np.array([1.5, -2.0, 0.25, 3.0])
    v = np.broadcast_to(c, (2, 2, 8, 4)).copy()
    for causal in (False, True):
        O, _ = oracle.attn_fwd(q, k, v, 1.1, causal)
        _close(O, np.broadcast_to(c, O.shape), 1e-14, "constant V rows are returned")


def pin_zero_scale(oracle):
    q, k, v = _qkv(5, 1, 3, 6, 6, 4)
    O, lse = oracle.attn_fwd(q, k, v, 0.0, False)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), 1e-14, "scale 0: mean of V")
    _close(lse, np.full(lse.shape, math.log(6)), 1e-14, "scale 0: lse = ln n")
    O, lse = oracle.attn_fwd(q, k, v, 0.0, True)
    n = np.arange(1, 7)
    prefix = np.cumsum(v, axis=2) / n[None, None, :, None]
    _close(O, prefix, 1e-14, "scale 0 causal: prefix mean of V")
    _close(lse, np.broadcast_to(np.log(n), lse.shape), 1e-14, "scale 0 causal: lse = ln(i+1)")


def pin_hardmax(oracle):
    # Key 2 wins every row by a score margin >= 800: exp(-800) underflows to
    # exactly 0 in float64, so O is exactly V[2] and lse is that score.
    d = 2
    q = np.array([[[[1.0, 0.0], [1.0, 0.0], [1.0, 0.0]]]])
    k = np.array([[[[0.0, 0.0], [-1.0, 0.0], [900.0, 0.0], [5.0, 0.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]]]])
    O, lse = oracle.attn_fwd(q, k, v, 1.0, False)
    assert np.array_equal(O[0, 0], np.broadcast_to(v[0, 0, 2], (3, d))), "hardmax row"
    assert np.array_equal(lse[0, 0], np.full(3, 900.0)), "hardmax lse"


def pin_bounds(oracle):
    q, k, v = _qkv(6, 2, 2, 11, 11, 6)
    scale = 0.6
    for causal in (False, True):
        O, lse = oracle.attn_fwd(q, k, v, scale, causal)
        S = scale * np.einsum("bhid,bhjd->bhij", q, k)
        i = np.arange(11)[:, None]
        j = np.arange(11)[None, :]
        vis = (j <= i) if causal else np.ones((11, 11), bool)
        Smax = np.where(vis, S, -np.inf).max(axis=-1)
        n = vis.sum(axis=1)
        assert np.all(lse >= Smax - 1e-12), "lse >= row max"
        assert np.all(lse <= Smax + np.log(n) + 1e-12), "lse <= row max + ln n"
        for r in range(11):
            vv = v[:, :, vis[r], :]
            assert np.all(O[:, :, r, :] >= vv.min(axis=2) - 1e-12), "O inside the hull of V"
            assert np.all(O[:, :, r, :] <= vv.max(axis=2) + 1e-12), "O inside the hull of V"


def pin_permutation(oracle):
    q, k, v = _qkv(7, 1, 2, 5, 9, 3)
    O, lse = oracle.attn_fwd(q, k, v, 0.7, False)
    p = _rng(70).permutation(9)
    O2, lse2 = oracle.attn_fwd(q, k[:, :, p], v[:, :, p], 0.7, False)
    _close(O2, O, 1e-13, "joint key/value permutation leaves O unchanged")
    _close(lse2, lse, 1e-13, "joint key/value permutation leaves lse unchanged")
    pq = _rng(71).permutation(5)
    O3, lse3 = oracle.attn_fwd(q[:, :, pq], k, v, 0.7, False)
    _close(O3, O[:, :, pq], 1e-13, "query permutation permutes O")
    _close(lse3, lse[:, :, pq], 1e-13, "query permutation permutes lse")


def pin_shift(oracle):
    q, k, v = _qkv(8, 1, 2, 6, 6, 4)
    scale = 0.5
    c = np.array([0.3, -1.2, 2.0, 0.7])
    for causal in (False, True):
        O, lse = oracle.attn_fwd(q, k, v, scale, causal)
        Ok, lsek = oracle.attn_fwd(q, k + c, v, scale, causal)
        _close(Ok, O, 1e-13, "adding one vector to every key leaves O unchanged")
        _close(lsek, lse + scale * (q @ c), 1e-13, "key shift moves lse by scale*q.c")
        Ov, _ = oracle.attn_fwd(q, k, v + c, scale, causal)
        _close(Ov, O + c, 1e-13, "adding c to every value row adds c to O")


def pin_blockwise_merge(oracle):
    # Splitting the keys into two blocks: exp(lse) adds up and O is the
    # exp(lse)-weighted mean of the block outputs (the running-statistics
    # merge of the blockwise method).
    q, k, v = _qkv(9, 1, 2, 4, 10, 3)
    O, lse = oracle.attn_fwd(q, k, v, 0.8, False)
    Oa, la = oracle.attn_fwd(q, k[:, :, :4], v[:, :, :4], 0.8, False)
    Ob, lb = oracle.attn_fwd(q, k[:, :, 4:], v[:, :, 4:], 0.8, False)
    _close(np.logaddexp(la, lb), lse, 1e-13, "lse merges by logaddexp")
    wa = np.exp(la - lse)[..., None]
    wb = np.exp(lb - lse)[..., None]
    _close(wa * Oa + wb * Ob, O, 1e-13, "O merges by exp(lse) weights")


def _torch_sdpa(q, k, v, scale, causal):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    O = torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], is_causal=causal, scale=scale)
    return t, O


def pin_torch_sdpa(oracle):
    cases = [(1, 2, 16, 16, 8, False), (2, 1, 13, 13, 4, True), (1, 2, 5, 12, 6, False),
             (1, 1, 12, 5, 3, True), (1, 1, 7, 19, 5, True)]
    for n, (B, H, Lq, Lk, d, causal) in enumerate(cases):
        q, k, v = _qkv(100 + n, B, H, Lq, Lk, d)
        scale = 1.0 / math.sqrt(d)
        with torch.no_grad():
            _, Ot = _torch_sdpa(q, k, v, scale, causal)
        O, _ = oracle.attn_fwd(q, k, v, scale, causal)
        _close(O, Ot.numpy(), 1e-12, f"torch fp64 sdpa case {n}")


def pin_rows_consistency(oracle):
    q, k, v = _qkv(10, 1, 2, 20, 20, 4)
    rows = np.array([[[0, 19, 7, 3], [5, 0, 19, 11]]])
    for causal in (False, True):
        O, lse = oracle.attn_fwd(q, k, v, 0.4, causal)
        Or, lr = oracle.attn_fwd_rows(q, k, v, 0.4, causal, rows)
        for h in range(2):
            _close(Or[0, h], O[0, h, rows[0, h]], 1e-14, "sampled rows equal full rows")
            _close(lr[0, h], lse[0, h, rows[0, h]], 1e-14, "sampled lse equal full lse")


# --------------------------------------------------------------------------
# backward pins
# --------------------------------------------------------------------------

def pin_golden_backward(oracle):
    g = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))["backward"]
    arr = lambda x: np.array(x)[None, None]
    dq, dk, dv = oracle.attn_bwd(arr(g["q"]), arr(g["k"]), arr(g["v"]), arr(g["dO"]),
                                 g["scale"], False)
    _close(dq[0, 0], g["dq"], 1e-14, "golden dq")
    _close(dk[0, 0], g["dk"], 1e-14, "golden dk")
    _close(dv[0, 0], g["dv"], 1e-14, "golden dv")


def pin_finite_differences(oracle):
    # Central differences of the loss <dO, O> in float64, step 1e-6.
    for causal, (Lq, Lk) in ((False, (4, 6)), (True, (5, 5))):
        q, k, v = _qkv(11 + causal, 1, 1, Lq, Lk, 3)
        dO = _rng(20 + causal).standard_normal((1, 1, Lq, 3))
        scale = 0.9
        dq, dk, dv = oracle.attn_bwd(q, k, v, dO, scale, causal)
        loss = lambda a, b, c: float(np.sum(dO * oracle.attn_fwd(a, b, c, scale, causal)[0]))
        h = 1e-6
        for name, x, grad in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = [q, k, v]; args_m = [q, k, v]
                pos = {"dq": 0, "dk": 1, "dv": 2}[name]
                args_p[pos] = xp; args_m[pos] = xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(grad, num, 2e-7, f"finite differences {name} causal={causal}")


def pin_torch_autograd(oracle):
    cases = [(1, 2, 9, 9, 4, True), (2, 1, 6, 11, 5, False), (1, 1, 17, 17, 8, True)]
    for n, (B, H, Lq, Lk, d, causal) in enumerate(cases):
        q, k, v = _qkv(200 + n, B, H, Lq, Lk, d)
        dO = _rng(300 + n).standard_normal((B, H, Lq, d))
        scale = 1.0 / math.sqrt(d)
        t, Ot = _torch_sdpa(q, k, v, scale, causal)
        Ot.backward(torch.tensor(dO))
        dq, dk, dv = oracle.attn_bwd(q, k, v, dO, scale, causal)
        _close(dq, t[0].grad.numpy(), 1e-12, f"torch autograd dq case {n}")
        _close(dk, t[1].grad.numpy(), 1e-12, f"torch autograd dk case {n}")
        _close(dv, t[2].grad.numpy(), 1e-12, f"torch autograd dv case {n}")


def pin_gradient_invariants(oracle):
    q, k, v = _qkv(12, 2, 2, 10, 10, 4)
    dO = _rng(13).standard_normal((2, 2, 10, 4))
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd(q, k, v, dO, 0.7, causal)
        # Shifting every key by one vector changes no output: sum_j dK_j = 0.
        _close(dk.sum(axis=2), np.zeros((2, 2, 4)), 1e-13, "sum of dK over keys is 0")
        # Rows of P sum to one: sum_j dV_j = sum_i dO_i.
        _close(dv.sum(axis=2), dO.sum(axis=2), 1e-13, "sum of dV equals sum of dO")


def pin_constant_values_backward(oracle):
    q, k, _ = _qkv(14, 1, 2, 7, 7, 3)
    v = np.broadcast_to(np.array([2.0, -1.0, 0.5]), (1, 2, 7, 3)).copy()
    dO = _rng(15).standard_normal((1, 2, 7, 3))
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd(q, k, v, dO, 0.9, causal)
        # O no longer depends on Q or K.
        _close(dq, np.zeros_like(dq), 1e-13, "constant V: dQ = 0")
        _close(dk, np.zeros_like(dk), 1e-13, "constant V: dK = 0")


def pin_bwd_heads_consistency(oracle):
    q, k, v = _qkv(16, 2, 3, 8, 8, 4)
    dO = _rng(17).standard_normal((2, 3, 8, 4))
    full = oracle.attn_bwd(q, k, v, dO, 0.5, True)
    heads = [(1, 2), (0, 0), (1, 0)]
    part = oracle.attn_bwd_heads(q, k, v, dO, 0.5, True, heads)
    for n, (b, h) in enumerate(heads):
        for a, f in zip(part, full):
            _close(a[n], f[b, h], 1e-14, "per-head backward equals full backward")


# --------------------------------------------------------------------------
# key-range pins (attention over one range of keys, and the merge of ranges)
# --------------------------------------------------------------------------

def _ranges(rng, Lk, n):
    cuts = np.sort(rng.integers(0, Lk + 1, size=n - 1))
    b = [0] + list(cuts) + [Lk]
    return list(zip(b[:-1], b[1:]))


def pin_keyrange_whole(oracle):
    # The range [0, Lk) is the whole key set.
    q, k, v = _qkv(40, 1, 2, 9, 9, 3)
    for causal in (False, True):
        O, lse = oracle.attn_fwd(q, k, v, 0.7, causal)
        Or, lr = oracle.attn_fwd_keyrange(q, k, v, 0.7, causal, 0, 9)
        _close(Or, O, 1e-14, "range [0, Lk) equals the whole")
        _close(lr, lse, 1e-14, "range [0, Lk) lse equals the whole")


def pin_keyrange_single_key(oracle):
    # One key in range: every row that sees it returns its value row and
    # lse = its score; causal rows before it see nothing (O = 0, lse = -inf).
    q, k, v = _qkv(41, 1, 1, 6, 6, 4)
    j = 3
    O, lse = oracle.attn_fwd_keyrange(q, k, v, 0.9, False, j, j + 1)
    _close(O[0, 0], np.repeat(v[0, 0, j][None], 6, axis=0), 1e-15, "single key returns V_j")
    _close(lse[0, 0], 0.9 * (q[0, 0] @ k[0, 0, j]), 1e-14, "single key lse is its score")
    Oc, lc = oracle.attn_fwd_keyrange(q, k, v, 0.9, True, j, j + 1)
    assert np.all(Oc[0, 0, :j] == 0) and np.all(np.isneginf(lc[0, 0, :j])), "rows before key j"
    _close(Oc[0, 0, j:], np.repeat(v[0, 0, j][None], 6 - j, axis=0), 1e-15, "rows from key j on")


def pin_keyrange_causal_rows(oracle):
    # Causal range [k0, k1) for row i is the non-causal attention over the
    # keys k0 .. min(k1, i + 1) - 1 (absolute indices), computed here from
    # the definition one row at a time with plain Python loops.
    q, k, v = _qkv(42, 1, 1, 7, 9, 2)
    k0, k1, s = 2, 6, 1.1
    O, lse = oracle.attn_fwd_keyrange(q, k, v, s, True, k0, k1)
    for i in range(7):
        keys = range(k0, min(k1, i + 1))
        if not keys:
            assert np.isneginf(lse[0, 0, i]) and np.all(O[0, 0, i] == 0), f"row {i} sees nothing"
            continue
        sc = [s * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(2)) for j in keys]
        mx = max(sc)
        z = sum(math.exp(x - mx) for x in sc)
        _close(lse[0, 0, i], mx + math.log(z), 1e-14, f"row {i} lse by loops")
        o = [sum(math.exp(x - mx) / z * v[0, 0, j, c] for x, j in zip(sc, keys)) for c in range(2)]
        _close(O[0, 0, i], o, 1e-14, f"row {i} output by loops")


def pin_merge_partition(oracle):
    # Any partition of the keys into ranges (some empty, some fully masked
    # for early causal rows) merges back to the whole: the running-statistics
    # recurrence over finished ranges.
    rng = _rng(43)
    for trial in range(6):
        Lq, Lk = int(rng.integers(1, 12)), int(rng.integers(1, 20))
        causal = bool(trial % 2)
        q, k, v = _qkv(44 + trial, 1, 2, Lq, Lk, 3)
        s = float(rng.uniform(0.2, 1.5))
        O, lse = oracle.attn_fwd(q, k, v, s, causal)
        parts = [oracle.attn_fwd_keyrange(q, k, v, s, causal, a, b)
                 for a, b in _ranges(rng, Lk, int(rng.integers(1, 6)))]
        Om, lm = oracle.merge_partials(np.stack([p[0] for p in parts]),
                                       np.stack([p[1] for p in parts]))
        _close(Om, O, 1e-13, f"merged ranges equal the whole (trial {trial})")
        _close(lm, lse, 1e-13, f"merged lse equals the whole (trial {trial})")


def pin_merge_library(oracle):
    # The merged lse is the log-sum-exp over ranges (torch.logsumexp as the
    # library routine); merging one result with itself adds log 2 to lse and
    # leaves O unchanged.
    r = _rng(45)
    Op = r.standard_normal((3, 1, 2, 5, 4))
    lp = r.standard_normal((3, 1, 2, 5)) * 3
    lp[1, 0, 0, 2] = -np.inf
    O, lse = oracle.merge_partials(Op, lp)
    _close(lse, torch.logsumexp(torch.tensor(lp), dim=0).numpy(), 1e-14, "lse is logsumexp")
    O2, l2 = oracle.merge_partials(np.stack([Op[0], Op[0]]), np.stack([lp[0], lp[0]]))
    _close(O2, Op[0], 1e-15, "self-merge keeps O")
    _close(l2, lp[0] + math.log(2.0), 1e-14, "self-merge adds log 2")


# --------------------------------------------------------------------------
# block-sparse pins
# --------------------------------------------------------------------------

def pin_blocksparse_all_kept(oracle):
    # Keeping every block is the dense attention.
    q, k, v = _qkv(50, 1, 2, 11, 13, 3)
    bm = np.ones((3, 4), dtype=np.uint8)
    for causal in (False, True):
        O, lse = oracle.attn_fwd(q, k, v, 0.6, causal)
        Ob, lb = oracle.attn_fwd_blocksparse(q, k, v, 0.6, causal, bm, block=4)
        _close(Ob, O, 1e-14, "all blocks kept equals dense")
        _close(lb, lse, 1e-14, "all blocks kept: lse equals dense")


def pin_blocksparse_block_diagonal(oracle):
    # Keeping only the diagonal blocks is independent attention inside each
    # block: the dense oracle on each block's own rows and keys.
    q, k, v = _qkv(51, 1, 1, 10, 10, 3)
    bm = np.eye(3, dtype=np.uint8)
    O, lse = oracle.attn_fwd_blocksparse(q, k, v, 0.9, False, bm, block=4)
    for a in range(0, 10, 4):
        b = min(a + 4, 10)
        Oa, la = oracle.attn_fwd(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], 0.9, False)
        _close(O[:, :, a:b], Oa, 1e-14, f"diagonal block at {a}")
        _close(lse[:, :, a:b], la, 1e-14, f"diagonal block lse at {a}")


def pin_blocksparse_key_column(oracle):
    # Keeping one key block for every row is attention over that key range.
    q, k, v = _qkv(52, 1, 2, 9, 14, 2)
    for causal in (False, True):
        bm = np.zeros((3, 4), dtype=np.uint8)
        bm[:, 1] = 1
        O, lse = oracle.attn_fwd_blocksparse(q, k, v, 1.2, causal, bm, block=4)
        Or, lr = oracle.attn_fwd_keyrange(q, k, v, 1.2, causal, 4, 8)
        assert np.array_equal(np.isneginf(lse), np.isneginf(lr)), "rows that see nothing"
        _close(O, Or, 1e-14, "one key block equals its key range")
        f = np.isfinite(lr)
        _close(lse[f], lr[f], 1e-14, "one key block: lse")


def pin_blocksparse_loops(oracle):
    # Per-element pure-Python loops on a tiny case (block 2, per-slice masks,
    # causal), including a row that sees nothing.
    q, k, v = _qkv(53, 1, 2, 5, 6, 2)
    bm = np.array([[[1, 0, 1], [0, 1, 0], [1, 1, 0]],
                   [[0, 1, 1], [1, 0, 1], [0, 0, 1]]], dtype=np.uint8)[None]
    s = 0.7
    O, lse = oracle.attn_fwd_blocksparse(q, k, v, s, True, bm, block=2)
    for h in range(2):
        for i in range(5):
            keys = [j for j in range(6) if bm[0, h, i // 2, j // 2] and j <= i]
            if not keys:
                assert np.isneginf(lse[0, h, i]) and np.all(O[0, h, i] == 0), f"h{h} row {i} empty"
                continue
            sc = [s * sum(q[0, h, i, c] * k[0, h, j, c] for c in range(2)) for j in keys]
            mx = max(sc)
            z = sum(math.exp(x - mx) for x in sc)
            _close(lse[0, h, i], mx + math.log(z), 1e-14, f"h{h} row {i} lse by loops")
            o = [sum(math.exp(x - mx) / z * v[0, h, j, c] for x, j in zip(sc, keys)) for c in range(2)]
            _close(O[0, h, i], o, 1e-14, f"h{h} row {i} output by loops")
    assert np.isneginf(lse[0, 1, 0]), "row 0 of head 1 sees no key (block 0,0 dropped)"


def pin_blocksparse_bwd_all_kept(oracle):
    # Keeping every block gives the dense gradients.
    q, k, v = _qkv(54, 1, 2, 9, 11, 3)
    dO = _rng(55).standard_normal((1, 2, 9, 3))
    bm = np.ones((3, 3), dtype=np.uint8)
    for causal in (False, True):
        ref = oracle.attn_bwd(q, k, v, dO, 0.7, causal)
        got = oracle.attn_bwd_blocksparse(q, k, v, dO, 0.7, causal, bm, block=4)
        for a, r, n in zip(got, ref, "qkv"):
            _close(a, r, 1e-13, f"all kept: d{n} equals dense")


def pin_blocksparse_bwd_block_diagonal(oracle):
    # Block-diagonal mask: each block's gradients are the dense backward of
    # that block alone; no gradient crosses blocks.
    q, k, v = _qkv(56, 1, 1, 10, 10, 2)
    dO = _rng(57).standard_normal((1, 1, 10, 2))
    got = oracle.attn_bwd_blocksparse(q, k, v, dO, 0.9, True, np.eye(3, dtype=np.uint8), block=4)
    for a in range(0, 10, 4):
        b = min(a + 4, 10)
        ref = oracle.attn_bwd(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], dO[:, :, a:b], 0.9, True)
        for x, r, n in zip(got, ref, "qkv"):
            _close(x[:, :, a:b], r, 1e-13, f"diagonal block {a}: d{n}")


def pin_blocksparse_bwd_finite_differences(oracle):
    # Central differences of <dO, O> on a tiny case (block 2, causal, a row
    # that sees nothing): the analytic gradients match to 1e-7.
    r = _rng(58)
    q, k, v = (r.standard_normal((1, 1, n, 2)) for n in (5, 6, 6))
    dO = r.standard_normal((1, 1, 5, 2))
    bm = np.array([[0, 1, 1], [1, 0, 1], [1, 1, 0]], dtype=np.uint8)
    s, eps = 0.8, 1e-6

    def loss(q_, k_, v_):
        O, _ = oracle.attn_fwd_blocksparse(q_, k_, v_, s, True, bm, block=2)
        return float((O * dO).sum())

    dq, dk, dv = oracle.attn_bwd_blocksparse(q, k, v, dO, s, True, bm, block=2)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        _close(g, num, 1e-7, f"finite differences d{name}")
    assert np.all(dq[0, 0, 0] == 0), "row 0 sees no key: its dQ is 0"


BLOCKSPARSE_PINS = [pin_blocksparse_all_kept, pin_blocksparse_block_diagonal,
                    pin_blocksparse_key_column, pin_blocksparse_loops,
                    pin_blocksparse_bwd_all_kept, pin_blocksparse_bwd_block_diagonal,
                    pin_blocksparse_bwd_finite_differences]

SPLITKV_PINS = [pin_keyrange_whole, pin_keyrange_single_key, pin_keyrange_causal_rows,
                pin_merge_partition, pin_merge_library]

FORWARD_PINS = [pin_golden_forward, pin_single_key, pin_causal_row0, pin_identity_values,
                pin_constant_values, pin_zero_scale, pin_hardmax, pin_bounds,
                pin_permutation, pin_shift, pin_blockwise_merge, pin_torch_sdpa,
                pin_rows_consistency]
BACKWARD_PINS = [pin_golden_backward, pin_finite_differences, pin_torch_autograd,
                 pin_gradient_invariants, pin_constant_values_backward,
                 pin_bwd_heads_consistency]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + SPLITKV_PINS + BLOCKSPARSE_PINS
