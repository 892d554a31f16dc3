"""Block-sparse forward (fa_fwd_blocksparse) against the fp64 oracle, on the
GPU through the C ABI.

What is checked:
* random seeded 128x128 block masks (shared by all slices and per slice),
  both masks, both head dimensions, ragged lengths, against
  oracle.attn_fwd_blocksparse at the bf16 forward tolerances, with rows
  that see no key returning exactly O = 0 and lse = -inf;
* a mask that keeps every block gives bitwise the dense forward's result
  (the extra work is masked tiles whose probabilities are exactly 0);
* a sliding-window + first-block pattern at the benchmark size
  (B1 H32 L4096 d128, causal), on sampled rows of every head;
* invalid calls.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_13_amd as fa
from tests.gpu_util import announce, assert_bf16_fwd, device, fwd_errors, to_dev
from workloads import BENCH_WORKLOAD, WORKLOADS, make_inputs, sample_rows, to_f64

pytestmark = pytest.mark.gpu
BLK = 128


def random_mask(shape, density, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(shape, generator=g) < density).to(torch.uint8)


def _check(O, lse, O_ref, lse_ref, what):
    O, lse = (x if isinstance(x, np.ndarray) else to_f64(x) for x in (O, lse))
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows without keys differ"
    assert np.all(O[empty] == 0.0), f"{what}: rows without keys must be 0"
    if (~empty).any():
        assert_bf16_fwd(fwd_errors(O[~empty], lse[~empty], O_ref[~empty], lse_ref[~empty]), what)


CASES = [
    # B, H, Lq, Lk, d, causal, per_slice, density
    (1, 2, 256, 256, 128, False, False, 0.5),
    (1, 2, 256, 256, 128, True, True, 0.6),
    (1, 2, 300, 500, 128, False, True, 0.5),
    (2, 2, 1000, 777, 64, True, False, 0.5),
    (1, 3, 513, 1100, 64, False, True, 0.3),
    (1, 1, 129, 4097, 128, False, False, 0.25),
    (2, 1, 1, 640, 128, False, True, 0.5),
    (1, 2, 768, 768, 128, True, True, 0.4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Lq{}Lk{}d{}-c{}-s{}-p{}".format(*c))
def test_blocksparse_matches_oracle(case):
    B, H, Lq, Lk, d, causal, per_slice, density = case
    q, k, v = make_inputs(B, H, Lq, Lk, d, "bf16", seed=Lq + 7 * Lk)
    nqb, nkb = -(-Lq // BLK), -(-Lk // BLK)
    bm = random_mask((B, H, nqb, nkb) if per_slice else (nqb, nkb), density, seed=Lq * Lk)
    scale = 1.0 / math.sqrt(d)
    O_ref, lse_ref = oracle.attn_fwd_blocksparse(to_f64(q), to_f64(k), to_f64(v), scale, causal,
                                                 bm.numpy(), block=BLK)
    qd, kd, vd, bmd = to_dev(q, k, v, bm)
    announce(f"blocksparse {case}")
    for out_dtype in (torch.bfloat16, torch.float32):
        O, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, scale=scale, causal=causal,
                                       out_dtype=out_dtype)
        torch.cuda.synchronize()
        _check(O, lse, O_ref, lse_ref, f"{case} out {out_dtype}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_all_blocks_kept_equals_dense_bitwise(d, causal):
    B, H, L = 1, 2, 700
    q, k, v = to_dev(*make_inputs(B, H, L, L, d, "bf16", seed=21))
    bm = torch.ones((-(-L // BLK), -(-L // BLK)), dtype=torch.uint8, device=device())
    announce(f"blocksparse all kept d{d} causal {causal}")
    Od, ld = fa.fa_fwd(q, k, v, causal=causal)
    Os, ls = fa.fa_fwd_blocksparse(q, k, v, bm, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(Od, Os) and torch.equal(ld, ls)


def test_all_blocks_dropped_gives_zero_rows():
    q, k, v = to_dev(*make_inputs(1, 2, 300, 300, 128, "bf16", seed=22))
    bm = torch.zeros((3, 3), dtype=torch.uint8, device=device())
    announce("blocksparse nothing kept")
    O, lse = fa.fa_fwd_blocksparse(q, k, v, bm)
    torch.cuda.synchronize()
    assert torch.all(O == 0) and torch.all(torch.isneginf(lse))


def test_window_pattern_benchmark_size_sampled_rows():
    # Sliding window of four blocks plus the first block, causal, at the
    # benchmark size; 16 sampled rows of every head, each against the
    # oracle's dense attention over exactly the keys its blocks keep.
    w = WORKLOADS[BENCH_WORKLOAD]
    q, k, v = make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed, amp=w.amp)
    nb = w.Lq // BLK
    i = np.arange(nb)
    bm = torch.from_numpy(((i[:, None] - i[None, :] < 4) | (i[None, :] == 0)).astype(np.uint8))
    rows = sample_rows(w.H, w.Lq, 16, seed=23, B=w.B)
    qd, kd, vd, bmd = to_dev(q, k, v, bm)
    announce("blocksparse window pattern B1 H32 L4096 d128 causal")
    O, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    O, lse = to_f64(O), to_f64(lse)
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    vis = oracle.block_visible(bm.numpy(), w.Lq, w.Lk, BLK, True)
    for h in range(w.H):
        for row in rows[0, h].tolist():
            keys = np.nonzero(vis[row])[0]
            O1, l1 = oracle.attn_fwd(q64[:, h:h + 1, row:row + 1], k64[:, h:h + 1, keys],
                                     v64[:, h:h + 1, keys], w.scale, False)
            _check(O[:, h:h + 1, row:row + 1], lse[:, h:h + 1, row:row + 1], O1, l1,
                   f"head {h} row {row}")


def test_invalid_calls_are_rejected():
    q, k, v = to_dev(*make_inputs(1, 1, 200, 200, 128, "bf16", seed=0))
    bm = torch.ones((2, 2), dtype=torch.uint8, device=device())
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_blocksparse(q.float(), k.float(), v.float(), bm)
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    with pytest.raises(ValueError):
        fa.fa_fwd_blocksparse(q, k, v, torch.ones((3, 2), dtype=torch.uint8, device=device()))


# ---- block-sparse backward --------------------------------------------------

from tests.gpu_util import BF16_GRAD_REL, rel_to_max  # noqa: E402

BWD_CASES = [
    # B, H, L, d, causal, per_slice, density
    (1, 2, 256, 128, False, False, 0.5),
    (1, 2, 384, 128, True, True, 0.6),
    (2, 2, 500, 64, True, False, 0.5),
    (1, 3, 640, 64, False, True, 0.4),
    (1, 2, 1000, 128, True, True, 0.3),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}H{}L{}d{}-c{}-s{}-p{}".format(*c))
def test_blocksparse_backward_matches_oracle(case):
    B, H, L, d, causal, per_slice, density = case
    q, k, v, do = make_inputs(B, H, L, L, d, "bf16", seed=L + d, with_dO=True)
    nb = -(-L // BLK)
    bm = random_mask((B, H, nb, nb) if per_slice else (nb, nb), density, seed=3 * L + 1)
    if per_slice:
        bm[0, 0, 0, :] = 0  # first row block of slice (0, 0) sees no key
    else:
        bm[0, :] = 0
    scale = 1.0 / math.sqrt(d)
    ref = oracle.attn_bwd_blocksparse(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal,
                                      bm.numpy(), block=BLK)
    qd, kd, vd, dod, bmd = to_dev(q, k, v, do, bm)
    announce(f"blocksparse bwd {case}")
    O, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, scale=scale, causal=causal)
    grads = fa.fa_bwd_blocksparse(qd, kd, vd, O, dod, lse, bmd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for g, r, name in zip(grads, ref, ("dQ", "dK", "dV")):
        err = rel_to_max(to_f64(g), r)
        assert err <= BF16_GRAD_REL, f"{case} {name}: rel-to-max {err:.3e}"
    # Rows that see no key get exactly zero dQ.
    assert torch.all(grads[0][0, 0, :BLK] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_all_blocks_kept_equals_dense_bitwise(d, causal):
    B, H, L = 1, 2, 768
    q, k, v, do = to_dev(*make_inputs(B, H, L, L, d, "bf16", seed=31, with_dO=True))
    bm = torch.ones((L // BLK, L // BLK), dtype=torch.uint8, device=device())
    announce(f"blocksparse bwd all kept d{d} causal {causal}")
    O, lse = fa.fa_fwd(q, k, v, causal=causal)
    dense = fa.fa_bwd(q, k, v, O, do, lse, causal=causal)
    sparse = fa.fa_bwd_blocksparse(q, k, v, O, do, lse, bm, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(dense, sparse):
        assert torch.equal(a, b)


def test_backward_window_pattern_benchmark_size_two_heads():
    # The launch the benchmark times: B1 H32 L4096 d128 causal, window of 4
    # blocks + the first block; two full heads against the oracle.
    from workloads import window_block_mask
    w = WORKLOADS[BENCH_WORKLOAD]
    q, k, v, do = make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed, amp=w.amp,
                              with_dO=True)
    bm = window_block_mask(w.Lq // BLK)
    qd, kd, vd, dod, bmd = to_dev(q, k, v, do, bm)
    announce("blocksparse bwd window pattern B1 H32 L4096 d128 causal")
    O, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, scale=w.scale, causal=True)
    grads = fa.fa_bwd_blocksparse(qd, kd, vd, O, dod, lse, bmd, scale=w.scale, causal=True)
    # A second call gives the same bits (every gradient row is summed in a
    # fixed order by one workgroup).
    again = fa.fa_bwd_blocksparse(qd, kd, vd, O, dod, lse, bmd, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert torch.equal(a, b)
    for h in (0, 17):
        sl = lambda t: to_f64(t[:, h:h + 1])
        ref = oracle.attn_bwd_blocksparse(sl(q), sl(k), sl(v), sl(do), w.scale, True, bm.numpy(),
                                          block=BLK)
        for g, r, name in zip(grads, ref, ("dQ", "dK", "dV")):
            err = rel_to_max(to_f64(g[:, h:h + 1]), r)
            assert err <= BF16_GRAD_REL, f"head {h} {name}: rel-to-max {err:.3e}"


# ---- lists longer than one register window (128 entries) ---------------------

@pytest.mark.parametrize("d", [64, 128])
def test_long_key_block_list_forward_and_backward(d):
    # 40000 keys = 313 key blocks at density 0.7: the key-block lists of the
    # forward and of the dQ kernel run past two windows of 128 entries.
    B, H, Lq, Lk = 1, 1, 256, 40000
    q, k, v, do = make_inputs(B, H, Lq, Lk, d, "bf16", seed=51, with_dO=True)
    bm = random_mask((-(-Lq // BLK), -(-Lk // BLK)), 0.7, seed=52)
    assert int(bm[0].sum()) > 128 and int(bm[1].sum()) > 128
    scale = 1.0 / math.sqrt(d)
    O_ref, lse_ref = oracle.attn_fwd_blocksparse(to_f64(q), to_f64(k), to_f64(v), scale, False,
                                                 bm.numpy(), block=BLK)
    ref = oracle.attn_bwd_blocksparse(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, False,
                                      bm.numpy(), block=BLK)
    qd, kd, vd, dod, bmd = to_dev(q, k, v, do, bm)
    announce(f"blocksparse long key list d{d}")
    O, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, scale=scale)
    grads = fa.fa_bwd_blocksparse(qd, kd, vd, O, dod, lse, bmd, scale=scale)
    torch.cuda.synchronize()
    _check(O, lse, O_ref, lse_ref, f"long key list d{d}")
    for g, r, name in zip(grads, ref, ("dQ", "dK", "dV")):
        err = rel_to_max(to_f64(g), r)
        assert err <= BF16_GRAD_REL, f"long key list d{d} {name}: rel-to-max {err:.3e}"


def test_long_query_block_list_backward():
    # 40000 queries = 313 query blocks at density 0.7: the dK/dV kernel's
    # query-block list runs past two windows of 128 entries.
    B, H, Lq, Lk, d = 1, 1, 40000, 256, 128
    q, k, v, do = make_inputs(B, H, Lq, Lk, d, "bf16", seed=53, with_dO=True)
    bm = random_mask((-(-Lq // BLK), -(-Lk // BLK)), 0.7, seed=54)
    bm[:, 0] = 1  # every row block sees at least one key block
    assert int(bm[:, 0].sum()) > 128 and int(bm[:, 1].sum()) > 128
    scale = 1.0 / math.sqrt(d)
    ref = oracle.attn_bwd_blocksparse(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, False,
                                      bm.numpy(), block=BLK)
    qd, kd, vd, dod, bmd = to_dev(q, k, v, do, bm)
    announce("blocksparse long query list")
    O, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, scale=scale)
    grads = fa.fa_bwd_blocksparse(qd, kd, vd, O, dod, lse, bmd, scale=scale)
    again = fa.fa_bwd_blocksparse(qd, kd, vd, O, dod, lse, bmd, scale=scale)
    torch.cuda.synchronize()
    # Lists of over 200 entries: the same bits again on a second call.
    for a, b in zip(grads, again):
        assert torch.equal(a, b)
    for g, r, name in zip(grads, ref, ("dQ", "dK", "dV")):
        err = rel_to_max(to_f64(g), r)
        assert err <= BF16_GRAD_REL, f"long query list {name}: rel-to-max {err:.3e}"
