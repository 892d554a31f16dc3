"""The largest sizes the C ABI accepts, on the GPU.

Per (batch, head) slice the byte offsets are 32-bit; the ABI accepts key and
query lengths up to (L + 256) * d * 4 < 2^31.  At d = 128 that is 4,194,048
keys (1 GiB per K or V slice).  These tests run the forward and the
key-split forward at exactly that key length with a few query rows, and
check sampled rows against the oracle (each sampled row is the full fp64
row over all keys).  One key more is rejected with FA_ERR_SHAPE.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_13_amd as fa
from tests.gpu_util import announce, assert_bf16_fwd, device, fwd_errors
from workloads import make_inputs, to_f64

pytestmark = pytest.mark.gpu

D = 128
LK_MAX = (1 << 31) // (D * 4) - 256 - 1   # largest Lk with (Lk + 256) * d * 4 < 2^31


def _inputs(Lq, Lk, seed):
    # Drawn on the CPU like every other workload (seeded N(0,1), bf16).
    return make_inputs(1, 1, Lq, Lk, D, "bf16", seed=seed)


def _check_rows(O, lse, q, k, v, rows, causal):
    rr = np.asarray(rows, dtype=np.int64)[None, None, :]
    O_ref, lse_ref = oracle.attn_fwd_rows(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(D),
                                          causal, rr)
    Og = to_f64(O)[:, :, rows]
    lg = to_f64(lse)[:, :, rows]
    assert_bf16_fwd(fwd_errors(Og, lg, O_ref, lse_ref), f"rows {rows}")


def test_forward_at_the_largest_key_length():
    Lq = 40
    q, k, v = _inputs(Lq, LK_MAX, seed=41)
    qd, kd, vd = (t.to(device()) for t in (q, k, v))
    announce(f"forward at Lk = {LK_MAX}")
    O, lse = fa.fa_fwd(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    _check_rows(O, lse, q, k, v, [0, 17, 39], causal=False)


def test_key_split_forward_at_the_largest_key_length():
    Lq = 3
    q, k, v = _inputs(Lq, LK_MAX, seed=42)
    qd, kd, vd = (t.to(device()) for t in (q, k, v))
    nsplit = fa.fa_fwd_splitkv_default_splits(1, 1, Lq, LK_MAX, D)
    announce(f"key-split forward at Lk = {LK_MAX}, nsplit {nsplit}")
    O, lse = fa.fa_fwd_splitkv(qd, kd, vd, causal=False, nsplit=nsplit)
    torch.cuda.synchronize()
    _check_rows(O, lse, q, k, v, [0, 1, 2], causal=False)


def test_one_key_more_is_rejected():
    q = torch.empty((1, 1, 4, D), dtype=torch.bfloat16, device=device())
    kv = torch.empty((1, 1, LK_MAX + 1, D), dtype=torch.bfloat16, device=device())
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(q, kv, kv)
    assert e.value.name == "FA_ERR_SHAPE"


def test_backward_at_the_largest_key_length_invariants():
    # At this size the oracle's backward does not fit; what holds at any size
    # is checked instead: sum_j dK_j = 0 (adding one vector to every key
    # leaves the output unchanged) and sum_j dV_j = sum_i dO_i (each row of P
    # sums to one), both relative to the sum of absolute values.
    Lq = 64
    q, k, v, do = make_inputs(1, 1, Lq, LK_MAX, D, "bf16", seed=43, with_dO=True)
    qd, kd, vd, dod = (t.to(device()) for t in (q, k, v, do))
    announce(f"backward at Lk = {LK_MAX}")
    O, lse = fa.fa_fwd(qd, kd, vd, causal=False)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, O, dod, lse, causal=False)
    torch.cuda.synchronize()
    dk64 = dk[0, 0].double()
    dv64 = dv[0, 0].double()
    s_dk = dk64.sum(0).abs().max().item()
    assert s_dk <= 1e-3 * dk64.abs().sum(0).max().item(), f"sum of dK rows {s_dk}"
    want = do[0, 0].double().sum(0).to(dv64.device)
    s_dv = (dv64.sum(0) - want).abs().max().item()
    assert s_dv <= 1e-3 * dv64.abs().sum(0).max().item() + 1e-2, f"sum of dV rows off by {s_dv}"
    assert torch.isfinite(dq).all()


def test_largest_query_length_causal():
    # Query and output offsets at the edge: Lq at the largest accepted length
    # against 100 keys, causal (rows from 99 on see every key).  Sampled rows
    # against the oracle; the backward through its two invariants.
    Lk = 100
    q, k, v, do = make_inputs(1, 1, LK_MAX, Lk, D, "bf16", seed=44, with_dO=True)
    qd, kd, vd, dod = (t.to(device()) for t in (q, k, v, do))
    announce(f"forward and backward at Lq = {LK_MAX}, Lk = {Lk}, causal")
    O, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, O, dod, lse, causal=True)
    torch.cuda.synchronize()
    _check_rows(O, lse, q, k, v, [0, 50, 99, 12345, LK_MAX - 1], causal=True)
    dk64, dv64 = dk[0, 0].double(), dv[0, 0].double()
    assert dk64.sum(0).abs().max().item() <= 1e-3 * dk64.abs().sum(0).max().item()
    want = do[0, 0].double().sum(0).to(dv64.device)
    assert (dv64.sum(0) - want).abs().max().item() <= 1e-3 * dv64.abs().sum(0).max().item() + 1e-2
    assert torch.isfinite(dq).all()
