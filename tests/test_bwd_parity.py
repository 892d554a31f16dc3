"""Backward parity: libfa's fa_bwd (HIP, gfx950) against the fp64 oracle on
the same seeded inputs, through the C ABI.  The GPU backward consumes the
GPU forward's own O and lse, as a training step would.  Needs an MI355X."""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_13_amd as fa
from tests.gpu_util import BF16_GRAD_REL, F32_REL, announce, f64, rel_to_max, to_dev
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu


def _gpu_grads(q, k, v, do, scale, causal):
    qd, kd, vd, dod = to_dev(q, k, v, do)
    O, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, O, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return f64(dq), f64(dk), f64(dv)


def _assert_grads(got, ref, tol, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        e = rel_to_max(g, r)
        assert e <= tol, f"{what}: {name} max|d|/max|ref| = {e:.3e} > {tol}"


SMALL = [
    (1, 1, 1, 1, 64), (1, 2, 1, 1, 128), (1, 1, 3, 17, 128), (2, 3, 129, 129, 64),
    (1, 2, 200, 333, 128), (1, 1, 1000, 1000, 128), (1, 2, 17, 300, 64), (1, 2, 300, 17, 128),
    (2, 2, 256, 256, 128), (1, 1, 127, 129, 128), (1, 2, 64, 64, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
def test_bf16_small_shapes(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v, do = make_inputs(B, H, Lq, Lk, d, "bf16", seed=Lq + 3 * Lk + d, with_dO=True)
    scale = 1.0 / math.sqrt(d)
    announce(f"bwd bf16 {shape} causal={causal}")
    got = _gpu_grads(q, k, v, do, scale, causal)
    ref = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), scale, causal)
    _assert_grads(got, ref, BF16_GRAD_REL, f"{shape} causal={causal}")


# The launcher picks 4, 8 or 16 columns per lane by grid size: 4 for
# (1, 2, 1, 1, 64), (1, 2, 200, 130, 64) and (1, 1, 128, 100, 128); 8 for
# (2, 1, 65, 300, 128) and (1, 3, 601, 601, 64) (ragged); 16 for (1, 8, 512,
# 512, 64).
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 64), (2, 1, 65, 300, 128), (1, 2, 200, 130, 64),
                                   (1, 1, 128, 100, 128), (1, 3, 601, 601, 64),
                                   (1, 8, 512, 512, 64)],
                         ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
def test_f32_small_shapes(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v, do = make_inputs(B, H, Lq, Lk, d, "f32", seed=9, with_dO=True)
    announce(f"bwd f32 {shape} causal={causal}")
    got = _gpu_grads(q, k, v, do, 0.15, causal)
    ref = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), 0.15, causal)
    _assert_grads(got, ref, F32_REL, f"f32 {shape} causal={causal}")


def test_backward_workload_every_head():
    # B2 H16 L2048 d128 causal, every element of every head.
    w = WORKLOADS["bwd_bf16_causal_B2H16L2048d128"]
    q, k, v, do = workload_inputs(w)
    announce(f"bwd {w.name}")
    got = _gpu_grads(q, k, v, do, w.scale, True)
    ref = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), w.scale, True)
    _assert_grads(got, ref, BF16_GRAD_REL, w.name)


def test_benchmark_shape_backward_sampled_heads_and_invariants():
    # The benchmark step's backward at B1 H32 L4096 d128 causal: four heads
    # element by element, and on every head the invariants
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.
    w = WORKLOADS["fwd_bf16_causal_B1H32L4096d128"]
    q, k, v, do = make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed, amp=w.amp,
                              with_dO=True)
    announce("bwd benchmark shape")
    dq, dk, dv = _gpu_grads(q, k, v, do, w.scale, True)
    heads = [(0, 0), (0, 7), (0, 20), (0, 31)]
    ref = oracle.attn_bwd_heads(f64(q), f64(k), f64(v), f64(do), w.scale, True, heads)
    for n, (b, h) in enumerate(heads):
        _assert_grads((dq[b, h], dk[b, h], dv[b, h]), (ref[0][n], ref[1][n], ref[2][n]),
                      BF16_GRAD_REL, f"head {h}")
    sum_dk = dk.sum(axis=2)
    assert np.abs(sum_dk).max() <= 2e-2 * np.abs(dk).max() * math.sqrt(w.Lk), "sum dK"
    sum_dv, sum_do = dv.sum(axis=2), f64(do).sum(axis=2)
    assert np.abs(sum_dv - sum_do).max() <= 2e-2 * np.abs(sum_do).max(), "sum dV = sum dO"


def test_empty_queries_give_zero_key_gradients():
    q, k, v, do = make_inputs(1, 2, 0, 40, 64, "bf16", seed=2, with_dO=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=qd.device)
    announce("bwd Lq=0")
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, torch.empty_like(qd), dod, lse, causal=False, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def test_autograd_matches_direct_calls():
    q, k, v, do = make_inputs(1, 2, 150, 150, 128, "bf16", seed=4, with_dO=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    qd.requires_grad_(True)
    kd.requires_grad_(True)
    vd.requires_grad_(True)
    announce("attention() backward")
    O = fa.attention(qd, kd, vd, causal=True)
    O.backward(dod)
    O2, lse = fa.fa_fwd(qd.detach(), kd.detach(), vd.detach(), causal=True)
    dq, dk, dv = fa.fa_bwd(qd.detach(), kd.detach(), vd.detach(), O2, dod, lse, causal=True)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), 1 / math.sqrt(128), True)
    _assert_grads((f64(qd.grad), f64(kd.grad), f64(vd.grad)), ref, BF16_GRAD_REL, "autograd")
    assert torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stages_equal_fused_call_across_two_streams(dtype):
    # fa_bwd_prepare, then fa_bwd_dkdv and fa_bwd_dq on two different
    # streams, give the same bits as fa_bwd.
    q, k, v, do = make_inputs(1, 3, 333, 333, 128, dtype, seed=12, with_dO=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    announce(f"bwd stages {dtype}")
    O, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    ref = fa.fa_bwd(qd, kd, vd, O, dod, lse, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(qd.dtype, 1, 3, 333, 333, 128), dtype=torch.uint8,
                     device=qd.device)
    fa.fa_bwd_prepare(O, dod, lse, 333, ws)
    ready = torch.cuda.Event()
    ready.record()
    side = torch.cuda.Stream()
    side.wait_event(ready)
    with torch.cuda.stream(side):
        dq = fa.fa_bwd_dq(qd, kd, vd, dod, ws, causal=True)
    dk, dv = fa.fa_bwd_dkdv(qd, kd, vd, dod, ws, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, ref[0]) and torch.equal(dk, ref[1]) and torch.equal(dv, ref[2])


@pytest.mark.parametrize("dtype,o32", [("bf16", False), ("bf16", True), ("f32", False)],
                         ids=["bf16", "bf16-fp32O", "f32"])
@pytest.mark.parametrize("shape,causal", [((1, 3, 333, 333, 128), True), ((2, 2, 200, 517, 64), False),
                                          ((1, 2, 517, 300, 64), True)],
                         ids=["B1H3L333d128c", "B2H2Lq200Lk517d64n", "B1H2Lq517Lk300d64c"])
def test_prepare_dq_then_dkdv_equals_fa_bwd(dtype, o32, shape, causal):
    # fa_bwd_prepare_dq (one kernel when O is bf16) then fa_bwd_dkdv give
    # fa_bwd's bits, and the statistics it leaves in the workspace are
    # fa_bwd_prepare's bit for bit.
    B, H, Lq, Lk, d = shape
    q, k, v, do = make_inputs(B, H, Lq, Lk, d, dtype, seed=7 * Lq + d, with_dO=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    announce(f"bwd prepare_dq {dtype} fp32O={o32} {shape} causal={causal}")
    kw = dict(out_dtype=torch.float32) if o32 else {}
    O, lse = fa.fa_fwd(qd, kd, vd, causal=causal, **kw)
    ref = fa.fa_bwd(qd, kd, vd, O, dod, lse, causal=causal)
    nbytes = fa.fa_bwd_workspace_bytes(qd.dtype, B, H, Lq, Lk, d)
    ws1 = torch.zeros(nbytes, dtype=torch.uint8, device=qd.device)
    ws2 = torch.zeros(nbytes, dtype=torch.uint8, device=qd.device)
    dq = fa.fa_bwd_prepare_dq(qd, kd, vd, O, dod, lse, ws1, causal=causal)
    dk, dv = fa.fa_bwd_dkdv(qd, kd, vd, dod, ws1, causal=causal)
    fa.fa_bwd_prepare(O, dod, lse, Lk, ws2)
    torch.cuda.synchronize()
    assert torch.equal(ws1, ws2)
    assert torch.equal(dq, ref[0]) and torch.equal(dk, ref[1]) and torch.equal(dv, ref[2])
    got = (f64(dq), f64(dk), f64(dv))
    want = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), 1 / math.sqrt(d), causal)
    _assert_grads(got, want, BF16_GRAD_REL if dtype == "bf16" else F32_REL,
                  f"prepare_dq {dtype} {shape}")


def _gpu_grads_f32_out(q, k, v, do, scale, causal):
    # The forward's fp32-output variant, whose O goes into the backward as
    # fp32 (o_dtype = FA_F32); dO stays bf16.
    qd, kd, vd, dod = to_dev(q, k, v, do)
    O, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal, out_dtype=torch.float32)
    assert O.dtype == torch.float32
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, O, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return f64(dq), f64(dk), f64(dv)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 64), (1, 2, 200, 333, 128), (2, 3, 129, 129, 64),
                                   (1, 2, 300, 17, 128), (2, 2, 256, 256, 128)],
                         ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
def test_bf16_inputs_fp32_output_backward(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v, do = make_inputs(B, H, Lq, Lk, d, "bf16", seed=5 * Lq + Lk + d, with_dO=True)
    scale = 1.0 / math.sqrt(d)
    announce(f"bwd bf16 with fp32 O {shape} causal={causal}")
    got = _gpu_grads_f32_out(q, k, v, do, scale, causal)
    ref = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), scale, causal)
    _assert_grads(got, ref, BF16_GRAD_REL, f"fp32 O {shape} causal={causal}")


def test_backward_workload_fp32_output_every_head():
    # B2 H16 L2048 d128 causal with the forward's fp32 O fed to the backward.
    w = WORKLOADS["bwd_bf16_causal_B2H16L2048d128"]
    q, k, v, do = workload_inputs(w)
    announce(f"bwd {w.name} fp32 O")
    got = _gpu_grads_f32_out(q, k, v, do, w.scale, True)
    ref = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), w.scale, True)
    _assert_grads(got, ref, BF16_GRAD_REL, w.name + " fp32 O")


def test_fp32_output_statistics_only_differ_through_o():
    # fa_bwd_prepare with fp32 O reads the same dO and lse; only D differs,
    # and by no more than the bf16 rounding of O can move it.
    q, k, v, do = make_inputs(1, 2, 300, 300, 128, "bf16", seed=31, with_dO=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    announce("bwd prepare fp32 O vs bf16 O")
    O32, lse = fa.fa_fwd(qd, kd, vd, causal=True, out_dtype=torch.float32)
    nbytes = fa.fa_bwd_workspace_bytes(torch.bfloat16, 1, 2, 300, 300, 128)
    ws32 = torch.empty(nbytes, dtype=torch.uint8, device=qd.device)
    ws16 = torch.empty(nbytes, dtype=torch.uint8, device=qd.device)
    fa.fa_bwd_prepare(O32, dod, lse, 300, ws32)
    fa.fa_bwd_prepare(O32.to(torch.bfloat16), dod, lse, 300, ws16)
    torch.cuda.synchronize()
    rows = 2 * 300
    stat = -(-rows * 4 // 256) * 256
    d32 = ws32[:rows * 4].view(torch.float32).double().cpu()
    d16 = ws16[:rows * 4].view(torch.float32).double().cpu()
    l32 = ws32[stat:stat + rows * 4].view(torch.float32)
    l16 = ws16[stat:stat + rows * 4].view(torch.float32)
    assert torch.equal(l32, l16)
    # D = -rowsum(dO * O) in fp64 from the fp32 O (the bf16 path stores -D).
    d_ref = -(f64(do).reshape(rows, 128) * f64(O32).reshape(rows, 128)).sum(axis=1)
    assert np.abs(d32.numpy() - d_ref).max() <= 1e-4 * max(1.0, np.abs(d_ref).max())
    assert not torch.equal(d32, d16)
