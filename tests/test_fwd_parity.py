"""Forward parity: libfa's fa_fwd (HIP, gfx950) against the fp64 oracle on
the same seeded inputs, through the C ABI.  Needs an MI355X."""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_13_amd as fa
from tests.gpu_util import (F32_REL, announce, assert_bf16_fwd, device, f64, fwd_errors,
                            rel_to_max, to_dev)
from workloads import WORKLOADS, make_inputs, sample_rows, workload_inputs

pytestmark = pytest.mark.gpu


# Several tiles and ragged tails in both lengths, both masks, Lq != Lk.
SMALL = [
    (1, 1, 1, 1, 64), (1, 2, 1, 1, 128), (1, 1, 3, 17, 128), (2, 3, 129, 129, 64),
    (1, 2, 200, 333, 128), (1, 1, 1000, 1000, 128), (1, 2, 17, 300, 64), (1, 2, 300, 17, 128),
    (2, 2, 256, 256, 128), (1, 3, 64, 64, 64), (1, 1, 127, 129, 128), (1, 2, 511, 1025, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
def test_bf16_small_shapes(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v = make_inputs(B, H, Lq, Lk, d, "bf16", seed=Lq * 7 + Lk + d)
    scale = 1.0 / math.sqrt(d)
    announce(f"fwd bf16 {shape} causal={causal}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attn_fwd(f64(q), f64(k), f64(v), scale, causal)
    assert O.dtype == torch.bfloat16 and lse.dtype == torch.float32
    assert_bf16_fwd(fwd_errors(f64(O), f64(lse), O_ref, lse_ref), f"{shape} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 200, 333, 128), (2, 2, 130, 130, 64)],
                         ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
def test_bf16_inputs_fp32_output(shape, causal):
    # The fp32 output skips the final bf16 rounding: tighter than bf16 O.
    B, H, Lq, Lk, d = shape
    q, k, v = make_inputs(B, H, Lq, Lk, d, "bf16", seed=11)
    announce(f"fwd bf16->f32 {shape} causal={causal}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=0.1, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attn_fwd(f64(q), f64(k), f64(v), 0.1, causal)
    e = fwd_errors(f64(O), f64(lse), O_ref, lse_ref)
    assert e["o_max"] <= 5e-3 and e["o_mean"] <= 5e-4 and e["lse_max"] <= 1e-3, e


def test_f32_workload():
    w = WORKLOADS["fwd_f32_B1H1L128d64"]
    q, k, v = workload_inputs(w)
    for causal in (False, True):
        announce(f"fwd f32 {w.name} causal={causal}")
        O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        O_ref, lse_ref = oracle.attn_fwd(f64(q), f64(k), f64(v), w.scale, causal)
        assert O.dtype == torch.float32
        assert rel_to_max(f64(O), O_ref) <= F32_REL
        assert rel_to_max(f64(lse), lse_ref) <= F32_REL


# The launcher picks 4, 8 or 16 columns per lane by grid size: at d = 64
# (1, 3, 300, 300) takes 4, (1, 3, 601, 601) 8 (ragged), (1, 7, 512, 512) 16
# with eight waves; at d = 128 (2, 1, 65, 300) takes 4, (1, 2, 300, 300) 8,
# (1, 4, 512, 512) 16.
@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 64), (2, 1, 65, 300, 128), (1, 3, 300, 300, 64),
                                   (1, 3, 601, 601, 64), (1, 7, 512, 512, 64),
                                   (1, 2, 300, 300, 128), (1, 4, 512, 512, 128)],
                         ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
@pytest.mark.parametrize("causal", [False, True])
def test_f32_small_shapes(shape, causal):
    B, H, Lq, Lk, d = shape
    q, k, v = make_inputs(B, H, Lq, Lk, d, "f32", seed=5)
    announce(f"fwd f32 {shape} causal={causal}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=0.2, causal=causal)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attn_fwd(f64(q), f64(k), f64(v), 0.2, causal)
    assert rel_to_max(f64(O), O_ref) <= F32_REL
    assert rel_to_max(f64(lse), lse_ref) <= F32_REL


@pytest.mark.parametrize("causal", [False, True])
def test_short_sequence_batch_workload_full(causal):
    # Every element of B4 H16 L1024 d64, both masks, against the full oracle.
    w = WORKLOADS["fwd_bf16_B4H16L1024d64"]
    q, k, v = workload_inputs(w)
    announce(f"fwd {w.name} causal={causal}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attn_fwd(f64(q), f64(k), f64(v), w.scale, causal)
    assert_bf16_fwd(fwd_errors(f64(O), f64(lse), O_ref, lse_ref), w.name)


def test_benchmark_workload_sampled_rows_and_full_heads():
    # B1 H32 L4096 d128 causal: 256 seeded rows of every head, plus two heads
    # compared element by element.
    w = WORKLOADS["fwd_bf16_causal_B1H32L4096d128"]
    q, k, v = workload_inputs(w)
    announce(f"fwd {w.name}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    O, lse = f64(O), f64(lse)
    qd, kd, vd = f64(q), f64(k), f64(v)
    rows = sample_rows(H=w.H, L=w.Lq, n=256, seed=w.seed).numpy()
    O_ref, lse_ref = oracle.attn_fwd_rows(qd, kd, vd, w.scale, True, rows)
    Og = np.take_along_axis(O, rows[..., None], axis=2)
    lg = np.take_along_axis(lse, rows, axis=2)
    assert_bf16_fwd(fwd_errors(Og, lg, O_ref, lse_ref), w.name + " sampled rows")
    for h in (0, 31):
        Oh, lh = oracle.attn_fwd(qd[:, h:h + 1], kd[:, h:h + 1], vd[:, h:h + 1], w.scale, True)
        assert_bf16_fwd(fwd_errors(O[:, h:h + 1], lse[:, h:h + 1], Oh, lh), f"{w.name} head {h}")


def test_long_context_workload_sampled_rows():
    # B1 H8 L32768 d128 causal: 256 seeded rows per head (rows 0 and 32767
    # included), each a full fp64 row over its visible keys.
    w = WORKLOADS["fwd_bf16_causal_B1H8L32768d128"]
    q, k, v = workload_inputs(w)
    announce(f"fwd {w.name}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(H=w.H, L=w.Lq, n=w.sample_rows, seed=w.seed).numpy()
    O_ref, lse_ref = oracle.attn_fwd_rows(f64(q), f64(k), f64(v), w.scale, True, rows)
    Og = np.take_along_axis(f64(O), rows[..., None], axis=2)
    lg = np.take_along_axis(f64(lse), rows, axis=2)
    assert_bf16_fwd(fwd_errors(Og, lg, O_ref, lse_ref), w.name)


@pytest.mark.parametrize("shape", [(1, 2, 4100, 4100, 128), (1, 2, 8200, 8200, 64),
                                   (1, 2, 3000, 4500, 128), (1, 1, 5000, 4097, 128)],
                         ids=lambda s: "B{}H{}Lq{}Lk{}d{}".format(*s))
def test_split_key_halves_long_causal(shape):
    # Few workgroups and at least 128 key tiles: the launch splits each
    # workgroup's keys over two wave groups and merges them.  256 seeded
    # rows per head (the first and last included), plus one full head.
    B, H, Lq, Lk, d = shape
    q, k, v = make_inputs(B, H, Lq, Lk, d, "bf16", seed=Lq + Lk + d)
    scale = 1.0 / math.sqrt(d)
    announce(f"fwd bf16 split halves {shape}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale, causal=True)
    torch.cuda.synchronize()
    O, lse = f64(O), f64(lse)
    qd, kd, vd = f64(q), f64(k), f64(v)
    rows = sample_rows(H=H, L=Lq, n=256, seed=d).numpy()
    O_ref, lse_ref = oracle.attn_fwd_rows(qd, kd, vd, scale, True, rows)
    Og = np.take_along_axis(O, rows[..., None], axis=2)
    lg = np.take_along_axis(lse, rows, axis=2)
    assert_bf16_fwd(fwd_errors(Og, lg, O_ref, lse_ref), f"{shape} sampled rows")
    if Lq * Lk <= 4100 * 4100:
        Oh, lh = oracle.attn_fwd(qd[:, :1], kd[:, :1], vd[:, :1], scale, True)
        assert_bf16_fwd(fwd_errors(O[:, :1], lse[:, :1], Oh, lh), f"{shape} head 0")


def test_constant_values_are_returned_at_full_size():
    # Property that holds at any size: constant V rows give O = that row.
    B, H, L, d = 1, 4, 4096, 128
    q, k, _ = make_inputs(B, H, L, L, d, "bf16", seed=21)
    c = torch.linspace(-2, 2, d).to(torch.bfloat16)
    v = c.expand(B, H, L, d).contiguous()
    announce("fwd constant V")
    O, _ = fa.fa_fwd(*to_dev(q, k, v), scale=1 / math.sqrt(d), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O.cpu(), v[:, :, :L].cpu())


def test_empty_query_length():
    q, k, v = make_inputs(1, 2, 0, 5, 64, "bf16", seed=1)
    announce("fwd Lq=0")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), causal=True)
    assert O.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)


def test_unsupported_head_dim_raises():
    q, k, v = make_inputs(1, 1, 8, 8, 96, "bf16", seed=1)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(*to_dev(q, k, v))
    assert e.value.name == "FA_ERR_UNSUPPORTED"


def test_autograd_wrapper_forward_matches():
    q, k, v = make_inputs(1, 2, 100, 100, 64, "bf16", seed=3)
    qd, kd, vd = to_dev(q, k, v)
    announce("attention() forward")
    O = fa.attention(qd, kd, vd, causal=True)
    O2, _ = fa.fa_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    assert device().type == "cuda"


# ---- softmax reference moves after the first tile ---------------------------
# The forward keeps a row's softmax reference until a tile's probabilities
# against it grow past a bound; these inputs make later tiles' scores exceed
# the first tile's by far, so the reference moves (once, several times, or
# by hundreds of units), with both masks and a ragged tail.

def _reference_move_inputs(kind, Lq, Lk, d, seed):
    q, k, v = make_inputs(1, 2, Lq, Lk, d, "bf16", seed=seed)
    qf, kf = q.float(), k.float()
    if kind == "ramp":        # scores grow along the keys: many moves
        kf = kf * torch.linspace(0.5, 6.0, Lk).view(1, 1, Lk, 1)
    elif kind == "late_key":  # one late key wins every row by ~30 log2 units
        qf[..., 0] = 4.0
        kf[:, :, Lk - 5] = 0.0
        kf[:, :, Lk - 5, 0] = 60.0
    elif kind == "huge_gap":  # one late key wins every row by ~1000 log2 units
        qf[..., 0] = 4.0
        kf[:, :, Lk - 5] = 0.0
        kf[:, :, Lk - 5, 0] = 2000.0
    elif kind == "spread":    # large score spread everywhere
        qf, kf = qf * 3.0, kf * 3.0
    return qf.to(torch.bfloat16), kf.to(torch.bfloat16), v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["ramp", "late_key", "huge_gap", "spread"])
@pytest.mark.parametrize("d", [64, 128])
def test_reference_moves_late(kind, causal, d):
    Lq, Lk = 300, 1000
    q, k, v = _reference_move_inputs(kind, Lq, Lk, d, seed=71 + d)
    scale = 1.0 / math.sqrt(d)
    announce(f"fwd reference moves {kind} d{d} causal={causal}")
    O, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attn_fwd(f64(q), f64(k), f64(v), scale, causal)
    assert np.isfinite(f64(O)).all() and np.isfinite(f64(lse)).all()
    # Peaked rows put nearly all weight on a few keys, so the bf16 rounding
    # of those probabilities (for the value product) and of the output is
    # not averaged away.  Each rounds to nearest with unit roundoff
    # u = 2^-8, so per element |dO_ic| <= 2u sum_j P_ij |V_jc|: the oracle's
    # output with |V| as the values bounds the error, elementwise and hence
    # in the mean (the 1e-2 / 1e-3 bars hold for spread-out rows of N(0,1)
    # values).  lse does not depend on V.
    e = fwd_errors(f64(O), f64(lse), O_ref, lse_ref)
    O_abs, _ = oracle.attn_fwd(f64(q), f64(k), np.abs(f64(v)), scale, causal)
    u = 2.0 ** -8
    what = f"{kind} d{d} causal={causal}"
    assert e["o_max"] <= 2 * u * O_abs.max(), f"{what}: {e}"
    assert e["o_mean"] <= 2 * u * O_abs.mean(), f"{what}: {e}"
    assert e["lse_max"] <= 1e-3, f"{what}: {e}"
