"""Key-split forward (fa_fwd_splitkv and its two stages) against the fp64
oracle, on the GPU through the C ABI.

What is checked:
* the whole call against the plain definition (oracle.attn_fwd) at the bf16
  forward tolerances, over short and long query blocks, ragged key lengths,
  both masks, both head dimensions, split counts from one to more ranges
  than there are keys, and bf16 and fp32 outputs;
* the partial stage alone: every range's normalised output and lse against
  the oracle's attention over that key range (oracle.attn_fwd_keyrange),
  including rows that see no key of a range (O = 0, lse = -inf exactly);
* the merge stage alone, fed the oracle's own per-range results, against the
  oracle's merge (fp32 arithmetic: 1e-5 relative);
* the decode workload (B8 H32, one query row, 16384 keys, d=128) in full,
  at the split count the library picks and in the launch configuration the
  benchmark times;
* invalid calls, and bitwise-identical results from repeated calls.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_13_amd as fa
from exact_io_aware_13_amd import _lib
from tests.gpu_util import announce, assert_bf16_fwd, device, fwd_errors, to_dev
from workloads import DECODE_WORKLOAD, WORKLOADS, make_inputs, to_f64

pytestmark = pytest.mark.gpu

TILE = 64  # keys per tile; ranges are whole tiles


def _chunk(Lk, nsplit):
    return -(-(-(-Lk // nsplit)) // TILE) * TILE


def _ranges(Lk, nsplit):
    c = _chunk(Lk, nsplit)
    return [(min(s * c, Lk), min((s + 1) * c, Lk)) for s in range(nsplit)]


def _inputs(B, H, Lq, Lk, d, seed):
    q, k, v = make_inputs(B, H, Lq, Lk, d, "bf16", seed=seed)
    return q, k, v, to_f64(q), to_f64(k), to_f64(v)


def _read_workspace(ws, B, H, Lq, d, nsplit):
    n_o = nsplit * B * H * Lq * d
    off = -(-n_o * 4 // 256) * 256
    raw = ws.cpu()
    Op = raw[: n_o * 4].view(torch.float32).reshape(nsplit, B, H, Lq, d).double().numpy()
    lp = raw[off: off + nsplit * B * H * Lq * 4].view(torch.float32).reshape(
        nsplit, B, H, Lq).double().numpy()
    return Op, lp


CASES = [
    # B, H, Lq, Lk, d, causal, nsplit (None: library default)
    (1, 2, 1, 1, 128, False, 1),
    (1, 2, 1, 1, 64, False, 3),
    (2, 3, 1, 1000, 128, False, None),
    (2, 3, 1, 1000, 64, True, None),
    (1, 2, 5, 777, 128, False, 4),
    (1, 2, 16, 4097, 128, False, 7),
    (1, 1, 17, 300, 64, True, 2),
    (1, 2, 40, 513, 128, True, 3),
    (2, 2, 33, 2048, 64, False, 16),
    (1, 1, 1, 65, 128, False, 2),
    (1, 2, 100, 100, 128, True, 5),
    (1, 1, 3, 640, 128, False, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Lq{}Lk{}d{}-{}-n{}".format(*c))
def test_splitkv_matches_oracle(case):
    B, H, Lq, Lk, d, causal, nsplit = case
    q, k, v, q64, k64, v64 = _inputs(B, H, Lq, Lk, d, seed=Lq * 131 + Lk)
    scale = 1.0 / math.sqrt(d)
    O_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, causal)
    qd, kd, vd = to_dev(q, k, v)
    announce(f"splitkv {case}")
    for out_dtype in (torch.bfloat16, torch.float32):
        O, lse = fa.fa_fwd_splitkv(qd, kd, vd, scale=scale, causal=causal, nsplit=nsplit,
                                   out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert_bf16_fwd(fwd_errors(to_f64(O), to_f64(lse), O_ref, lse_ref),
                        f"{case} out {out_dtype}")


@pytest.mark.parametrize("case", [(1, 2, 5, 777, 128, False, 4), (1, 2, 40, 513, 128, True, 3),
                                  (1, 1, 17, 300, 64, True, 2), (1, 1, 3, 200, 64, False, 9)],
                         ids=lambda c: "B{}H{}Lq{}Lk{}d{}-{}-n{}".format(*c))
def test_partial_stage_matches_oracle_ranges(case):
    B, H, Lq, Lk, d, causal, nsplit = case
    q, k, v, q64, k64, v64 = _inputs(B, H, Lq, Lk, d, seed=7 + Lk)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = to_dev(q, k, v)
    need = fa.fa_fwd_splitkv_workspace_bytes(torch.bfloat16, B, H, Lq, Lk, d, nsplit)
    ws = torch.empty(need, dtype=torch.uint8, device=device())
    announce(f"splitkv partial {case}")
    fa.fa_fwd_splitkv_partial(qd, kd, vd, ws, nsplit, scale=scale, causal=causal)
    torch.cuda.synchronize()
    Op, lp = _read_workspace(ws, B, H, Lq, d, nsplit)
    for s, (a, b) in enumerate(_ranges(Lk, nsplit)):
        O_s, l_s = oracle.attn_fwd_keyrange(q64, k64, v64, scale, causal, a, b)
        empty = np.isneginf(l_s)
        assert np.array_equal(np.isneginf(lp[s]), empty), f"range {s}: rows without keys differ"
        assert np.all(Op[s][empty] == 0.0), f"range {s}: rows without keys must be 0"
        if (~empty).any():
            e = fwd_errors(Op[s][~empty], lp[s][~empty], O_s[~empty], l_s[~empty])
            assert_bf16_fwd(e, f"range {s} [{a}, {b})")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_stage_matches_oracle_merge(d, out_dtype):
    B, H, Lq, Lk, nsplit = 2, 3, 7, 500, 5
    q, k, v, q64, k64, v64 = _inputs(B, H, Lq, Lk, d, seed=11)
    parts = [oracle.attn_fwd_keyrange(q64, k64, v64, 0.3, True, a, b) for a, b in _ranges(Lk, nsplit)]
    Op = np.stack([p[0] for p in parts]).astype(np.float32)
    lp = np.stack([p[1] for p in parts]).astype(np.float32)
    O_ref, lse_ref = oracle.merge_partials(Op.astype(np.float64), lp.astype(np.float64))
    need = fa.fa_fwd_splitkv_workspace_bytes(torch.bfloat16, B, H, Lq, Lk, d, nsplit)
    host = torch.zeros(need, dtype=torch.uint8)
    n_o = Op.size
    host[: n_o * 4] = torch.from_numpy(Op.reshape(-1).copy()).view(torch.uint8)
    off = -(-n_o * 4 // 256) * 256
    host[off: off + lp.size * 4] = torch.from_numpy(lp.reshape(-1).copy()).view(torch.uint8)
    ws = host.to(device())
    O = torch.empty((B, H, Lq, d), dtype=out_dtype, device=device())
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=device())
    announce(f"splitkv merge d{d} {out_dtype}")
    fa.fa_fwd_splitkv_merge(ws, B, H, Lq, d, nsplit, O, lse)
    torch.cuda.synchronize()
    tol_o = 1e-5 if out_dtype == torch.float32 else 2.0 ** -8
    err_o = np.abs(to_f64(O) - O_ref).max() / max(1.0, np.abs(O_ref).max())
    assert err_o <= tol_o, err_o
    assert np.abs(to_f64(lse) - lse_ref).max() <= 1e-5 * max(1.0, np.abs(lse_ref).max())


def test_decode_workload_full():
    w = WORKLOADS[DECODE_WORKLOAD]
    q, k, v = make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed, amp=w.amp)
    O_ref, lse_ref = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), w.scale, False)
    qd, kd, vd = to_dev(q, k, v)
    nsplit = fa.fa_fwd_splitkv_default_splits(w.B, w.H, w.Lq, w.Lk, w.d)
    announce(f"splitkv decode workload nsplit {nsplit}")
    O, lse = fa.fa_fwd_splitkv(qd, kd, vd, scale=w.scale, causal=False, nsplit=nsplit)
    torch.cuda.synchronize()
    assert_bf16_fwd(fwd_errors(to_f64(O), to_f64(lse), O_ref, lse_ref), "decode workload")
    # A second split count over the same inputs agrees within rounding.
    O2, lse2 = fa.fa_fwd_splitkv(qd, kd, vd, scale=w.scale, causal=False, nsplit=nsplit * 2 + 1)
    torch.cuda.synchronize()
    assert_bf16_fwd(fwd_errors(to_f64(O2), to_f64(lse2), O_ref, lse_ref), "decode, other split")


def test_repeat_calls_are_bitwise_identical():
    q, k, v = to_dev(*make_inputs(2, 4, 3, 3000, 128, "bf16", seed=12))
    announce("splitkv determinism")
    a = fa.fa_fwd_splitkv(q, k, v, nsplit=6)
    b = fa.fa_fwd_splitkv(q, k, v, nsplit=6)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_invalid_calls_are_rejected():
    dev = device()
    q, k, v = to_dev(*make_inputs(1, 1, 2, 100, 128, "bf16", seed=0))
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv(q.float(), k.float(), v.float(), nsplit=2)
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv(q, k, v, nsplit=0, workspace=torch.empty(1 << 16, dtype=torch.uint8,
                                                                   device=dev))
    assert e.value.name == "FA_ERR_ARG"
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv(q, k, v, nsplit=2, workspace=torch.empty(16, dtype=torch.uint8, device=dev))
    assert e.value.name == "FA_ERR_WORKSPACE"
