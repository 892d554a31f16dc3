"""Host-side arithmetic of bench.py (CPU only): the FLOP and byte counts its
roofline figures divide by, the counter-summary lookup, and the refusal of
more than one GPU.  The expected values are written out from the shapes,
not taken from bench.py."""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_flops_of_the_benchmark_step(bench):
    # Two products of 2 d FLOPs per visible pair; causal keeps L^2 / 2 pairs
    # per slice; the backward is 2.5x (five products against two).
    B, H, L, d = 1, 32, 4096, 128
    fwd, bwd = bench.flops(B, H, L, L, d, True)
    assert fwd == 2 ** 37 == 4 * d * (L * L // 2) * B * H
    assert bwd == 2.5 * fwd
    fwd_nc, _ = bench.flops(B, H, L, L, d, False)
    assert fwd_nc == 2 * fwd


def test_kernel_table_bytes_and_flops(bench):
    B, H, L, d = 1, 32, 4096, 128
    t = B * H * L * d * 2            # one bf16 [B,H,L,d] tensor: 32 MiB
    r = B * H * L * 4                # one fp32 [B,H,L] vector: 512 KiB
    assert t == 32 * 2 ** 20 and r == 512 * 2 ** 10
    kt = bench.kernel_table(B, H, L, d)
    # forward: Q, K, V in, O out, lse out
    assert kt["fwd_bf16_kernel"]["bytes"] == 4 * t + r == 134_742_016
    # dK/dV: Q, K, V, dO, lse2, D in; dK, dV out
    assert kt["bwd_dkdv_kernel"]["bytes"] == 6 * t + 2 * r == 202_375_168
    # dQ with the row statistics: Q, K, V, dO, O, lse in; D, lse2 and dQ out
    assert kt["bwd_dq_kernel"]["bytes"] == 6 * t + 3 * r
    assert set(kt) == {"fwd_bf16_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"}
    f1 = 2 * d * (L * L // 2) * B * H  # one product over the visible pairs
    assert kt["fwd_bf16_kernel"]["flops"] == 2 * f1
    assert kt["bwd_dkdv_kernel"]["flops"] == 4 * f1
    assert kt["bwd_dq_kernel"]["flops"] == f1 and kt["bwd_dq_kernel"]["executed"] == 3 * f1
    # the three main kernels together carry the step's forward + backward FLOPs
    fwd, bwd = bench.flops(B, H, L, L, d, True)
    assert sum(kt[k]["flops"] for k in kt) == fwd + bwd


def test_decode_bytes(bench):
    from workloads import DECODE_WORKLOAD, WORKLOADS
    w = WORKLOADS[DECODE_WORKLOAD]
    assert (w.B, w.H, w.Lq, w.Lk, w.d) == (8, 32, 1, 16384, 128)
    kv = 2 * (8 * 32 * 16384 * 128 * 2)       # K and V, 1 GiB each
    qo = 2 * (8 * 32 * 1 * 128 * 2)          # Q in, O out
    assert bench.decode_bytes(w) == kv + qo + 8 * 32 * 4 == 2_147_615_744


def test_measured_traffic_follows_the_source(bench, tmp_path, monkeypatch):
    # A counter summary counts only while its recorded source hash is the
    # kernel source's current one.
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_sha256": bench.source_hash("fa_fwd_bf16.hip"), "traffic_bytes_per_launch": 123456}
    (tmp_path / "fwd_bf16_kernel_B1H32L4096d128_causal_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("fwd_bf16_kernel", "fa_fwd_bf16.hip") == 123456
    rec["source_sha256"] = "0" * 64
    (tmp_path / "fwd_bf16_kernel_B1H32L4096d128_causal_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("fwd_bf16_kernel", "fa_fwd_bf16.hip") is None
    assert bench.measured_traffic("no_such_kernel", "fa_fwd_bf16.hip") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_workload_byte_counts(bench):
    # Forward: Q, K, V in (element size esz), O out (o_esz), lse out (fp32).
    assert bench.fwd_bytes(4, 16, 1024, 1024, 64, 2, 2) == 4 * 16 * (4 * 1024 * 64 * 2 + 1024 * 4)
    assert bench.fwd_bytes(1, 1, 128, 128, 64, 4, 4) == 4 * 128 * 64 * 4 + 128 * 4 == 131_584
    # Longer keys than queries: K and V scale with Lk, Q and O with Lq.
    assert bench.fwd_bytes(1, 1, 10, 30, 64, 2, 4) == 10 * 64 * 2 + 2 * 30 * 64 * 2 + 10 * 64 * 4 + 40
    # Backward: Q, K, V, O, dO, lse in; dQ, dK, dV out.
    t = 2 * 16 * 2048 * 128 * 2
    assert bench.bwd_bytes(2, 16, 2048, 2048, 128, 2) == 8 * t + 2 * 16 * 2048 * 4


def test_workload_entry_arithmetic(bench):
    # 1.3744e11 FLOP in 110 us is 1249.5 TFLOP/s, half the 2500 peak; with
    # 134.7 MB the byte rate is 1225 GB/s and the intensity above the ridge.
    e = bench._entry("x", "fa_fwd", "w", 110.0, [110.0], 10, 2 ** 37, 134_742_016, 2500.0,
                     "bf16 dense matrix core")
    assert abs(e["tflops"] - 2 ** 37 / 110e-6 / 1e12) < 0.01
    assert abs(e["frac_of_peak"] - 2 ** 37 / 110e-6 / 1e12 / 2500.0) < 1e-4
    assert abs(e["hbm_gbs"] - 134_742_016 / 110e-6 / 1e9) < 0.1
    assert e["ridge_flop_per_byte"] == 312.5 and e["bound"] == "mfma"
    low = bench._entry("y", "fa_fwd", "w", 10.0, [10.0], 10, 1e6, 1e6, 2500.0, "bf16 dense matrix core")
    assert low["bound"] == "hbm"
