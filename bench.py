"""Benchmark: exact attention forward + backward on one MI355X.

One step is one pass of the whole hot path over one batch: fa_fwd (O, lse)
then fa_bwd (D statistic, dQ/dK/dV) through the C ABI, at B1 H32 L4096
d128, causal, bf16 inputs with fp32 accumulation.  Inputs, outputs and the
workspace are resident in device memory before timing starts.

Throughput uses the algorithmic FLOP count: forward 4*B*H*Lq*Lk*d, halved
for the causal mask, backward 2.5x the forward.  The line also carries the
dominant kernel's roofline position (timed with HIP events on the stream the
library launches on) and the fp64 CPU oracle timed on a bounded sample of
the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import exact_io_aware_13_amd as fa  # noqa: E402
from workloads import BENCH_WORKLOAD, WORKLOADS, make_inputs  # noqa: E402

METRIC = "attn fwd+bwd TFLOP/s & % bf16 MFMA peak, B1 H32 L4096 d128 causal"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E peak (published)


def flops(B, H, Lq, Lk, d, causal):
    fwd = 4.0 * B * H * Lq * Lk * d * (0.5 if causal else 1.0)
    return fwd, 2.5 * fwd


def hbm_bytes(B, H, Lq, Lk, d):
    """Algorithmic bytes: each tensor read or written once (bf16, fp32 stats)."""
    q, kv = B * H * Lq * d * 2, B * H * Lk * d * 2
    stats = B * H * Lq * 4
    fwd = q + 2 * kv + q + stats                            # Q, K, V in; O, lse out
    bwd = (q + 2 * kv + q + q + stats) + (q + 2 * kv)       # Q K V O dO lse in; dQ dK dV out
    return fwd, bwd


def cpu_baseline(w, seconds_target=15.0):
    """The fp64 oracle (forward + backward) on whole heads of the workload."""
    import numpy as np
    import oracle
    from workloads import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
    q, k, v, do = make_inputs(1, 1, w.Lq, w.Lk, w.d, w.dtype, seed=w.seed, amp=w.amp, with_dO=True)
    q, k, v, do = (to_f64(t) for t in (q, k, v, do))
    heads, t0 = 0, time.perf_counter()
    while True:
        oracle.attn_fwd(q, k, v, w.scale, True)
        oracle.attn_bwd(q, k, v, do, w.scale, True)
        heads += 1
        el = time.perf_counter() - t0
        if el >= seconds_target or heads >= w.H:
            break
    f_fwd, f_bwd = flops(1, heads, w.Lq, w.Lk, w.d, True)
    return {"value": (f_fwd + f_bwd) / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {w.H} heads (fwd+bwd, fp64 numpy, full S per head), "
                      f"{el:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        x = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4,
                          "launches": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the attention kernels run per device with no "
              f"cross-GPU exchange); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    w = WORKLOADS[BENCH_WORKLOAD]
    dev = torch.device("cuda", 0)
    B, H, L, d = w.B, w.H, w.Lq, w.d
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, L, L, d, "bf16", seed=w.seed, amp=w.amp,
                                                  with_dO=True))
    O = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(torch.bfloat16, B, H, L, L, d), dtype=torch.uint8,
                     device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, scale=w.scale, causal=True, out=O, lse=lse)
        if ev is not None:
            ev[1].record()
        fa.fa_bwd(q, k, v, O, do, lse, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    f_fwd, f_bwd = flops(B, H, L, L, d, True)
    b_fwd, b_bwd = hbm_bytes(B, H, L, L, d)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    if bwd_ms >= fwd_ms:
        dom, dom_flops, dom_ms, dom_bytes = "fa_bwd (bwd_pre, bwd_main, dq_convert)", f_bwd, bwd_ms, b_bwd
    else:
        dom, dom_flops, dom_ms, dom_bytes = "fwd_bf16_kernel", f_fwd, fwd_ms, b_fwd
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "exact attention fwd+bwd B1 H32 L4096 d128 causal",
                   "B": B, "H": H, "L": L, "d": d, "causal": True, "scale": w.scale,
                   "inputs": "0.5*N(0,1) seed 2, bf16"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_bytes": dom_bytes,
                     "algorithmic_gbs": round(dom_bytes / (dom_ms * 1e-3) / 1e9, 1)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
