"""Benchmark: exact attention forward + backward on one MI355X.

One step is one pass of the whole hot path over one batch through the C ABI:
fa_fwd (O, lse), then the backward in its two kernels, fa_bwd_prepare_dq (the
per-row statistics D and base-2 lse, and dQ, in one kernel) and fa_bwd_dkdv
-- together exactly fa_bwd -- at B1 H32 L4096 d128, causal, bf16 inputs with
fp32 accumulation.  Inputs, outputs and
the workspace are resident in device memory before timing starts.

Throughput uses the algorithmic FLOP count: forward 4*B*H*Lq*Lk*d, halved for
the causal mask, backward 2.5x the forward (five matrix products).  The dQ
kernel recomputes S and dP, which the count does not credit.

The timed region is K steps with an event only at each end.  Every kernel
is then timed in a second pass of the same K steps with HIP events recorded
before and after each kernel on the stream the library launches on (torch's
current stream, passed to every call); events between kernels slow the step
by ~3 %, so they stay out of the region that gives "value".  The line carries
the roofline position of the kernel with the largest measured time: its
algorithmic FLOPs per launch over its average duration, against the bf16
matrix-core peak, and -- when a counter summary for the current kernel source
exists under profiles/ -- the HBM bytes measured by rocprofv3.  The fp64 CPU
oracle is timed on a bounded sample of the same workload.

After the timed steps, the key-split forward (fa_fwd_splitkv) is measured on
the decode workload (B8 H32, one query row, 16384 keys, d128) and reported
under "decode" with its HBM roofline, and the block-sparse forward
and its backward (fa_fwd_blocksparse / fa_bwd_blocksparse, same shape as the
main step, causal, sliding window of four 128-key blocks plus the first
block) under "blocksparse"; neither is part of "value".

Every other workload of the study is measured too, under "workloads": the
fp32 forward at B1 H1 L128 d64, the bf16 forward at B4 H16 L1024 d64 without
and with the causal mask, the forward and the backward at the headline shape,
the long-context forward at B1 H8 L32768 d128 and the backward at B2 H16
L2048 d128.  Each is captured R calls at a time in a HIP graph (so host-side
launch cost does not enter the time of the small ones) and replayed 5 times;
the median per-call time gives TFLOP/s, the fraction of the matrix-core (or,
for fp32, vector) peak, and algorithmic HBM GB/s against 8 TB/s.  The fp64
oracle is timed beside each on the host: all cores, and one core for the
small shapes; the long-context oracle computes 256 sampled rows per head and
says so.  The shader clock is measured by a one-wave probe kernel
(libfa_clock.so) that reads the shader cycle counter against the 100 MHz
real-time counter, alone and beside each of the step's main kernels.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                       [--no-workloads]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import exact_io_aware_13_amd as fa  # noqa: E402
from workloads import BENCH_WORKLOAD, DECODE_WORKLOAD, WORKLOADS, make_inputs  # noqa: E402

METRIC = "attn fwd+bwd TFLOP/s & % bf16 MFMA peak, B1 H32 L4096 d128 causal"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak (published)
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector peak (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E peak (published)
MIN_WARMUP_S = 0.25           # least busy time before the timed steps
CSRC = os.path.join(ROOT, "exact_io_aware_13_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def flops(B, H, Lq, Lk, d, causal):
    fwd = 4.0 * B * H * Lq * Lk * d * (0.5 if causal else 1.0)
    return fwd, 2.5 * fwd


def kernel_table(B, H, L, d):
    """Per kernel: source file, algorithmic FLOPs and HBM bytes per launch.

    One matrix product over the visible (query, key) pairs is f1 = fwd / 2.
    The forward does 2 (S, PV); dK/dV does 4 of the backward's 5 (S, dP, dV,
    dK); dQ does 1 algorithmic product (dQ) plus S and dP again, and also
    forms the row statistics (reading O and lse, writing D and base-2 lse).
    Bytes: every tensor the kernel must touch, read or written once.
    """
    f_fwd, _ = flops(B, H, L, L, d, True)
    f1 = f_fwd / 2
    t = B * H * L * d * 2          # one [B,H,L,d] bf16 tensor
    r = B * H * L * 4              # one [B,H,L] fp32 row vector
    return {
        "fwd_bf16_kernel": dict(src="fa_fwd_bf16.hip", flops=2 * f1, executed=2 * f1,
                                bytes=3 * t + t + r),
        "bwd_dkdv_kernel": dict(src="fa_bwd_bf16.hip", flops=4 * f1, executed=4 * f1,
                                bytes=4 * t + 2 * r + 2 * t),
        "bwd_dq_kernel": dict(src="fa_bwd_bf16.hip", flops=1 * f1, executed=3 * f1,
                              bytes=5 * t + r + 2 * r + t),
    }


def source_hash(name):
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()


def measured_traffic(kernel, src, workload="B1H32L4096d128_causal"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_hash(src):
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(w, seconds_target=15.0):
    """The fp64 oracle (forward + backward) on whole heads of the workload."""
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


def decode_bytes(w):
    """Algorithmic HBM bytes of one decode forward: Q, K, V read once, O and
    lse written once."""
    t_q = w.B * w.H * w.Lq * w.d * 2
    t_kv = w.B * w.H * w.Lk * w.d * 2
    return 2 * t_q + 2 * t_kv + w.B * w.H * w.Lq * 4


def decode_cpu_baseline(w, seconds_target=3.0):
    """The fp64 oracle on whole (batch, head) slices of the decode workload."""
    import oracle
    from workloads import to_f64
    q, k, v = make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed)
    q, k, v = (to_f64(t) for t in (q, k, v))
    n, t0 = 0, time.perf_counter()
    while True:
        b, h = divmod(n, w.H)
        oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], w.scale,
                        False)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds_target or n >= w.B * w.H:
            break
    per_slice = decode_bytes(w) / (w.B * w.H)
    return {"value": round(n * per_slice / el / 1e9, 3), "unit": "GB/s", "kind": "oracle",
            "sample": f"{n} of {w.B * w.H} slices (fp64 numpy), {el:.1f} s wall"}


def bench_decode(steps, warmup, with_cpu):
    """The key-split forward on the decode workload: per-kernel HIP-event
    times on the launching stream, HBM roofline of the whole call."""
    w = WORKLOADS[DECODE_WORKLOAD]
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed))
    O = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=dev)
    nsplit = fa.fa_fwd_splitkv_default_splits(w.B, w.H, w.Lq, w.Lk, w.d)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(torch.bfloat16, w.B, w.H, w.Lq, w.Lk, w.d,
                                                       nsplit), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd_splitkv_partial(q, k, v, ws, nsplit, scale=w.scale, causal=False)
        if ev is not None:
            ev[1].record()
        fa.fa_fwd_splitkv_merge(ws, w.B, w.H, w.Lq, w.d, nsplit, O, lse)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    part = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    merge = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    total = part + merge
    nbytes = decode_bytes(w)
    ws_bytes = nsplit * w.B * w.H * w.Lq * (w.d + 1) * 4
    achieved = nbytes / (total * 1e-3) / 1e9
    out = {
        "workload": f"decode forward B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} d{w.d} non-causal, bf16",
        "call": "fa_fwd_splitkv_partial + fa_fwd_splitkv_merge",
        "nsplit": nsplit, "steps": steps, "warmup": warmup,
        "us": round(total * 1e3, 2),
        "kernels": {"splitkv_partial_kernel": {"us": round(part * 1e3, 2)},
                    "splitkv_merge_kernel": {"us": round(merge * 1e3, 2)}},
        "roofline": {"kernel": "splitkv_partial_kernel + splitkv_merge_kernel", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": nbytes, "workspace_bytes_written_and_read": ws_bytes,
                     "traffic": measured_traffic("splitkv_partial_kernel", "fa_splitkv_bf16.hip",
                                                 workload="decode_B8H32Lq1Lk16384d128")},
        "cpu_baseline": decode_cpu_baseline(w) if with_cpu else None,
    }
    return out


def bench_blocksparse(steps, warmup, with_cpu):
    """Block-sparse forward on the benchmark shape (B1 H32 L4096 d128,
    causal) with a sliding window of 4 blocks plus the first block."""
    from workloads import window_block_mask
    w = WORKLOADS[BENCH_WORKLOAD]
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed,
                                              amp=w.amp))
    nb = -(-w.Lq // fa.SPARSE_BLOCK)
    bm_cpu = window_block_mask(nb)
    bm = bm_cpu.to(dev)
    O = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=dev)
    rows = torch.arange(w.Lq) // fa.SPARSE_BLOCK
    vis = bm_cpu.bool()[rows[:, None], rows[None, :]] & torch.ones(w.Lq, w.Lk, dtype=torch.bool).tril()
    pairs = int(vis.sum()) * w.B * w.H
    flops_alg = 4.0 * w.d * pairs
    do = make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16", seed=w.seed, amp=w.amp,
                     with_dO=True)[3].to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(torch.bfloat16, w.B, w.H, w.Lq, w.Lk, w.d),
                     dtype=torch.uint8, device=dev)
    fwd = lambda: fa.fa_fwd_blocksparse(q, k, v, bm, scale=w.scale, causal=True, out=O, lse=lse)
    bwd = lambda: fa.fa_bwd_blocksparse(q, k, v, O, do, lse, bm, scale=w.scale, causal=True,
                                        dq=dq, dk=dk, dv=dv, workspace=ws)
    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fwd()
        ev[i][1].record()
        bwd()
        ev[i][2].record()
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    ms_b = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    achieved = flops_alg / (ms * 1e-3) / 1e12
    out = {
        "workload": f"block-sparse forward B{w.B} H{w.H} L{w.Lq} d{w.d} causal, 128x128 blocks: "
                    "window of 4 blocks + first block",
        "visible_pairs": pairs, "dense_causal_pairs": w.B * w.H * w.Lq * (w.Lq + 1) // 2,
        "us": round(ms * 1e3, 2),
        "bwd_us": round(ms_b * 1e3, 2),
        "bwd_tflops_visible_pairs": round(2.5 * flops_alg / (ms_b * 1e-3) / 1e12, 2),
        "roofline": {"kernel": "fwd_bf16_kernel (block-sparse)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "algorithmic_flops": flops_alg, "traffic": None},
        "cpu_baseline": None,
    }
    if with_cpu:
        import oracle
        from workloads import to_f64
        qh, kh, vh = (to_f64(t[:, :1]) for t in make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, "bf16",
                                                             seed=w.seed, amp=w.amp))
        t0 = time.perf_counter()
        oracle.attn_fwd_blocksparse(qh, kh, vh, w.scale, True, bm_cpu.numpy(),
                                    block=fa.SPARSE_BLOCK)
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(flops_alg / w.H / el / 1e12, 5), "unit": "TFLOP/s",
                               "kind": "oracle",
                               "sample": f"1 of {w.H} heads (fp64 numpy, full masked S), {el:.1f} s"}
    return out


# ---- every workload of the study, one method -------------------------------

GRAPH_REPEATS = 5


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the affinity set
        return len(os.sched_getaffinity(0))


def graph_time_us(call, est_us):
    """Median per-call GPU time of ``call``: R calls captured in one HIP
    graph, the graph replayed GRAPH_REPEATS times with HIP events around each
    replay on the current stream (the stream the calls launch on).  Returns
    (median_us, [per-call us of each replay], R)."""
    R = int(min(200, max(4, 20000.0 / max(est_us, 1.0))))   # ~20 ms per replay
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(R):
            call()
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(GRAPH_REPEATS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / R)
    del g
    return sorted(per)[len(per) // 2], [round(x, 3) for x in per], R


def oracle_time_us(fn, one_core, min_runs=1, budget_s=10.0):
    """Wall time of the oracle call ``fn``: one warm-up, then runs until
    ``budget_s`` has passed (at least ``min_runs``); the median in us."""
    from threadpoolctl import threadpool_limits
    ctx = threadpool_limits(1) if one_core else None
    try:
        if ctx is not None:
            ctx.__enter__()
        fn()
        ts, t0 = [], time.perf_counter()
        while len(ts) < min_runs or (time.perf_counter() - t0 < budget_s and len(ts) < 200):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return sorted(ts)[len(ts) // 2] * 1e6, len(ts)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def fwd_bytes(B, H, Lq, Lk, d, esz, o_esz):
    """Algorithmic HBM bytes of one forward: Q, K, V read, O and lse written."""
    return B * H * ((Lq + 2 * Lk) * d * esz + Lq * d * o_esz + Lq * 4)


def bwd_bytes(B, H, Lq, Lk, d, esz):
    """Algorithmic HBM bytes of one backward: Q, K, V, O, dO and lse read,
    dQ, dK, dV written."""
    return B * H * ((3 * Lq + 4 * Lk) * d * esz + Lq * 4 + Lq * d * esz)


def _entry(name, call, what, us, reps, R, fl, nbytes, peak_tflops, peak_name):
    tf = fl / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    ai = fl / nbytes
    ridge = peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9)
    return {
        "workload": what, "call": call, "us": round(us, 3), "us_per_replay": reps,
        "calls_per_graph": R, "replays": GRAPH_REPEATS, "stat": "median",
        "algorithmic_flops": fl, "algorithmic_bytes": nbytes,
        "tflops": round(tf, 2), "peak_tflops": peak_tflops, "peak": peak_name,
        "frac_of_peak": round(tf / peak_tflops, 4),
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "flop_per_byte": round(ai, 1), "ridge_flop_per_byte": round(ridge, 1),
        "bound": "mfma" if (ai > ridge and peak_name.startswith("bf16")) else
                 ("valu" if ai > ridge else "hbm"),
    }


def bench_workloads(with_cpu):
    """Every workload of the study through the C ABI (see the module notes)."""
    import oracle
    from workloads import sample_rows, to_f64, workload_inputs
    dev = torch.device("cuda", 0)
    out = {}
    threads = _blas_threads()

    def forward_case(wname, causal, label, est_us, one_core, rows=None):
        w = WORKLOADS[wname]
        q, k, v = workload_inputs(w, with_dO=False)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        O = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=dev)
        call = lambda: fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=causal, out=O, lse=lse)
        us, reps, R = graph_time_us(call, est_us)
        fl, _ = flops(w.B, w.H, w.Lq, w.Lk, w.d, causal)
        esz = 4 if w.dtype == "f32" else 2
        e = _entry(label, "fa_fwd", f"forward {w.dtype} B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} d{w.d} "
                   f"{'causal' if causal else 'non-causal'}", us, reps, R, fl,
                   fwd_bytes(w.B, w.H, w.Lq, w.Lk, w.d, esz, esz),
                   PEAK_F32_VALU_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS,
                   "fp32 vector" if w.dtype == "f32" else "bf16 dense matrix core")
        if with_cpu:
            qf, kf, vf = (to_f64(t) for t in (q, k, v))
            if rows is None:
                fn = lambda: oracle.attn_fwd(qf, kf, vf, w.scale, causal)
                us_all, n_all = oracle_time_us(fn, False, budget_s=3.0)
                cb = {"kind": "oracle", "all_cores": {"us": round(us_all, 1), "cores": threads,
                                                      "runs": n_all},
                      "sample": "the whole workload (fp64 numpy, full S per slice), median of runs"}
                if one_core:
                    us_1, n_1 = oracle_time_us(fn, True, budget_s=3.0)
                    cb["one_core"] = {"us": round(us_1, 1), "cores": 1, "runs": n_1}
                cb["gpu_speedup_vs_all_cores"] = round(us_all / us, 1)
            else:
                ridx = sample_rows(w.H, w.Lq, rows, w.seed, B=w.B).numpy()
                fn = lambda: oracle.attn_fwd_rows(qf, kf, vf, w.scale, causal, ridx)
                us_s, n_s = oracle_time_us(fn, False, budget_s=0.0)
                pairs = sum(int(r) + 1 if causal else w.Lk for r in ridx.ravel())
                fl_s = 4.0 * w.d * pairs
                cb = {"kind": "oracle", "all_cores": {"us": round(us_s, 1), "cores": threads,
                                                      "runs": n_s},
                      "sample": f"{rows} seeded query rows per head, every head (fp64 numpy, "
                                f"full rows over the visible keys): {fl_s:.3e} of {fl:.3e} FLOP",
                      "tflops_on_sample": round(fl_s / (us_s * 1e-6) / 1e12, 5)}
            e["cpu_baseline"] = cb
        out[label] = e

    def backward_case(wname, label, est_us, heads_budget_s):
        w = WORKLOADS[wname]
        q, k, v, do = workload_inputs(w, with_dO=True)
        qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
        O, lse = fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=True)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(qd.dtype, w.B, w.H, w.Lq, w.Lk, w.d),
                         dtype=torch.uint8, device=dev)
        call = lambda: fa.fa_bwd(qd, kd, vd, O, dod, lse, scale=w.scale, causal=True, dq=dq, dk=dk,
                                 dv=dv, workspace=ws)
        us, reps, R = graph_time_us(call, est_us)
        _, fl = flops(w.B, w.H, w.Lq, w.Lk, w.d, True)
        e = _entry(label, "fa_bwd", f"backward bf16 B{w.B} H{w.H} L{w.Lq} d{w.d} causal "
                   "(D statistic, dK/dV, dQ)", us, reps, R, fl,
                   bwd_bytes(w.B, w.H, w.Lq, w.Lk, w.d, 2), PEAK_BF16_TFLOPS,
                   "bf16 dense matrix core")
        if with_cpu:
            qf, kf, vf, dof = (to_f64(t) for t in (q, k, v, do))
            n, t0 = 0, time.perf_counter()
            while n < w.B * w.H:
                b, h = divmod(n, w.H)
                oracle.attn_bwd(qf[b:b + 1, h:h + 1], kf[b:b + 1, h:h + 1], vf[b:b + 1, h:h + 1],
                                dof[b:b + 1, h:h + 1], w.scale, True)
                n += 1
                if time.perf_counter() - t0 >= heads_budget_s:
                    break
            el = time.perf_counter() - t0
            per_slice_us = el / n * 1e6
            e["cpu_baseline"] = {
                "kind": "oracle", "all_cores": {"us": round(per_slice_us * w.B * w.H, 1),
                                                "cores": threads, "runs": 1},
                "sample": f"{n} of {w.B * w.H} slices timed (backward, which recomputes the "
                          f"forward; fp64 numpy, full S), {el:.1f} s wall, scaled to all slices",
                "tflops": round(fl / w.B / w.H * n / el / 1e12, 5)}
        out[label] = e

    forward_case("fwd_f32_B1H1L128d64", False, "fwd_f32_B1H1L128d64", 10.0, True)
    forward_case("fwd_bf16_B4H16L1024d64", False, "fwd_bf16_B4H16L1024d64_noncausal", 25.0, True)
    forward_case("fwd_bf16_B4H16L1024d64", True, "fwd_bf16_B4H16L1024d64_causal", 15.0, True)
    forward_case(BENCH_WORKLOAD, True, "fwd_bf16_B1H32L4096d128_causal", 130.0, False, rows=256)
    forward_case("fwd_bf16_causal_B1H8L32768d128", True, "fwd_bf16_B1H8L32768d128_causal",
                 2000.0, False, rows=256)
    backward_case(BENCH_WORKLOAD, "bwd_bf16_B1H32L4096d128_causal", 450.0, 8.0)
    backward_case("bwd_bf16_causal_B2H16L2048d128", "bwd_bf16_B2H16L2048d128_causal", 150.0, 8.0)
    return out


def measure_clock(kernels):
    """Shader clock from the probe library (libfa_clock.so): one wave spins
    for N shader-clock cycles and reads the shader cycle counter and the
    100 MHz real-time counter at its start and end.  Measured alone, and on a
    second stream while each of ``kernels`` (name -> call) runs back to back
    from a captured graph on the current stream (the spin wave then shares
    the chip with that kernel and sees its clock)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_13_amd", "libfa_clock.so"))
    lib.fa_clock_spin.restype = ctypes.c_int
    lib.fa_clock_spin.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    buf = torch.zeros(4, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream()

    def spin(cycles):
        with torch.cuda.stream(side):
            if lib.fa_clock_spin(buf.data_ptr(), cycles, side.cuda_stream) != 0:
                raise RuntimeError("clock probe launch failed")

    def ghz():
        torch.cuda.synchronize()
        t0, r0, t1, r1 = buf.tolist()
        return (t1 - t0) / ((r1 - r0) / 100e6) / 1e9

    spin(20_000_000)
    out = {"idle_ghz": round(ghz(), 3)}
    for name, call in kernels.items():
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            call()
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(40):
                call()
        torch.cuda.synchronize()
        vals = []
        for _ in range(3):
            g.replay()                 # the chip is busy before the spin starts
            spin(8_000_000)
            for _ in range(3):
                g.replay()
            vals.append(ghz())
        out[name + "_ghz"] = round(sorted(vals)[1], 3)
        del g
    out["method"] = ("in-kernel shader cycle counter against the 100 MHz real-time counter, "
                     "one spinning wave on a second stream; median of 3 per kernel")
    out["published_peak_clock_ghz"] = 2.4
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode and block-sparse forwards measured after the main step")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload measurements (other shapes; used when profiling "
                         "the headline step's kernels by name)")
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
    names = ["fwd_bf16_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel"]

    def step(ev=None):
        # Events go on torch's current stream, the stream every call below
        # launches its kernel on.
        calls = [
            lambda: fa.fa_fwd(q, k, v, scale=w.scale, causal=True, out=O, lse=lse),
            lambda: fa.fa_bwd_prepare_dq(q, k, v, O, do, lse, ws, scale=w.scale, causal=True,
                                         dq=dq),
            lambda: fa.fa_bwd_dkdv(q, k, v, do, ws, scale=w.scale, causal=True, dk=dk, dv=dv),
        ]
        for i, call in enumerate(calls):
            if ev is not None:
                ev[i].record()
            call()
        if ev is not None:
            ev[len(calls)].record()

    # Warmup: the W steps asked for, then more untimed steps until the GPU has
    # been busy for at least MIN_WARMUP_S, so that clocks have ramped up
    # before the timed region whatever W is.  The extra count is reported.
    t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        for _ in range(10):
            step()
        extra += 10
        torch.cuda.synchronize()
    # The timed region: K steps with events only at its two ends.  An event
    # recorded between kernels is not free (measured: 5 per step made the
    # step ~3 % slower), so the per-kernel times come from a second pass of
    # K steps with an event before and after every kernel.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    i_start = torch.cuda.Event(enable_timing=True)
    i_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    i_start.record()
    for i in range(args.steps):
        step(evs[i])
    i_end.record()
    torch.cuda.synchronize()
    ms_step_instrumented = i_start.elapsed_time(i_end) / args.steps
    kms = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i, n in enumerate(names)}

    # Five more blocks of the same K steps (untimed for value): the spread
    # of the step time, reported as a median.
    blocks = []
    for _ in range(5):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(args.steps):
            step()
        b1.record()
        torch.cuda.synchronize()
        blocks.append(b0.elapsed_time(b1) / args.steps)
    clock = measure_clock({
        "fwd_bf16_kernel": lambda: fa.fa_fwd(q, k, v, scale=w.scale, causal=True, out=O, lse=lse),
        "bwd_dkdv_kernel": lambda: fa.fa_bwd_dkdv(q, k, v, do, ws, scale=w.scale, causal=True,
                                                  dk=dk, dv=dv),
        "bwd_dq_kernel": lambda: fa.fa_bwd_prepare_dq(q, k, v, O, do, lse, ws, scale=w.scale,
                                                      causal=True, dq=dq),
    })

    f_fwd, f_bwd = flops(B, H, L, L, d, True)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    table = kernel_table(B, H, L, d)
    kernels = {}
    for n in names:
        t = table[n]
        s = kms[n] * 1e-3
        kernels[n] = {"ms": round(kms[n], 4),
                      "algorithmic_tflops": round(t["flops"] / s / 1e12, 2),
                      "executed_tflops": round(t["executed"] / s / 1e12, 2),
                      "algorithmic_gbs": round(t["bytes"] / s / 1e9, 1)}
    dom = max(names, key=lambda n: kms[n])
    t = table[dom]
    achieved = t["flops"] / (kms[dom] * 1e-3) / 1e12
    traffic = measured_traffic(dom, t["src"])
    fwd_ms = kms["fwd_bf16_kernel"]
    bwd_ms = sum(kms[n] for n in names[1:])
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_extra_steps": extra,
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
        "kernels": kernels,
        "kernel_timing": {"pass": "a second pass of the same K steps with an event before and after "
                                  "every kernel, on the stream the kernels run on",
                          "ms_per_step": round(ms_step_instrumented, 4)},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_bytes": t["bytes"]},
        "cpu_baseline": None,
        "repeats": {"blocks": 5, "steps_per_block": args.steps,
                    "ms_per_step": [round(x, 4) for x in blocks],
                    "median_ms_per_step": round(sorted(blocks)[2], 4),
                    "median_tflops": round((f_fwd + f_bwd) / (sorted(blocks)[2] * 1e-3) / 1e12, 2)},
        "clock": clock,
    }
    if not args.no_workloads:
        try:
            line["workloads"] = bench_workloads(not args.no_cpu_baseline)
        except Exception as e:  # noqa: BLE001  (recorded instead of losing the main line)
            line["workloads"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_decode:
        # Measured after the timed steps above; not part of value.  A failure
        # here is recorded in the line instead of losing the main measurement.
        for key, fn in (("decode", bench_decode), ("blocksparse", bench_blocksparse)):
            try:
                line[key] = fn(args.steps, max(args.warmup, 20), not args.no_cpu_baseline)
            except Exception as e:  # noqa: BLE001
                line[key] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
