"""The library's calls inside a captured HIP graph.  Needs an MI355X.

Every entry point only launches kernels on the stream it is given (no
allocation, no memset, no host synchronisation), so a caller can capture a
forward + backward step, or a key-split decode call, into a graph and
replay it.  Each replay must give bitwise the result of the same calls run
eagerly (the kernels are deterministic), also after the graph's inputs
were overwritten in place between replays, with the caller's own eager work
and synchronisations in between.
"""

import math

import pytest
import torch

import exact_io_aware_13_amd as fa
from tests.gpu_util import announce, to_dev
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm up on a side stream (as torch asks before capture), then capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_forward_backward_step_replays_bitwise():
    B, H, L, d = 1, 4, 1000, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = to_dev(*make_inputs(B, H, L, L, d, "bf16", seed=61, with_dO=True))
    O = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(q.dtype, B, H, L, L, d), dtype=torch.uint8,
                     device=q.device)

    def step():
        fa.fa_fwd(q, k, v, scale=scale, causal=True, out=O, lse=lse)
        fa.fa_bwd(q, k, v, O, do, lse, scale=scale, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)

    def eager(qq, kk, vv, dd):
        O2, lse2 = fa.fa_fwd(qq, kk, vv, scale=scale, causal=True)
        g2 = fa.fa_bwd(qq, kk, vv, O2, dd, lse2, scale=scale, causal=True)
        return (O2, lse2) + tuple(g2)

    announce("graph capture: fwd + bwd B1 H4 L1000 d128 causal")
    g = _capture(step)
    inputs = [(q.clone(), k.clone(), v.clone(), do.clone())]
    for seed in (62, 63):
        inputs.append(to_dev(*make_inputs(B, H, L, L, d, "bf16", seed=seed, with_dO=True)))
    for rep, (qn, kn, vn, dn) in enumerate(inputs):
        q.copy_(qn), k.copy_(kn), v.copy_(vn), do.copy_(dn)
        for t in (O, lse, dq, dk, dv):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager(qn, kn, vn, dn)
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "lse", "dQ", "dK", "dV"), (O, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"


def test_splitkv_decode_replays_bitwise():
    B, H, Lq, Lk, d = 2, 8, 1, 5000, 128
    q, k, v = to_dev(*make_inputs(B, H, Lq, Lk, d, "bf16", seed=64))
    nsplit = 24
    O = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(q.dtype, B, H, Lq, Lk, d, nsplit),
                     dtype=torch.uint8, device=q.device)

    def call():
        fa.fa_fwd_splitkv(q, k, v, nsplit=nsplit, out=O, lse=lse, workspace=ws)

    announce("graph capture: split-KV B2 H8 Lq1 Lk5000 d128")
    g = _capture(call)
    for rep, seed in enumerate((64, 65, 66)):
        qn, kn, vn = to_dev(*make_inputs(B, H, Lq, Lk, d, "bf16", seed=seed))
        q.copy_(qn), k.copy_(kn), v.copy_(vn)
        O.zero_(), lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        O_e, lse_e = fa.fa_fwd_splitkv(qn, kn, vn, nsplit=nsplit)
        torch.cuda.synchronize()
        assert torch.equal(O, O_e), f"replay {rep}: O differs from the eager call"
        assert torch.equal(lse, lse_e), f"replay {rep}: lse differs from the eager call"
