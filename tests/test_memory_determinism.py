"""Device-memory footprint and run-to-run determinism of the HIP path.
Needs an MI355X.

Memory: the glossary page "Flash Attention" (section "Worked example")
sizes one head's 4096 x 4096 score matrix at 16,777,216 entries, 32 MiB at
two bytes each, growing 4x when the length doubles.  The library allocates
nothing: the forward's peak allocation is exactly its caller-provided
outputs, and the backward's extra memory is the workspace, linear in L.
"""

import json
import os

import pytest
import torch

import exact_io_aware_13_amd as fa
from tests.gpu_util import announce, to_dev
from workloads import make_inputs

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_forward_allocates_nothing_beyond_outputs():
    mem = json.load(open(os.path.join(GOLDEN, "worked_example_memory.json")))
    L, H, d = mem["L"], 32, 128
    q, k, v = to_dev(*make_inputs(1, H, L, L, d, "bf16", seed=2))
    out = torch.empty_like(q)
    lse = torch.empty((1, H, L), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    announce("memory: forward")
    fa.fa_fwd(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base
    # The naive path would need one score matrix per head: 32 MiB each here.
    assert mem["bytes"] == L * L * mem["bytes_per_element"] == 32 * 2 ** 20


def test_backward_workspace_is_linear_and_small():
    mem = json.load(open(os.path.join(GOLDEN, "worked_example_memory.json")))
    sizes = {}
    for L in (mem["L"], mem["L_doubled"]):
        H, d = 4, 128
        q, k, v, do = to_dev(*make_inputs(1, H, L, L, d, "bf16", seed=3, with_dO=True))
        O, lse = fa.fa_fwd(q, k, v, causal=True)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(torch.bfloat16, 1, H, L, L, d),
                         dtype=torch.uint8, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        announce(f"memory: backward L={L}")
        fa.fa_bwd(q, k, v, O, do, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated() == base
        sizes[L] = ws.numel()
        # Workspace per head is far below that head's score matrix.
        assert ws.numel() / H < mem["bytes"] * (L / mem["L"]) ** 2 / 10
    assert sizes[mem["L_doubled"]] == 2 * sizes[mem["L"]]


def test_forward_is_bitwise_deterministic():
    q, k, v = to_dev(*make_inputs(2, 8, 1500, 1500, 128, "bf16", seed=8))
    announce("determinism: forward")
    runs = [fa.fa_fwd(q, k, v, causal=c) for c in (True, True, False, False)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    assert torch.equal(runs[2][0], runs[3][0]) and torch.equal(runs[2][1], runs[3][1])


def test_backward_is_bitwise_deterministic():
    # Every gradient row is owned by one workgroup and summed in a fixed
    # order (no atomics), so repeated calls agree bit for bit, with and
    # without the causal mask and with a ragged length.
    q, k, v, do = to_dev(*make_inputs(1, 8, 2000, 2000, 128, "bf16", seed=6, with_dO=True))
    announce("determinism: backward")
    for causal in (True, False):
        O, lse = fa.fa_fwd(q, k, v, causal=causal)
        g1 = fa.fa_bwd(q, k, v, O, do, lse, causal=causal)
        g2 = fa.fa_bwd(q, k, v, O, do, lse, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)
