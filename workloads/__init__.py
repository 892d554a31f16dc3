"""Seeded synthetic workloads for exact attention.

This module only draws inputs; it holds none of the attention arithmetic, so
the oracle and the HIP path can both be fed from it without sharing any
method code.  Inputs are drawn on the CPU with a seeded torch generator,
full-shape fp32 ``randn`` for Q, K, V (then dO) in that order, multiplied by
the workload's amplitude and rounded to the compute dtype with
round-to-nearest-even.  The same rounded values go to the GPU and, upcast to
float64, to the oracle.

Workloads (shapes and seeds of the exact-attention study: a 4096-token
sequence whose single-head score matrix has 16,777,216 entries, scaled to 32
heads; a 32768-token long-context case; a short-sequence batch; a small fp32
case; a backward case; and a decode case, one query row per sequence
against a long key cache):
"""

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str            # "f32" or "bf16": input (and default output) dtype
    causal: tuple         # the mask settings this workload is run with
    seed: int
    scale: float
    amp: float = 1.0      # inputs are amp * N(0, 1)
    backward: bool = False
    sample_rows: int = 0  # >0: the oracle checks this many rows per head
    notes: str = field(default="", compare=False)

    @property
    def shape_q(self):
        return (self.B, self.H, self.Lq, self.d)

    @property
    def shape_kv(self):
        return (self.B, self.H, self.Lk, self.d)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_f32_B1H1L128d64", 1, 1, 128, 128, 64, "f32", (False,), 0,
                 1.0 / math.sqrt(64)),
        Workload("fwd_bf16_B4H16L1024d64", 4, 16, 1024, 1024, 64, "bf16",
                 (False, True), 1, 1.0 / 8.0),
        Workload("fwd_bf16_causal_B1H32L4096d128", 1, 32, 4096, 4096, 128, "bf16",
                 (True,), 2, 1.0 / math.sqrt(128), amp=0.5),
        Workload("fwd_bf16_causal_B1H8L32768d128", 1, 8, 32768, 32768, 128, "bf16",
                 (True,), 3, 1.0 / math.sqrt(128), sample_rows=256),
        Workload("bwd_bf16_causal_B2H16L2048d128", 2, 16, 2048, 2048, 128, "bf16",
                 (True,), 4, 1.0 / math.sqrt(128), backward=True),
        # Decode: one new query row per sequence against a 16384-key cache,
        # 8 sequences x 32 heads (the key-split forward's workload).
        Workload("decode_bf16_B8H32Lq1Lk16384d128", 8, 32, 1, 16384, 128, "bf16",
                 (False,), 5, 1.0 / math.sqrt(128)),
    ]
}

# The headline benchmark shape: forward + backward, causal, B1 H32 L4096 d128.
BENCH_WORKLOAD = "fwd_bf16_causal_B1H32L4096d128"
# The key-split forward's shape, measured beside it.
DECODE_WORKLOAD = "decode_bf16_B8H32Lq1Lk16384d128"

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(B, H, Lq, Lk, d, dtype="bf16", seed=0, amp=1.0, with_dO=False):
    """Draw Q, K, V (and dO) on the CPU: amp * N(0,1), rounded to ``dtype``.

    Returns a tuple of CPU tensors in ``dtype``; Q is [B,H,Lq,d], K and V are
    [B,H,Lk,d], dO (if asked) is [B,H,Lq,d].
    """
    g = torch.Generator().manual_seed(seed)
    tdt = TORCH_DTYPES[dtype]
    out = []
    for shape in [(B, H, Lq, d), (B, H, Lk, d), (B, H, Lk, d)] + (
            [(B, H, Lq, d)] if with_dO else []):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if amp != 1.0:
            x = x * amp
        out.append(x.to(tdt))
    return tuple(out)


def workload_inputs(w, with_dO=None):
    """Inputs of a named workload (``w`` is a Workload or its name)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if with_dO is None:
        with_dO = w.backward
    return make_inputs(w.B, w.H, w.Lq, w.Lk, w.d, w.dtype, w.seed, w.amp, with_dO)


def sample_rows(H, L, n, seed, B=1):
    """Seeded query-row sample, [B, H, n] int64, drawn head by head.

    One generator seeded with ``seed`` draws ``randperm(L)`` for each
    (batch, head) in order.  The sample is rows 0 and L-1 (the first row and
    the row that sees every key) followed by the first n-2 permuted rows that
    are neither, so the n rows are distinct.
    """
    if not 2 <= n <= L:
        raise ValueError("need 2 <= n <= L")
    g = torch.Generator().manual_seed(seed)
    rows = torch.empty((B, H, n), dtype=torch.int64)
    for b in range(B):
        for h in range(H):
            perm = torch.randperm(L, generator=g)
            rest = perm[(perm != 0) & (perm != L - 1)][: n - 2]
            rows[b, h, 0] = 0
            rows[b, h, 1] = L - 1
            rows[b, h, 2:] = rest
    return rows


def window_block_mask(n_blocks, window=4, first=True):
    """Block mask [n_blocks, n_blocks] (uint8 CPU tensor): row block i keeps
    key blocks i-window+1 .. i (a sliding window) and, with ``first``, key
    block 0 -- a local window plus the leading tokens.  An input of the
    block-sparse forward; no attention arithmetic."""
    i = torch.arange(n_blocks)
    keep = (i[:, None] - i[None, :] < window) & (i[None, :] <= i[:, None])
    if first:
        keep |= (i[None, :] == 0)
    return keep.to(torch.uint8)


def to_f64(x):
    """CPU float64 numpy copy of a tensor (any dtype, any device)."""
    return x.detach().to("cpu", torch.float64).numpy()
