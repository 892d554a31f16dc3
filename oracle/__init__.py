"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  This package is the correctness reference that the
GPU kernels are checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path (the HIP
library and its Python binding) never calls it and shares no code with it.

Every function here is written from the method's plain definition as stated on
the source pages ("FlashAttention: Fast and Memory-Efficient Exact Attention
with IO-Awareness" as summarised on the glossary, blog and annotated-code
pages):

* "How Flash Attention Improves Transformer Memory Efficiency ...", section
  "Why Standard Attention Consumes Quadratic Memory": the score matrix S of
  shape B x H x L_q x L_k and the post-softmax matrix P that weights V.
* "What Is FlashAttention? ...", section "The problem it solves": build the
  score matrix, apply softmax row-wise, multiply by the values.
* The annotated-code page, section "The Three Running Statistics":
  results over separate key ranges combine exactly through their softmax
  normalisers (``splitkv``: one key range, and the merge).
* Glossary page, FAQ on block-sparse extensions: a block mask removes whole
  (query block, key block) rectangles; what remains is the same definition
  under that mask (``blocksparse``).
* The annotated-code page, section "Backward Pass Efficiency": the
  backward keeps per-row statistics (D_i and the softmax normaliser) instead
  of the matrices.  The gradient formulas themselves are the chain rule
  through the forward definition (the pages do not print them).

Pins: every function is checked by tests under ``-m "not gpu"`` against
closed forms, special cases, invariants, finite differences and PyTorch's own
CPU fp64 attention; none is "parity unpinned".
"""

from .attention import (
    visible_mask,
    attn_fwd,
    attn_fwd_rows,
    attn_bwd,
    attn_bwd_heads,
)
from .splitkv import attn_fwd_keyrange, merge_partials
from .blocksparse import attn_bwd_blocksparse, attn_fwd_blocksparse, block_visible

__all__ = [
    "visible_mask",
    "attn_fwd",
    "attn_fwd_rows",
    "attn_bwd",
    "attn_bwd_heads",
    "attn_fwd_keyrange",
    "merge_partials",
    "attn_fwd_blocksparse",
    "attn_bwd_blocksparse",
    "block_visible",
]
