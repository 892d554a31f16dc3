"""Exact blockwise scaled-dot-product attention for AMD Instinct MI355X.

The computation lives in libfa.so (hand-written HIP kernels for gfx950
behind the C ABI declared in include/fa.h).  This package loads it and
exposes the same calls on torch tensors:

    fa_fwd(q, k, v, scale, causal)            -> (O, lse)
    fa_fwd_blocksparse(q, k, v, block_mask, scale, causal) -> (O, lse),
                                                 128x128 blocks removed
    fa_bwd(q, k, v, o, do, lse, scale, causal) -> (dQ, dK, dV)
    fa_bwd_prepare / fa_bwd_dkdv / fa_bwd_dq     (the backward's stages)
    fa_bwd_prepare_dq                           (stages 1 and 3 in one kernel)
    fa_bwd_blocksparse(q, k, v, o, do, lse, block_mask, ...) -> (dQ, dK, dV)
    fa_bwd_workspace_bytes(dtype, B, H, Lq, Lk, d)
    fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, ...)  fa_bwd with the
                                                 statistics in a fixed per-GPU
                                                 array (no allocation)
    fa_fwd_splitkv(q, k, v, scale, causal, nsplit)  -> (O, lse), keys split
                                                       in ranges (decode shape)
    fa_fwd_splitkv_partial / fa_fwd_splitkv_merge     (its stages)
    attention(q, k, v, causal=False, scale=None)   (autograd)
"""

from .binding import (FlashAttentionFn, attention, fa_bwd, fa_bwd_blocksparse, fa_bwd_dkdv,
                      fa_bwd_dq, fa_bwd_noalloc, fa_bwd_prepare_dq, fa_bwd_noalloc_max_scratch_bytes,
                      fa_bwd_prepare, fa_bwd_workspace_bytes, fa_fwd, fa_fwd_blocksparse,
                      fa_fwd_splitkv, SPARSE_BLOCK,
                      fa_fwd_splitkv_default_splits, fa_fwd_splitkv_merge,
                      fa_fwd_splitkv_partial, fa_fwd_splitkv_workspace_bytes)
from ._lib import FaError, LIB_PATH, load as load_library

__all__ = ["attention", "fa_fwd", "fa_fwd_blocksparse", "SPARSE_BLOCK", "fa_bwd",
           "fa_bwd_blocksparse", "fa_bwd_prepare", "fa_bwd_dkdv", "fa_bwd_dq",
           "fa_bwd_prepare_dq", "fa_bwd_noalloc", "fa_bwd_noalloc_max_scratch_bytes",
           "fa_bwd_workspace_bytes", "fa_fwd_splitkv", "fa_fwd_splitkv_partial",
           "fa_fwd_splitkv_merge", "fa_fwd_splitkv_workspace_bytes",
           "fa_fwd_splitkv_default_splits", "FlashAttentionFn",
           "FaError", "LIB_PATH", "load_library"]
