"""Python binding of libfa with the C ABI's names.

``fa_fwd``, ``fa_fwd_blocksparse``, ``fa_bwd`` (and its stages ``fa_bwd_prepare``, ``fa_bwd_dkdv``,
``fa_bwd_dq``, ``fa_bwd_prepare_dq``), ``fa_bwd_workspace_bytes`` and the key-split forward
(``fa_fwd_splitkv`` and its stages) only marshal torch tensors
(device pointers, sizes, the current HIP stream) into the C calls;
all arithmetic runs in the library's HIP kernels.  PyTorch supplies device
memory and streams.  ``attention`` wraps both calls in an autograd Function
with the signature of the annotated-code page's usage example,
``(q, k, v, causal, scale)`` on [B, H, L, d] tensors, where an omitted scale
is 1/sqrt(d) ("How Flash Attention Improves Transformer Memory Efficiency
...", section "Basic Flash Attention Forward Pass").
"""

import math

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FA_F32, torch.bfloat16: _lib.FA_BF16}


def _code(dtype):
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}; libfa takes float32 or bfloat16") from None


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _check_tensor(name, t, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous ([B,H,L,d] row-major)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def fa_fwd(q, k, v, scale=None, causal=False, out_dtype=None, out=None, lse=None):
    """O, lse = attention(q, k, v) through libfa's ``fa_fwd``.

    q [B,H,Lq,d], k and v [B,H,Lk,d]: contiguous, on one GPU, float32 or
    bfloat16.  ``out_dtype`` defaults to the input dtype (float32 is allowed
    for bfloat16 inputs).  Returns (O [B,H,Lq,d], lse [B,H,Lq] float32).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    _check_tensor("k", k, dev, q.dtype, (B, H, Lk, d))
    _check_tensor("v", v, dev, q.dtype, (B, H, Lk, d))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=out_dtype, device=dev)
    _check_tensor("out", out, dev, out_dtype, (B, H, Lq, d))
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    lib = _lib.load()
    st = lib.fa_fwd(_code(q.dtype), _code(out_dtype), B, H, Lq, Lk, d, _ptr(q), _ptr(k), _ptr(v),
                    float(scale), int(bool(causal)), _ptr(out), _ptr(lse), _stream(dev))
    _lib.check(st)
    return out, lse


SPARSE_BLOCK = 128  # query and key block edge of the block-sparse mask


def fa_fwd_blocksparse(q, k, v, block_mask, scale=None, causal=False, out_dtype=None, out=None,
                       lse=None):
    """O, lse through libfa's ``fa_fwd_blocksparse``.

    ``block_mask``: uint8 (or bool) device tensor [ceil(Lq/128), ceil(Lk/128)]
    shared by every slice, or [B, H, ceil(Lq/128), ceil(Lk/128)]; nonzero
    keeps a 128 x 128 (query, key) block.  Rows that see no key return O = 0
    and lse = -inf.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    _check_tensor("k", k, dev, q.dtype, (B, H, Lk, d))
    _check_tensor("v", v, dev, q.dtype, (B, H, Lk, d))
    nqb, nkb = -(-Lq // SPARSE_BLOCK), -(-Lk // SPARSE_BLOCK)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    if tuple(block_mask.shape) == (nqb, nkb):
        slices = 1
    elif tuple(block_mask.shape) == (B, H, nqb, nkb):
        slices = B * H
    else:
        raise ValueError(f"block_mask must be [{nqb}, {nkb}] or [{B}, {H}, {nqb}, {nkb}]")
    _check_tensor("block_mask", block_mask, dev, torch.uint8)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=out_dtype, device=dev)
    _check_tensor("out", out, dev, out_dtype, (B, H, Lq, d))
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    st = _lib.load().fa_fwd_blocksparse(_code(q.dtype), _code(out_dtype), B, H, Lq, Lk, d,
                                        _ptr(q), _ptr(k), _ptr(v), float(scale), int(bool(causal)),
                                        _ptr(block_mask), slices, _ptr(out), _ptr(lse),
                                        _stream(dev))
    _lib.check(st)
    return out, lse


def fa_bwd_workspace_bytes(dtype, B, H, Lq, Lk, d):
    """Bytes of workspace ``fa_bwd`` needs (0 for sizes it would reject)."""
    return int(_lib.load().fa_bwd_workspace_bytes(_code(dtype), B, H, Lq, Lk, d))


def fa_bwd(q, k, v, o, do, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
           workspace=None):
    """dQ, dK, dV through libfa's ``fa_bwd``.

    o and lse are the forward's outputs (o in the input dtype, or float32
    beside bfloat16 inputs: the C call's o_dtype is o's dtype), do the
    gradient of o in the input dtype.  ``workspace`` (a uint8 device tensor)
    is allocated here when not given.  Returns (dq, dk, dv) in the input
    dtype.
    """
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    for name, t, shp in (("k", k, (B, H, Lk, d)), ("v", v, (B, H, Lk, d)),
                         ("do", do, (B, H, Lq, d))):
        _check_tensor(name, t, dev, q.dtype, shp)
    _check_tensor("o", o, dev, None, (B, H, Lq, d))
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, dev, q.dtype, ref.shape)
    need = fa_bwd_workspace_bytes(q.dtype, B, H, Lq, Lk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    lib = _lib.load()
    st = lib.fa_bwd(_code(q.dtype), _code(o.dtype), B, H, Lq, Lk, d, _ptr(q), _ptr(k), _ptr(v),
                    _ptr(o), _ptr(do), _ptr(lse), float(scale), int(bool(causal)), _ptr(dq),
                    _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)
    return dq, dk, dv


def fa_bwd_noalloc_max_scratch_bytes():
    """Bytes of the fixed statistics array ``fa_bwd_noalloc`` uses per GPU."""
    return int(_lib.load().fa_bwd_noalloc_max_scratch_bytes())


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False):
    """dQ, dK, dV through libfa's ``fa_bwd_noalloc``: ``fa_bwd`` with its
    statistics in the library's fixed per-GPU array instead of a workspace.
    The outputs must be given (nothing is allocated, here or in the call);
    calls that overlap on one GPU race on that array."""
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    for name, t, shp in (("k", k, (B, H, Lk, d)), ("v", v, (B, H, Lk, d)),
                         ("do", do, (B, H, Lq, d)), ("dq", dq, (B, H, Lq, d)),
                         ("dk", dk, (B, H, Lk, d)), ("dv", dv, (B, H, Lk, d))):
        _check_tensor(name, t, dev, q.dtype, shp)
    _check_tensor("o", o, dev, None, (B, H, Lq, d))
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib.load().fa_bwd_noalloc(_code(q.dtype), _code(o.dtype), B, H, Lq, Lk, d, _ptr(q),
                                    _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), float(scale),
                                    int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _stream(dev))
    _lib.check(st)
    return dq, dk, dv


def fa_bwd_blocksparse(q, k, v, o, do, lse, block_mask, scale=None, causal=False, dq=None,
                       dk=None, dv=None, workspace=None):
    """dQ, dK, dV through libfa's ``fa_bwd_blocksparse``: the backward of
    :func:`fa_fwd_blocksparse` with the same ``block_mask``."""
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    for name, t, shp in (("k", k, (B, H, Lk, d)), ("v", v, (B, H, Lk, d)),
                         ("do", do, (B, H, Lq, d))):
        _check_tensor(name, t, dev, q.dtype, shp)
    _check_tensor("o", o, dev, None, (B, H, Lq, d))
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    nqb, nkb = -(-Lq // SPARSE_BLOCK), -(-Lk // SPARSE_BLOCK)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    if tuple(block_mask.shape) == (nqb, nkb):
        slices = 1
    elif tuple(block_mask.shape) == (B, H, nqb, nkb):
        slices = B * H
    else:
        raise ValueError(f"block_mask must be [{nqb}, {nkb}] or [{B}, {H}, {nqb}, {nkb}]")
    _check_tensor("block_mask", block_mask, dev, torch.uint8)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, dev, q.dtype, ref.shape)
    need = fa_bwd_workspace_bytes(q.dtype, B, H, Lq, Lk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_bwd_blocksparse(_code(q.dtype), _code(o.dtype), B, H, Lq, Lk, d, _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(o), _ptr(do), _ptr(lse), float(scale),
                                        int(bool(causal)), _ptr(block_mask), slices, _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                        _stream(dev))
    _lib.check(st)
    return dq, dk, dv


def _bwd_shapes(q, k, v, do):
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    for name, t, shp in (("k", k, (B, H, Lk, d)), ("v", v, (B, H, Lk, d)),
                         ("do", do, (B, H, Lq, d))):
        _check_tensor(name, t, dev, q.dtype, shp)
    return B, H, Lq, Lk, d, dev


def fa_bwd_prepare(o, do, lse, Lk, workspace):
    """Stage 1 of ``fa_bwd``: per-row statistics into ``workspace``.

    ``do`` is in the input dtype, ``o`` in that dtype or float32.  ``Lk`` is
    the key length of the later stages (it sizes the checks).
    """
    B, H, Lq, d = o.shape
    dev = o.device
    _check_tensor("o", o, dev)
    _check_tensor("do", do, dev, None, o.shape)
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_bwd_prepare(_code(do.dtype), _code(o.dtype), B, H, Lq, Lk, d, _ptr(o), _ptr(do), _ptr(lse),
                                    _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)


def fa_bwd_dkdv(q, k, v, do, workspace, scale=None, causal=False, dk=None, dv=None):
    """Stage 2 of ``fa_bwd``: dK and dV from a prepared workspace."""
    B, H, Lq, Lk, d, dev = _bwd_shapes(q, k, v, do)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dk", dk, dev, q.dtype, k.shape)
    _check_tensor("dv", dv, dev, q.dtype, v.shape)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_bwd_dkdv(_code(q.dtype), B, H, Lq, Lk, d, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(do), float(scale), int(bool(causal)), _ptr(dk), _ptr(dv),
                                 _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)
    return dk, dv


def fa_bwd_dq(q, k, v, do, workspace, scale=None, causal=False, dq=None):
    """Stage 3 of ``fa_bwd``: dQ from a prepared workspace."""
    B, H, Lq, Lk, d, dev = _bwd_shapes(q, k, v, do)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    _check_tensor("dq", dq, dev, q.dtype, q.shape)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_bwd_dq(_code(q.dtype), B, H, Lq, Lk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                               float(scale), int(bool(causal)), _ptr(dq), _ptr(workspace),
                               workspace.numel(), _stream(dev))
    _lib.check(st)
    return dq


def fa_bwd_prepare_dq(q, k, v, o, do, lse, workspace, scale=None, causal=False, dq=None):
    """Stages 1 and 3 of ``fa_bwd`` in one call (one kernel with bf16 ``o``):
    the per-row statistics into ``workspace``, and dQ.  ``fa_bwd_dkdv`` can
    follow it on the same stream."""
    B, H, Lq, Lk, d, dev = _bwd_shapes(q, k, v, do)
    _check_tensor("o", o, dev, None, (B, H, Lq, d))
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    _check_tensor("dq", dq, dev, q.dtype, q.shape)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_bwd_prepare_dq(_code(q.dtype), _code(o.dtype), B, H, Lq, Lk, d, _ptr(q),
                                       _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                       float(scale), int(bool(causal)), _ptr(dq), _ptr(workspace),
                                       workspace.numel(), _stream(dev))
    _lib.check(st)
    return dq


def fa_fwd_splitkv_default_splits(B, H, Lq, Lk, d):
    """Split count that fills the current device for these sizes."""
    return int(_lib.load().fa_fwd_splitkv_default_splits(B, H, Lq, Lk, d))


def fa_fwd_splitkv_workspace_bytes(dtype, B, H, Lq, Lk, d, nsplit):
    """Bytes of workspace the key-split forward needs (0 if it would reject)."""
    return int(_lib.load().fa_fwd_splitkv_workspace_bytes(_code(dtype), B, H, Lq, Lk, d, nsplit))


def _splitkv_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dev = q.device
    _check_tensor("q", q, dev)
    _check_tensor("k", k, dev, q.dtype, (B, H, Lk, d))
    _check_tensor("v", v, dev, q.dtype, (B, H, Lk, d))
    return B, H, Lq, Lk, d, dev


def fa_fwd_splitkv(q, k, v, scale=None, causal=False, nsplit=None, out_dtype=None, out=None,
                   lse=None, workspace=None):
    """O, lse = attention(q, k, v) through libfa's ``fa_fwd_splitkv``.

    Same operation and outputs as :func:`fa_fwd`, with the keys cut into
    ``nsplit`` ranges (default: ``fa_fwd_splitkv_default_splits``).  bfloat16
    inputs; ``workspace`` (uint8 device tensor) is allocated when not given.
    """
    B, H, Lq, Lk, d, dev = _splitkv_shapes(q, k, v)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if nsplit is None:
        nsplit = fa_fwd_splitkv_default_splits(B, H, Lq, Lk, d)
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=out_dtype, device=dev)
    _check_tensor("out", out, dev, out_dtype, (B, H, Lq, d))
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    if workspace is None:
        need = fa_fwd_splitkv_workspace_bytes(q.dtype, B, H, Lq, Lk, d, nsplit)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_fwd_splitkv(_code(q.dtype), _code(out_dtype), B, H, Lq, Lk, d, _ptr(q),
                                    _ptr(k), _ptr(v), float(scale), int(bool(causal)), int(nsplit),
                                    _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                    _stream(dev))
    _lib.check(st)
    return out, lse


def fa_fwd_splitkv_partial(q, k, v, workspace, nsplit, scale=None, causal=False):
    """Partial stage of the key-split forward: per-range results into
    ``workspace`` (layout in include/fa.h)."""
    B, H, Lq, Lk, d, dev = _splitkv_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_tensor("workspace", workspace, dev, torch.uint8)
    st = _lib.load().fa_fwd_splitkv_partial(_code(q.dtype), B, H, Lq, Lk, d, _ptr(q), _ptr(k),
                                            _ptr(v), float(scale), int(bool(causal)), int(nsplit),
                                            _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)


def fa_fwd_splitkv_merge(workspace, B, H, Lq, d, nsplit, out, lse):
    """Merge stage of the key-split forward: O and lse from the per-range
    results in ``workspace``."""
    dev = workspace.device
    _check_tensor("workspace", workspace, dev, torch.uint8)
    _check_tensor("out", out, dev, None, (B, H, Lq, d))
    _check_tensor("lse", lse, dev, torch.float32, (B, H, Lq))
    st = _lib.load().fa_fwd_splitkv_merge(_code(out.dtype), B, H, Lq, d, int(nsplit),
                                          _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                          _stream(dev))
    _lib.check(st)
    return out, lse


class FlashAttentionFn(torch.autograd.Function):
    """Autograd wrapper: forward saves O and lse, backward calls fa_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = fa_fwd(q, k, v, scale=scale, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = fa_bwd(q, k, v, o, do.contiguous(), lse, scale=ctx.scale, causal=ctx.causal)
        return dq, dk, dv, None, None


def attention(q, k, v, causal=False, scale=None):
    """Exact attention on [B, H, L, d] tensors; differentiable.

    ``scale`` defaults to 1/sqrt(d); ``causal`` hides key j from query row i
    when j > i.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return FlashAttentionFn.apply(q.contiguous(), k.contiguous(), v.contiguous(), bool(causal),
                                  float(scale))
