"""ctypes loader for libfa.so, the C-ABI attention library (include/fa.h).

The library is loaded after torch so that it binds to the HIP runtime torch
already mapped (both use the soname libamdhip64.so.7); stream handles from
torch are then valid inside libfa.  A missing or unloadable library raises:
there is no fallback path.
"""

import ctypes
import os

import torch  # noqa: F401  (maps torch's HIP runtime first)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32 = 0
FA_BF16 = 1

STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
    4: "FA_ERR_ALIGN", 5: "FA_ERR_WORKSPACE", 6: "FA_ERR_HIP", 7: "FA_ERR_ARG",
}

EXPORTS = ("fa_fwd", "fa_fwd_blocksparse", "fa_bwd", "fa_bwd_blocksparse", "fa_bwd_prepare", "fa_bwd_dkdv", "fa_bwd_dq",
           "fa_bwd_prepare_dq", "fa_bwd_workspace_bytes", "fa_fwd_splitkv", "fa_fwd_splitkv_partial",
           "fa_fwd_splitkv_merge", "fa_fwd_splitkv_workspace_bytes",
           "fa_fwd_splitkv_default_splits", "fa_bwd_noalloc", "fa_bwd_noalloc_max_scratch_bytes",
           "fa_status_str", "fa_version")

_lib = None


class FaError(RuntimeError):
    """A libfa call returned a status other than FA_OK."""

    def __init__(self, status, message):
        super().__init__(message)
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


def _declare(lib):
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.fa_fwd.restype = i32
    lib.fa_fwd.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, f32, i32, vp, vp, vp]
    lib.fa_fwd_blocksparse.restype = i32
    lib.fa_fwd_blocksparse.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, f32, i32, vp,
                                       i64, vp, vp, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, f32, i32,
                           vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_blocksparse.restype = i32
    lib.fa_bwd_blocksparse.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                       f32, i32, vp, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_prepare.restype = i32
    lib.fa_bwd_prepare.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.fa_bwd_dkdv.restype = i32
    lib.fa_bwd_dkdv.argtypes = [i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, f32, i32, vp, vp, vp,
                                ctypes.c_size_t, vp]
    lib.fa_bwd_dq.restype = i32
    lib.fa_bwd_dq.argtypes = [i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, f32, i32, vp, vp,
                              ctypes.c_size_t, vp]
    lib.fa_bwd_prepare_dq.restype = i32
    lib.fa_bwd_prepare_dq.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                      f32, i32, vp, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64]
    lib.fa_fwd_splitkv.restype = i32
    lib.fa_fwd_splitkv.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, f32, i32, i64,
                                   vp, vp, vp, ctypes.c_size_t, vp]
    lib.fa_fwd_splitkv_partial.restype = i32
    lib.fa_fwd_splitkv_partial.argtypes = [i32, i64, i64, i64, i64, i64, vp, vp, vp, f32, i32, i64,
                                           vp, ctypes.c_size_t, vp]
    lib.fa_fwd_splitkv_merge.restype = i32
    lib.fa_fwd_splitkv_merge.argtypes = [i32, i64, i64, i64, i64, i64, vp, ctypes.c_size_t, vp, vp,
                                         vp]
    lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64]
    lib.fa_fwd_splitkv_default_splits.restype = i64
    lib.fa_fwd_splitkv_default_splits.argtypes = [i64, i64, i64, i64, i64]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_bwd_noalloc.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, f32,
                                   i32, vp, vp, vp, vp]
    lib.fa_bwd_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_noalloc_max_scratch_bytes.argtypes = []
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [i32]
    lib.fa_version.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []


def load():
    """Load libfa.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m exact_io_aware_13_amd.build` "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(LIB_PATH)
        _declare(lib)
        _lib = lib
    return _lib


def check(status):
    """Raise FaError for a non-zero status."""
    if status != 0:
        msg = load().fa_status_str(status).decode()
        raise FaError(status, msg)
