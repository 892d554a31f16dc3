"""The C ABI on the host: exported symbols, status codes of invalid calls
(all rejected before any HIP call, so these run without a GPU), workspace
sizing and the single HIP runtime.  Every call here is invalid or empty by
construction; none reaches a kernel launch."""

import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

from exact_io_aware_13_amd import _lib  # noqa: E402

F32, BF16 = _lib.FA_F32, _lib.FA_BF16
OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, ARG = range(8)
P = 0x10000  # a 16-byte-aligned stand-in address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _fwd(lib, in_dt=BF16, out_dt=BF16, B=1, H=2, Lq=64, Lk=64, d=128, Q=P, K=P, V=P,
         scale=0.125, causal=1, O=P, lse=P):
    return lib.fa_fwd(in_dt, out_dt, B, H, Lq, Lk, d, Q, K, V, scale, causal, O, lse, None)


def _bwd(lib, in_dt=BF16, o_dt=None, B=1, H=2, Lq=64, Lk=64, d=128, ptrs=None, scale=0.125,
         causal=1, ws=P, ws_bytes=None):
    p = dict(Q=P, K=P, V=P, O=P, dO=P, lse=P, dQ=P, dK=P, dV=P)
    p.update(ptrs or {})
    o_dt = in_dt if o_dt is None else o_dt
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(in_dt, B, H, Lq, Lk, d)
    return lib.fa_bwd(in_dt, o_dt, B, H, Lq, Lk, d, p["Q"], p["K"], p["V"], p["O"], p["dO"], p["lse"],
                      scale, causal, p["dQ"], p["dK"], p["dV"], ws, ws_bytes, None)


def test_exports_match_header(lib):
    declared = set(re.findall(r"FA_API\s+[\w\s\*]*?\b(fa_\w+)\s*\(", open(HEADER).read()))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), f"libfa does not export {name}"


def test_exports_are_only_the_c_api():
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    text = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert text == set(_lib.EXPORTS), text


def test_every_kernel_launch_stub_is_defined():
    # A kernel whose host-side launch stub the compiler dropped (it has done
    # so silently for some lambda captures passed to buffer-load builtins)
    # leaves an undefined __device_stub__ symbol: the launch would fail only
    # when the library is loaded on a GPU machine.
    out = os.popen(f"nm -D --undefined-only {_lib.LIB_PATH}").read()
    missing = [l.split()[-1] for l in out.splitlines() if "__device_stub__" in l]
    assert not missing, missing


def test_version(lib):
    assert lib.fa_version().decode().startswith("libfa ")
    assert "gfx950" in lib.fa_version().decode()


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_str(code).decode().startswith(name)
    assert lib.fa_status_str(99).decode() == "unknown fa_status"


@pytest.mark.parametrize("kw,status", [
    (dict(in_dt=5), ARG), (dict(out_dt=-1), ARG), (dict(scale=float("nan")), ARG),
    (dict(scale=float("inf")), ARG),
    (dict(B=-1), SHAPE), (dict(Lq=-3), SHAPE), (dict(d=0), SHAPE), (dict(Lk=0), SHAPE),
    (dict(Lq=1 << 24), SHAPE), (dict(Lk=1 << 24), SHAPE), (dict(B=1 << 20, H=1 << 20), SHAPE),
    # Sizes whose products overflow int64 are rejected before any product.
    (dict(B=1 << 40, H=1 << 40), SHAPE), (dict(B=1 << 62, H=4), SHAPE),
    (dict(Lq=2 ** 63 - 1), SHAPE), (dict(Lk=2 ** 63 - 1), SHAPE),
    (dict(B=2 ** 63 - 1, H=2 ** 63 - 1, Lq=2 ** 63 - 1, Lk=2 ** 63 - 1), SHAPE),
    (dict(d=96), UNSUP), (dict(d=32), UNSUP), (dict(d=256), UNSUP),
    (dict(in_dt=F32, out_dt=BF16), UNSUP),
    (dict(Q=None), NULL), (dict(K=None), NULL), (dict(V=None), NULL), (dict(O=None), NULL),
    (dict(lse=None), NULL),
    (dict(Q=P + 8), ALIGN), (dict(V=P + 2), ALIGN), (dict(O=P + 4), ALIGN), (dict(lse=P + 4), ALIGN),
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Lq=0), dict(Lq=0, Lk=0),
                                dict(B=0, Lk=0)])
def test_fwd_empty_is_ok_and_touches_nothing(lib, kw):
    assert _fwd(lib, Q=None, K=None, V=None, O=None, lse=None, **kw) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(in_dt=3), ARG), (dict(scale=float("nan")), ARG),
    # O's dtype: an unknown value, and bf16 O beside fp32 inputs.
    (dict(o_dt=2), ARG), (dict(o_dt=-1), ARG), (dict(in_dt=F32, o_dt=BF16), UNSUP),
    (dict(Lk=0), SHAPE), (dict(d=80), UNSUP),
    (dict(B=1 << 40, H=1 << 40), SHAPE), (dict(Lq=2 ** 63 - 1, Lk=2 ** 63 - 1), SHAPE),
    (dict(ptrs=dict(dO=None)), NULL), (dict(ptrs=dict(lse=None)), NULL),
    (dict(ptrs=dict(dV=None)), NULL), (dict(ptrs=dict(dQ=None)), NULL),
    (dict(ptrs=dict(dK=P + 8)), ALIGN), (dict(ptrs=dict(O=P + 2)), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=100), WS), (dict(ws=P + 4), ALIGN),
])
def test_bwd_rejects(lib, kw, status):
    assert _bwd(lib, **kw) == status


def _stage(lib, name, in_dt=BF16, o_dt=None, B=1, H=2, Lq=64, Lk=64, d=128, ptrs=None,
           scale=0.125, causal=1, ws=P, ws_bytes=None):
    p = dict(Q=P, K=P, V=P, O=P, dO=P, lse=P, dQ=P, dK=P, dV=P)
    p.update(ptrs or {})
    o_dt = in_dt if o_dt is None else o_dt
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(in_dt, B, H, Lq, Lk, d)
    if name == "prepare":
        return lib.fa_bwd_prepare(in_dt, o_dt, B, H, Lq, Lk, d, p["O"], p["dO"], p["lse"], ws, ws_bytes,
                                  None)
    if name == "dkdv":
        return lib.fa_bwd_dkdv(in_dt, B, H, Lq, Lk, d, p["Q"], p["K"], p["V"], p["dO"], scale,
                               causal, p["dK"], p["dV"], ws, ws_bytes, None)
    if name == "prepare_dq":
        return lib.fa_bwd_prepare_dq(in_dt, o_dt, B, H, Lq, Lk, d, p["Q"], p["K"], p["V"], p["O"],
                                     p["dO"], p["lse"], scale, causal, p["dQ"], ws, ws_bytes, None)
    return lib.fa_bwd_dq(in_dt, B, H, Lq, Lk, d, p["Q"], p["K"], p["V"], p["dO"], scale, causal,
                         p["dQ"], ws, ws_bytes, None)


@pytest.mark.parametrize("name,kw,status", [
    ("prepare", dict(in_dt=4), ARG), ("prepare", dict(Lk=0), SHAPE), ("prepare", dict(d=48), UNSUP),
    ("prepare", dict(o_dt=7), ARG), ("prepare", dict(in_dt=F32, o_dt=BF16), UNSUP),
    ("prepare", dict(ptrs=dict(O=None)), NULL), ("prepare", dict(ptrs=dict(lse=None)), NULL),
    ("prepare", dict(ptrs=dict(dO=P + 2)), ALIGN), ("prepare", dict(ws=None), WS),
    ("prepare", dict(ws_bytes=8), WS),
    ("dkdv", dict(scale=float("nan")), ARG), ("dkdv", dict(ptrs=dict(K=None)), NULL),
    ("dkdv", dict(ptrs=dict(dV=None)), NULL), ("dkdv", dict(ptrs=dict(Q=None)), NULL),
    ("dkdv", dict(ptrs=dict(dK=P + 8)), ALIGN), ("dkdv", dict(ws=None), WS),
    ("dq", dict(ptrs=dict(dQ=None)), NULL), ("dq", dict(ptrs=dict(V=None)), NULL),
    ("dq", dict(ptrs=dict(dO=None)), NULL), ("dq", dict(ptrs=dict(Q=P + 4)), ALIGN),
    ("dq", dict(ws_bytes=0), WS), ("dq", dict(d=96), UNSUP),
    # Both stages' checks: O, lse and O's dtype (prepare), K, V and dQ (dQ).
    ("prepare_dq", dict(in_dt=4), ARG), ("prepare_dq", dict(o_dt=7), ARG),
    ("prepare_dq", dict(in_dt=F32, o_dt=BF16), UNSUP), ("prepare_dq", dict(scale=float("inf")), ARG),
    ("prepare_dq", dict(Lk=0), SHAPE), ("prepare_dq", dict(d=32), UNSUP),
    ("prepare_dq", dict(ptrs=dict(O=None)), NULL), ("prepare_dq", dict(ptrs=dict(lse=None)), NULL),
    ("prepare_dq", dict(ptrs=dict(dQ=None)), NULL), ("prepare_dq", dict(ptrs=dict(K=None)), NULL),
    ("prepare_dq", dict(ptrs=dict(V=None)), NULL), ("prepare_dq", dict(ptrs=dict(O=P + 2)), ALIGN),
    ("prepare_dq", dict(ptrs=dict(dQ=P + 8)), ALIGN), ("prepare_dq", dict(ws=None), WS),
    ("prepare_dq", dict(ws_bytes=64), WS),
])
def test_bwd_stages_reject(lib, name, kw, status):
    assert _stage(lib, name, **kw) == status


def test_bwd_stages_ignore_pointers_they_do_not_use(lib):
    # Each stage validates only what it reads or writes: the rest may be NULL
    # (the call is still rejected, here for a missing workspace, so nothing
    # is launched).
    nul = {k: None for k in ("Q", "K", "V", "dQ", "dK", "dV")}
    assert _stage(lib, "prepare", ptrs=nul, ws=None) == WS
    assert _stage(lib, "dkdv", ptrs=dict(O=None, lse=None, dQ=None), ws=None) == WS
    assert _stage(lib, "dq", ptrs=dict(O=None, lse=None, dK=None, dV=None), ws=None) == WS
    assert _stage(lib, "prepare_dq", ptrs=dict(dK=None, dV=None), ws=None) == WS


def test_bwd_stages_empty_is_ok(lib):
    nul = {k: None for k in ("Q", "K", "V", "O", "dO", "lse", "dQ", "dK", "dV")}
    for name in ("prepare", "dkdv", "dq", "prepare_dq"):
        assert _stage(lib, name, B=0, ptrs=nul, ws=None, ws_bytes=0) == OK


def test_bwd_empty_is_ok(lib):
    nul = {k: None for k in ("Q", "K", "V", "O", "dO", "lse", "dQ", "dK", "dV")}
    assert _bwd(lib, B=0, ptrs=nul, ws=None, ws_bytes=0) == OK


def test_launch_work_items_fit_32_bits(lib):
    # A dispatch carries its work-item count (grid x workgroup size) in 32
    # bits: sizes whose largest launch would exceed it are rejected, sizes
    # just below are accepted (the workspace helper validates like fa_bwd
    # and returns 0 for what fa_bwd rejects).
    assert lib.fa_bwd_workspace_bytes(BF16, 1, 65536, 4096, 4096, 128) == 0
    assert lib.fa_bwd_workspace_bytes(BF16, 1, 60000, 4096, 4096, 128) > 0
    assert lib.fa_bwd_workspace_bytes(BF16, 1, 131072, 4096, 4096, 64) == 0
    assert lib.fa_bwd_workspace_bytes(BF16, 1, 120000, 4096, 4096, 64) > 0
    assert lib.fa_bwd_workspace_bytes(F32, 1, 32768, 4096, 4096, 64) == 0
    assert lib.fa_bwd_workspace_bytes(F32, 1, 30000, 4096, 4096, 64) > 0
    assert _fwd(lib, B=1, H=65536, Lq=4096, Lk=4096) == SHAPE
    assert _fwd(lib, B=2, H=32768, Lq=4096, Lk=4096, in_dt=F32, out_dt=F32, d=64) == SHAPE


def test_workspace_is_linear_in_length(lib):
    mem = json.load(open(os.path.join(ROOT, "tests", "golden", "worked_example_memory.json")))
    L, L2 = mem["L"], mem["L_doubled"]
    w1 = lib.fa_bwd_workspace_bytes(BF16, 1, 1, L, L, 128)
    w2 = lib.fa_bwd_workspace_bytes(BF16, 1, 1, L2, L2, 128)
    # D statistic and base-2 lse: exactly 2 * 4 L bytes here.
    assert w1 == 2 * L * 4
    assert w2 == 2 * w1                               # linear in L ...
    assert mem["MiB_doubled"] == mem["growth_when_L_doubles"] * mem["MiB"]  # ... the scores grow 4x
    assert mem["elements"] == L * L and mem["bytes"] == L * L * mem["bytes_per_element"]
    assert w1 < mem["bytes"] / 10                     # far below one head's score matrix
    assert lib.fa_bwd_workspace_bytes(F32, 1, 1, L, L, 128) == 2 * L * 4
    assert lib.fa_bwd_workspace_bytes(BF16, 1, 1, L, L, 96) == 0
    for L_ in (1024, 2048, 4096, 8192):
        assert lib.fa_bwd_workspace_bytes(BF16, 1, 32, L_, L_, 128) == 32 * L_ * 8


def test_one_hip_runtime_is_mapped(lib):
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


# ---- key-split forward ------------------------------------------------------

def _skv(lib, in_dt=BF16, out_dt=BF16, B=1, H=2, Lq=4, Lk=1000, d=128, Q=P, K=P, V=P,
         scale=0.125, causal=0, nsplit=3, O=P, lse=P, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_splitkv_workspace_bytes(BF16, B, H, Lq, Lk, d, nsplit)
    return lib.fa_fwd_splitkv(in_dt, out_dt, B, H, Lq, Lk, d, Q, K, V, scale, causal, nsplit,
                              O, lse, ws, ws_bytes, None)


def test_splitkv_workspace_layout(lib):
    # Opart [nsplit,B,H,Lq,d] fp32 padded to 256 bytes, then LSEpart [nsplit,B,H,Lq].
    def expect(B, H, Lq, d, n):
        o = -(-(n * B * H * Lq * d * 4) // 256) * 256
        return o + -(-(n * B * H * Lq * 4) // 256) * 256
    for (B, H, Lq, Lk, d, n) in [(8, 32, 1, 16384, 128, 2), (1, 1, 3, 7, 64, 5), (2, 3, 17, 100, 128, 1)]:
        assert lib.fa_fwd_splitkv_workspace_bytes(BF16, B, H, Lq, Lk, d, n) == expect(B, H, Lq, d, n)
    assert lib.fa_fwd_splitkv_workspace_bytes(F32, 1, 1, 4, 8, 64, 2) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(BF16, 1, 1, 4, 8, 64, 0) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(BF16, 1, 1, 4, 8, 96, 2) == 0


def test_splitkv_default_splits_in_range(lib):
    n = lib.fa_fwd_splitkv_default_splits(8, 32, 1, 16384, 128)
    assert 1 <= n <= 64  # at least 256 keys per range
    assert lib.fa_fwd_splitkv_default_splits(1, 1, 1, 100, 128) == 1
    assert lib.fa_fwd_splitkv_default_splits(0, 1, 1, 100, 128) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(in_dt=F32, out_dt=F32), UNSUP), (dict(d=96), UNSUP), (dict(in_dt=9), ARG),
    (dict(scale=float("nan")), ARG), (dict(nsplit=0, ws_bytes=1 << 20), ARG),
    (dict(nsplit=4097, ws_bytes=1 << 30), ARG), (dict(Lk=0), SHAPE), (dict(B=-1), SHAPE),
    (dict(Q=None), NULL), (dict(K=None), NULL), (dict(V=None), NULL), (dict(O=None), NULL),
    (dict(lse=None), NULL), (dict(Q=P + 4), ALIGN), (dict(lse=P + 8), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=64), WS), (dict(ws=P + 4), ALIGN),
    (dict(B=0), OK), (dict(Lq=0), OK),
])
def test_splitkv_rejects(lib, kw, status):
    assert _skv(lib, **kw) == status


def test_splitkv_stages_validate_their_own_pointers(lib):
    ws = lib.fa_fwd_splitkv_workspace_bytes(BF16, 1, 2, 4, 1000, 128, 3)
    # The partial stage takes no O/lse; the merge takes no Q/K/V.
    assert lib.fa_fwd_splitkv_partial(BF16, 1, 2, 4, 1000, 128, None, P, P, 0.1, 0, 3, P, ws,
                                      None) == NULL
    assert lib.fa_fwd_splitkv_merge(BF16, 1, 2, 4, 128, 3, P, ws, None, P, None) == NULL
    assert lib.fa_fwd_splitkv_merge(BF16, 1, 2, 4, 128, 3, P, ws - 4, P, P, None) == WS
    assert lib.fa_fwd_splitkv_merge(BF16, 1, 2, 4, 128, 0, P, ws, P, P, None) == ARG


# ---- block-sparse forward -----------------------------------------------------

def _bs(lib, in_dt=BF16, out_dt=BF16, B=1, H=2, Lq=300, Lk=500, d=128, Q=P, K=P, V=P,
        scale=0.125, causal=0, mask=P + 1, slices=1, O=P, lse=P):
    return lib.fa_fwd_blocksparse(in_dt, out_dt, B, H, Lq, Lk, d, Q, K, V, scale, causal, mask,
                                  slices, O, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_dt=F32, out_dt=F32), UNSUP), (dict(d=96), UNSUP), (dict(Lk=4096 * 128 + 1), UNSUP),
    (dict(slices=3), ARG), (dict(slices=0), ARG), (dict(scale=float("nan")), ARG),
    (dict(Lk=0), SHAPE), (dict(mask=None), NULL), (dict(Q=None), NULL), (dict(lse=None), NULL),
    (dict(Q=P + 4), ALIGN), (dict(O=P + 2), ALIGN), (dict(B=0), OK), (dict(Lq=0), OK),
])
def test_blocksparse_rejects(lib, kw, status):
    # The mask itself may have any alignment (P + 1 above is accepted).
    assert _bs(lib, **kw) == status


def test_blocksparse_accepts_per_slice_mask_count(lib):
    assert _bs(lib, B=2, H=3, slices=6, Lq=0) == OK
    assert _bs(lib, B=2, H=3, slices=5, Lq=0) == ARG


def test_bwd_blocksparse_rejects(lib):
    ws = lib.fa_bwd_workspace_bytes(BF16, 1, 2, 300, 300, 128)
    call = lambda **kw: lib.fa_bwd_blocksparse(
        kw.get("dt", BF16), kw.get("o_dt", kw.get("dt", BF16)), 1, 2, 300, kw.get("Lk", 300), 128, P, P, P, P, P, P, 0.1, 1,
        kw.get("mask", P + 1), kw.get("slices", 1), P, P, P, P, kw.get("ws", ws), None)
    assert call(dt=F32) == UNSUP
    assert call(o_dt=5) == ARG
    assert call(dt=F32, o_dt=BF16) == UNSUP
    assert call(slices=3) == ARG
    assert call(mask=None) == NULL
    assert call(ws=8) == WS
    assert call(Lk=4096 * 128 + 1) == UNSUP


# ---- backward without a workspace argument --------------------------------

def _bwd_na(lib, in_dt=BF16, o_dt=None, B=1, H=2, Lq=64, Lk=64, d=128, ptrs=None, scale=0.125,
            causal=1):
    p = dict(Q=P, K=P, V=P, O=P, dO=P, lse=P, dQ=P, dK=P, dV=P)
    p.update(ptrs or {})
    o_dt = in_dt if o_dt is None else o_dt
    return lib.fa_bwd_noalloc(in_dt, o_dt, B, H, Lq, Lk, d, p["Q"], p["K"], p["V"], p["O"],
                              p["dO"], p["lse"], scale, causal, p["dQ"], p["dK"], p["dV"], None)


def test_noalloc_scratch_size(lib):
    # 16 MiB: D and the base-2 lse (4 bytes each) for 2^21 query rows.
    assert lib.fa_bwd_noalloc_max_scratch_bytes() == 16 * 2 ** 20
    rows = 2 ** 21
    assert lib.fa_bwd_workspace_bytes(BF16, 1, 1, rows, 64, 64) == 16 * 2 ** 20


@pytest.mark.parametrize("kw,status", [
    (dict(in_dt=9), ARG), (dict(o_dt=5), ARG), (dict(scale=float("nan")), ARG),
    (dict(in_dt=F32, o_dt=BF16), UNSUP), (dict(d=96), UNSUP), (dict(Lk=0), SHAPE),
    (dict(B=1 << 40, H=1 << 40), SHAPE),
    # Statistics beyond the fixed array: one row more than 2^21, in any split.
    (dict(B=1, H=1, Lq=2 ** 21 + 1, Lk=64, d=64), WS), (dict(B=4, H=8, Lq=65537, d=64), WS),
    (dict(ptrs=dict(dQ=None)), NULL), (dict(ptrs=dict(lse=None)), NULL),
    (dict(ptrs=dict(K=None)), NULL), (dict(ptrs=dict(dV=P + 8)), ALIGN),
    (dict(ptrs=dict(O=P + 4)), ALIGN),
])
def test_noalloc_rejects_before_any_hip_call(lib, kw, status):
    assert _bwd_na(lib, **kw) == status


def test_noalloc_empty_is_ok(lib):
    nul = {k: None for k in ("Q", "K", "V", "O", "dO", "lse", "dQ", "dK", "dV")}
    assert _bwd_na(lib, B=0, ptrs=nul) == OK
    assert _bwd_na(lib, Lq=0, Lk=0, ptrs=nul) == OK
