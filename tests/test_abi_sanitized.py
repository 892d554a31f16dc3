"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

fa_api.hip -- argument validation, workspace layout and dispatch -- is built
for the host with g++ and both sanitizers, its kernel launchers replaced by
stand-ins that return success (tests/abi_sanitize/launch_stubs.cpp).  Every
call that tests/test_abi.py makes is recorded with the status the real
library returns, then replayed against that build
(tests/abi_sanitize/replay.cpp), which must return the same status; a
sanitizer finding (an out-of-bounds access, a signed overflow in a size
product, ...) aborts the replay.  Valid calls that reach the stand-ins and
sizes at the edges of int64 are replayed too."""

import inspect
import itertools
import os
import shutil
import subprocess

import pytest

from tests import test_abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "abi_sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, ARG = range(8)
P = test_abi.P
BIG = 2 ** 63 - 1


class Recorder:
    """Forwards calls to the real library and records (name, args, result)."""

    def __init__(self, lib):
        self._lib = lib
        self.calls = []

    def __getattr__(self, name):
        fn = getattr(self._lib, name)

        def call(*args):
            r = fn(*args)
            rec = len(r) if isinstance(r, bytes) else int(r)
            self.calls.append((name, args, rec))
            return r
        return call


def _fmt(x):
    if x is None:
        return "0"
    if isinstance(x, float):
        return repr(x) + "f"
    return str(int(x))


def _line(name, args, result):
    return " ".join([name] + [_fmt(a) for a in args] + ["=>", str(result)])


def _run_abi_tests(rec):
    """Call every test of test_abi.py that takes the library, over every
    parameter combination, with the recorder as the library."""
    n = 0
    for name, fn in inspect.getmembers(test_abi, inspect.isfunction):
        if not name.startswith("test_") or "lib" not in inspect.signature(fn).parameters:
            continue
        grids = []
        for mark in getattr(fn, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names = [s.strip() for s in mark.args[0].split(",")]
            grids.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in mark.args[1]])
        for combo in itertools.product(*grids):
            kw = {}
            for d in combo:
                kw.update(d)
            fn(rec, **kw)
            n += 1
    return n


# Calls the real library cannot make without a GPU (they pass every check and
# would launch kernels): the stand-ins make them return FA_OK.
VALID = [
    ("fa_fwd", (1, 1, 1, 2, 300, 500, 128, P, P, P, 0.125, 1, P, P, None), OK),
    ("fa_fwd", (0, 0, 2, 3, 129, 17, 64, P, P, P, -0.5, 0, P, P, None), OK),
    ("fa_fwd", (1, 0, 1, 1, 4_194_047, 4_194_047, 128, P, P, P, 0.1, 1, P, P, None), OK),
    ("fa_bwd", (1, 0, 1, 2, 300, 300, 128, P, P, P, P, P, P, 0.1, 1, P, P, P, P, 1 << 20, None), OK),
    ("fa_bwd", (0, 0, 1, 2, 64, 640, 64, P, P, P, P, P, P, 0.1, 0, P, P, P, P, 1 << 20, None), OK),
    ("fa_bwd_blocksparse", (1, 1, 1, 2, 300, 300, 128, P, P, P, P, P, P, 0.1, 1, P + 1, 2, P, P, P,
                            P, 1 << 20, None), OK),
    ("fa_fwd_blocksparse", (1, 1, 2, 3, 256, 300, 64, P, P, P, 0.1, 0, P + 3, 6, P, P, None), OK),
    ("fa_fwd_splitkv", (1, 0, 8, 32, 1, 16384, 128, P, P, P, 0.1, 0, 2, P, P, P, 1 << 24, None), OK),
    ("fa_bwd_prepare", (1, 0, 1, 2, 300, 300, 128, P, P, P, P, 1 << 20, None), OK),
    ("fa_bwd_dkdv", (1, 1, 2, 300, 300, 128, P, P, P, P, 0.1, 1, P, P, P, 1 << 20, None), OK),
    ("fa_bwd_dq", (1, 1, 2, 300, 300, 128, P, P, P, P, 0.1, 1, P, P, 1 << 20, None), OK),
    ("fa_bwd_prepare_dq", (1, 1, 1, 2, 300, 300, 128, P, P, P, P, P, P, 0.1, 1, P, P, 1 << 20, None),
     OK),
    ("fa_bwd_prepare_dq", (1, 0, 1, 2, 300, 300, 64, P, P, P, P, P, P, 0.1, 0, P, P, 1 << 20, None),
     OK),
    # Sizes at the edges of int64 and of the 32-bit per-slice offsets.
    ("fa_fwd", (1, 1, BIG, BIG, BIG, BIG, 128, P, P, P, 0.1, 1, P, P, None), SHAPE),
    ("fa_fwd", (1, 1, -BIG - 1, 1, 1, 1, 128, P, P, P, 0.1, 1, P, P, None), SHAPE),
    ("fa_fwd", (1, 1, 2 ** 31 - 1, 2 ** 31 - 1, 1, 1, 64, P, P, P, 0.1, 1, P, P, None), SHAPE),
    ("fa_bwd_workspace_bytes", (1, 2 ** 40, 2 ** 40, 64, 64, 128), 0),
    ("fa_bwd_workspace_bytes", (1, 1, 1, BIG, BIG, 64), 0),
    ("fa_fwd_splitkv_workspace_bytes", (1, 2 ** 31 - 1, 2, 2 ** 20, 64, 128, 4096), 0),
    ("fa_fwd_splitkv_workspace_bytes", (1, BIG, BIG, BIG, BIG, 64, 4096), 0),
    ("fa_bwd_noalloc", (1, 1, BIG, 1, 1, 1, 64, P, P, P, P, P, P, 0.1, 1, P, P, P, None), SHAPE),
    ("fa_fwd_splitkv_default_splits", (BIG, BIG, BIG, BIG, 128), 1),
]


def _compiler():
    cxx = shutil.which("g++")
    if not cxx:
        pytest.skip("g++ not available")
    return cxx


def test_abi_host_code_is_sanitizer_clean(tmp_path):
    from exact_io_aware_13_amd import _lib
    rec = Recorder(_lib.load())
    n_tests = _run_abi_tests(rec)
    assert n_tests > 100 and len(rec.calls) > 100
    calls = tmp_path / "calls.txt"
    calls.write_text("\n".join([_line(*c) for c in rec.calls] + [_line(*c) for c in VALID]) + "\n")

    exe = tmp_path / "replay"
    # Host-only build: the HIP headers in host mode (no device compiler),
    # HIP_SYMBOL spelled out as the runtime headers define it.
    cmd = [_compiler(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-DHIP_SYMBOL(x)=((const void*)&(x))",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "exact_io_aware_13_amd", "csrc"),
           "-I", os.path.join(ROCM, "include"),
           "-x", "c++", os.path.join(ROOT, "exact_io_aware_13_amd", "csrc", "fa_api.hip"),
           "-x", "none", os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "replay.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe), str(calls)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "0 mismatches" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
