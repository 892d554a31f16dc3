"""Builds libfa.so (the C-ABI attention library) for gfx950 with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then linked into ``libfa.so`` next to this file.  The benchmark's
shader-clock probe (``clock/clock_probe.hip``) is built apart, into
``libfa_clock.so``: it is no part of the attention library.  hipcc
cross-compiles for gfx950 without a GPU present.

Run:  python -m exact_io_aware_13_amd.build
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
CLOCK_SRC = os.path.join(PKG, "clock", "clock_probe.hip")
CLOCK_LIB = os.path.join(PKG, "libfa_clock.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from forming packed fp32 VALU ops.
# -fno-honor-nans / -mno-amdgpu-ieee: the kernels never see NaNs (masked
# scores are -inf, which both flags keep exact), and without them every
# fmaxf input is first re-quieted by an extra max instruction.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, cc, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [cc, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx-only feature flag; that note is noise.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose=False):
    """Compile every HIP source and link libfa.so.  Always recompiles."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    # A kernel whose host-side instantiation the compiler dropped leaves an
    # undefined launch stub behind; fail here rather than at load time.
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        missing = [l.split()[-1] for l in und.splitlines() if "_ZN2fa" in l]
        if missing:
            raise RuntimeError("libfa links with undefined internal symbols: " + ", ".join(missing))
    os.replace(tmp, LIB)
    build_clock_probe(cc)
    return LIB


def build_clock_probe(cc=None):
    """Compile the benchmark's shader-clock probe into libfa_clock.so."""
    cc = cc or hipcc()
    tmp = CLOCK_LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-O3", "-fPIC", "-shared", "-fvisibility=hidden",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", CLOCK_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, CLOCK_LIB)
    return CLOCK_LIB


if __name__ == "__main__":
    print(build(verbose=True))
