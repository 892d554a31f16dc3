"""Register budget of the fp32 kernels (CPU only: a gfx950 device-code
compile, no GPU).  Every fp32 kernel instantiation must fit its registers
without spilling to scratch memory: a spill turns every access of the
spilled values into a memory round trip."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_13_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def test_fp32_kernels_do_not_spill(tmp_path):
    from exact_io_aware_13_amd import build
    out = tmp_path / "f32.s"
    flags = [f for f in build.CFLAGS if f not in ("-fPIC",)]
    r = subprocess.run([_hipcc(), *flags, "--cuda-device-only", "-S", "-o", str(out),
                        os.path.join(CSRC, "fa_f32.hip")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    meta = out.read_text()
    names = re.findall(r"\.name:\s+(\S+_f32_kernel\S*)", meta)
    # fwd, pre, dK/dV, dQ over d and the causal flag; dK/dV and dQ with 4, 8
    # or 16 columns per lane; the eight-wave forward at d = 64 with 4, 8 or
    # 16 columns and the four-wave forward at d = 128 with 4 or 8
    assert len(names) == 40, names
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", meta)]
    scratch = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", meta)]
    assert spills and max(spills) == 0, spills
    assert scratch and max(scratch) == 0, scratch
    # Every workgroup's LDS fits a compute unit (160 KiB).
    lds = [int(x) for x in re.findall(r"\.group_segment_fixed_size:\s+(\d+)", meta)]
    assert len(lds) == len(names) and max(lds) <= 160 * 1024, lds
