"""Build-time check of the decode kernels' resources (CPU; hipcc
cross-compiles for gfx950 here).

Every decode, combine and prologue kernel is written to fit its register budget (the launch
bounds and waves-per-EU each kernel declares): a kernel that spilled would
stream its spills through scratch memory: extra vector-memory operations
and HBM traffic inside the KV loop, which is bound by its KV loads.  Checked in the
generated code of every instance, so a change that pushes one over its
budget fails here rather than as a slower run.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "load_balanced_split_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _asm(tmp_path, source):
    out = tmp_path / (source + ".s")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                           "--cuda-device-only", "-S", os.path.join(CSRC, source),
                           "-o", str(out)], stderr=subprocess.DEVNULL)
    return out.read_text()


def _descriptors(asm):
    """{kernel: private segment size} from the kernel descriptors."""
    res = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, re.S):
        size = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2))
        res[m.group(1)] = int(size.group(1)) if size else None
    return res


@pytest.mark.parametrize("source,at_least", [("decode.hip", 48), ("combine.hip", 2),
                                             ("prologue.hip", 16)])
def test_kernels_do_not_spill(tmp_path, source, at_least):
    asm = _asm(tmp_path, source)
    kernels = _descriptors(asm)
    assert len(kernels) >= at_least, sorted(kernels)
    spilled = {k: v for k, v in kernels.items() if v != 0}
    assert not spilled, spilled
    assert "scratch_store" not in asm and "scratch_load" not in asm
