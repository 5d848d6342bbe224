"""Every kernel of the library keeps its values in registers (no GPU needed).

Each HIP source is compiled for gfx950 to device assembly with the library's flags, and
the code-object metadata of every kernel is read: no VGPR may be spilled and no kernel may
use scratch memory. (SGPRs spilled into lanes of a VGPR cost a lane write and read each, and
use no memory; the persistent GEMM spills a few that way.) The GEMM kernels run two waves per SIMD with up to 256
registers each; a change of schedule that pushes a loop past that budget compiles and
computes correct results, only far slower (a persistent GEMM once spilled 203 VGPRs this
way), so this is checked on every build rather than found in a profile."""
import os
import re
import shutil
import subprocess

import pytest

from transformer_gemm_epilogue_amd.build import CSRC, SOURCES, compile_flags


def _kernels(asm: str):
    meta = asm[asm.index("amdhsa.kernels:"):]
    for blk in meta.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        if not name:
            continue
        vals = {k: int(m.group(1)) for k in ("vgpr_count", "vgpr_spill_count", "sgpr_spill_count",
                                               "private_segment_fixed_size")
                if (m := re.search(rf"\.{k}:\s+(\d+)", blk))}
        yield name.group(1), vals


@pytest.mark.parametrize("source", SOURCES)
def test_no_kernel_spills_or_uses_scratch(source, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / (source + ".s")
    cmd = [hipcc, *compile_flags(), "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, source)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    kernels = list(_kernels(out.read_text()))
    assert kernels, "no kernels found in the device assembly"
    bad = [(n, v) for n, v in kernels if v.get("vgpr_spill_count", 0) or v.get("private_segment_fixed_size", 0)]
    assert not bad, bad
    assert all(v.get("vgpr_count", 0) <= 256 for _, v in kernels)
