"""The C ABI's host-side validation under the address and undefined-behaviour
sanitizers (no GPU).

tests/host_sanitize/abi_validation.cpp calls every entry point with NULL, misaligned,
overlapping and extreme arguments (each int argument swept over values around the shape
limits and the int range). It is compiled here together with the library's sources,
with both sanitizers on the host code only, and run on this machine, which has no GPU:
calls that pass validation must then fail in the HIP runtime (CODA_ERR_HIP), and any
sanitizer report fails the test. The driver refuses to run where a GPU is visible."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_gemm_epilogue_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_validation.cpp")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="host-only check: it is meant for a machine without a GPU")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_validation")
    srcs = [os.path.join(CSRC, f) for f in ("coda_gemm.hip", "coda_aux.hip", "coda_bwd.hip", "coda_ce.hip")]
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", DRIVER, *srcs, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    print(out[-2000:])
    assert run.returncode == 0, out[-4000:]
    assert "0 failures" in out and "runtime error" not in out and "AddressSanitizer" not in out
