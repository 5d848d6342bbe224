"""Compiles tests/c_abi/fwd_program.cpp, the C-ABI consumer with neither Python nor torch,
against the in-tree libcoda.so (hipcc, host code only; the library is found next to the
package through the binary's run path). Called by __graft_entry__.build() after the
library is built."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROGRAM = os.path.join(HERE, "fwd_program")


def build(verbose: bool = False) -> str:
    from transformer_gemm_epilogue_amd.build import hipcc
    pkg = os.path.join(ROOT, "transformer_gemm_epilogue_amd")
    cmd = [hipcc(), "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "fwd_program.cpp"), f"-L{pkg}", "-lcoda",
           "-Wl,-rpath,$ORIGIN/../../transformer_gemm_epilogue_amd", "-o", PROGRAM + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(PROGRAM + ".tmp", PROGRAM)
    return PROGRAM


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    print(build(verbose=True))
