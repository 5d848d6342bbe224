"""Build step for libcoda.so: compiles the HIP sources for gfx950 with hipcc.

The library is built in-tree (next to this file) so that it travels with the source
tree; nothing is JIT-compiled or cached elsewhere. The build embeds a SHA-256 of what
it was built from (every file under csrc/, include/coda.h and the compile flags), which
the library returns from coda_build_source_hash(); loading compares it with the sources
next to the library and refuses a stale build.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libcoda.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["coda_gemm.hip", "coda_aux.hip", "coda_bwd.hip", "coda_ce.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcoda.so)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # Packed fp32 VALU ops stay disabled: the compiler must not form v_pk_*_f32.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-function",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def source_hash(root: str = ROOT, extra_flags=()) -> str:
    """SHA-256 (hex) of every file under <root>/transformer_gemm_epilogue_amd/csrc and of
    <root>/include/coda.h, in sorted order of their paths, and of the compile flags."""
    csrc = os.path.join(root, "transformer_gemm_epilogue_amd", "csrc")
    files = sorted(os.path.join("transformer_gemm_epilogue_amd", "csrc", f) for f in os.listdir(csrc)
                   if os.path.isfile(os.path.join(csrc, f)))
    files.append(os.path.join("include", "coda.h"))
    h = hashlib.sha256()
    for rel in files:
        h.update(rel.encode() + b"\0")
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read() + b"\0")
    flags = [f for f in compile_flags() if not f.startswith("-I")] + list(extra_flags)
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def build(verbose: bool = False, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    digest = source_hash(extra_flags=extra_flags)
    cmd = [hipcc(), *compile_flags(), *extra_flags, f'-DCODA_SOURCE_HASH="{digest}"', "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
