"""The C ABI from C (CPU checks): include/coda.h compiles as strict C99 and C89 with every
entry point named from C (tests/c_abi/header_check.c), and the C++ consumer program that
the GPU tests run (tests/c_abi/fwd_program, built by __graft_entry__.build()) is built
from its current source and resolves libcoda.so to the in-tree library."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CDIR = os.path.join(ROOT, "tests", "c_abi")


@pytest.mark.parametrize("std", ["c99", "c89"])
def test_header_compiles_as_c(tmp_path, std):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    flags = ["-Wall", "-Wextra", "-pedantic", "-Werror"] if std == "c99" else ["-fsyntax-only"]
    out = [] if std == "c89" else ["-c", "-o", str(tmp_path / "hc.o")]
    res = subprocess.run([cc, f"-std={std}", *flags, f"-I{os.path.join(ROOT, 'include')}",
                          os.path.join(CDIR, "header_check.c"), *out], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_header_check_names_every_declared_entry_point():
    import re
    header = open(os.path.join(ROOT, "include", "coda.h")).read()
    declared = set(re.findall(r"^(?:int|const char\*)\s+(coda_\w+)\s*\(", header, re.M))
    named = set(re.findall(r"\(any_fn\)&(coda_\w+)", open(os.path.join(CDIR, "header_check.c")).read()))
    assert declared and declared == named


def test_consumer_program_is_built_and_links_the_in_tree_library():
    prog = os.path.join(CDIR, "fwd_program")
    assert os.path.exists(prog), "run __graft_entry__.build() first"
    assert os.path.getmtime(prog) >= os.path.getmtime(os.path.join(CDIR, "fwd_program.cpp"))
    res = subprocess.run(["ldd", prog], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    line = next(ln for ln in res.stdout.splitlines() if "libcoda.so" in ln)
    assert os.path.realpath(line.split("=>")[1].split("(")[0].strip()) == \
        os.path.realpath(os.path.join(ROOT, "transformer_gemm_epilogue_amd", "libcoda.so"))
