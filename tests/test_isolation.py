"""The oracle and the product path stay apart (CPU checks).

- Nothing in the package (binding, build step, HIP sources) or in the C header names the
  oracle, and importing the package loads no module of it.
- The oracle imports nothing of the package, and shares no source file with it.
- bench.py imports the oracle only inside cpu_baseline (its CPU leg), and the smoke test
  only inside smoke(); the workload generators hold none of the method's arithmetic and
  import neither side.
"""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "transformer_gemm_epilogue_amd")


def _files(top, exts):
    for d, _, fs in os.walk(top):
        if "__pycache__" in d:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(d, f)


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    out = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out += [(a.name.split(".")[0], node) for a in node.names]
        elif isinstance(node, ast.ImportFrom) and node.module:
            out.append((node.module.split(".")[0], node))
    return tree, out


def test_package_and_header_do_not_name_the_oracle():
    for path in list(_files(PKG, (".py", ".hip", ".hpp", ".h", ".cpp"))) + [os.path.join(ROOT, "include", "coda.h")]:
        text = open(path, errors="replace").read()
        assert "import oracle" not in text and "from oracle" not in text, path
        assert "coda_oracle" not in text, path
        if path.endswith(".py"):
            for mod, _ in _imports(path)[1]:
                assert mod != "oracle", f"{path} imports the oracle"


def test_importing_the_package_loads_no_oracle_module():
    code = ("import sys; sys.path.insert(0, %r); import transformer_gemm_epilogue_amd; "
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "[]"


def test_oracle_imports_nothing_of_the_product():
    for path in _files(os.path.join(ROOT, "oracle"), (".py",)):
        for mod, _ in _imports(path)[1]:
            assert mod not in ("transformer_gemm_epilogue_amd", "bench", "__graft_entry__"), path


def test_workload_generators_import_neither_side():
    for path in _files(os.path.join(ROOT, "workloads"), (".py",)):
        for mod, _ in _imports(path)[1]:
            assert mod not in ("oracle", "transformer_gemm_epilogue_amd"), path


def _functions_importing_oracle(path):
    tree, imps = _imports(path)
    owners = set()
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.AsyncFunctionDef)):
            for node in ast.walk(fn):
                if isinstance(node, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in node.names):
                    owners.add(fn.name)
                if isinstance(node, ast.ImportFrom) and (node.module or "").split(".")[0] == "oracle":
                    owners.add(fn.name)
    total = sum(1 for mod, _ in imps if mod == "oracle")
    return owners, total


def test_bench_and_smoke_import_the_oracle_only_in_their_cpu_legs():
    owners, total = _functions_importing_oracle(os.path.join(ROOT, "bench.py"))
    assert owners == {"cpu_baseline"} and total == 1
    owners, total = _functions_importing_oracle(os.path.join(ROOT, "__graft_entry__.py"))
    assert owners == {"smoke"} and total == 1


def test_missing_library_fails_loudly(tmp_path):
    """A copy of the package without its built library refuses to run any op: there is
    no CPU or eager fallback behind the binding."""
    import shutil
    dst = tmp_path / "transformer_gemm_epilogue_amd"
    shutil.copytree(PKG, dst, ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import torch, transformer_gemm_epilogue_amd as c\n"
            "assert c.__file__.startswith(%r), c.__file__\n"
            "x = torch.zeros((8, 8), dtype=torch.bfloat16)\n"
            "for fn in (lambda: c.lib(), lambda: c.coda_gemm_swiglu(x, torch.zeros((8, 16), dtype=torch.bfloat16))):\n"
            "    try:\n"
            "        fn()\n"
            "    except Exception as e:\n"
            "        print('refused:', type(e).__name__)\n"
            "    else:\n"
            "        print('ran')\n") % (str(tmp_path), str(tmp_path))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=str(tmp_path))
    assert out.returncode == 0, out.stderr
    lines = out.stdout.split("\n")
    assert lines[0] == "refused: RuntimeError" and lines[1].startswith("refused:"), out.stdout
