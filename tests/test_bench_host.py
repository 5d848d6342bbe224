"""Host checks of bench.py (no GPU): the one-GPU contract and the source fingerprint that
ties the committed HBM counter record to the kernels it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "..")


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    for n in ("2", "8"):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                             capture_output=True, text=True, timeout=120)
        assert res.returncode == 2, res.stderr
        assert "one GPU" in res.stderr
        assert res.stdout == ""  # no JSON line


def test_source_fingerprint_is_stable_and_covers_the_gemm_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    h = bench.source_hash()
    assert h == bench.source_hash() and len(h) == 64
    # a one-byte change in any of GEMM1's sources changes it (on a copy of the sources)
    csrc = tmp_path / "transformer_gemm_epilogue_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.GEMM1_SOURCES:
        (csrc / name).write_bytes(open(os.path.join(ROOT, "transformer_gemm_epilogue_amd", "csrc", name), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.source_hash() == h
    for name in bench.GEMM1_SOURCES:
        orig = (csrc / name).read_bytes()
        (csrc / name).write_bytes(orig + b" ")
        assert bench.source_hash() != h, name
        (csrc / name).write_bytes(orig)
    assert "coda_gemm.hpp" in bench.GEMM1_SOURCES and "coda_gemm.hip" in bench.GEMM1_SOURCES
