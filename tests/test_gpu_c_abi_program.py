"""The C ABI without Python: tests/c_abi/fwd_program (plain hipMalloc'd buffers, the null
stream, no torch) runs the forward rewrite and GEMM + SwiGLU as a child process on inputs
from the seeded workload generators. Its outputs match the fp64 oracle, and equal, bit
for bit, the same calls made through the Python binding."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "c_abi", "fwd_program")


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def test_c_program_matches_oracle_and_binding(coda, tmp_path):
    import torch
    assert os.path.exists(PROGRAM), "run __graft_entry__.build() first"
    M, K, D, N1, F = 300, 264, 520, 264, 136
    wl = W.gemm_rmsnorm_fwd_inputs(4700, M, K, D, N1, 1e-5)
    ws = W.swiglu(seed=4701, M=M, K=K, F=F)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        for a in (wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], ws["x"], ws["w"]):
            f.write(np.ascontiguousarray(a, dtype=np.uint16).tobytes())
    log(f"c program M={M} K={K} D={D} N1={N1} F={F}")
    res = subprocess.run([PROGRAM, str(inp), str(outp), str(M), str(K), str(D), str(N1), "1e-5", str(F)],
                         capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0
    nb = coda.num_partials(D)
    raw = np.fromfile(outp, dtype=np.uint8)
    sizes = [M * D * 2, M * D * 2, M * nb * 4, M * 4, M * N1 * 2, M * F * 2]
    assert raw.size == sum(sizes)
    parts = np.split(raw, np.cumsum(sizes)[:-1])
    h1, h2, y, sw = (parts[i].view(np.uint16) for i in (0, 1, 4, 5))
    part, r = parts[2].view(np.float32).reshape(M, nb), parts[3].view(np.float32)
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    assert_close_tiles("h1", O.decode_bf16(h1.reshape(M, D)), ref["h1"])
    assert_close_tiles("y", O.decode_bf16(y.reshape(M, N1)), ref["y"])
    assert_close("r", r, ref["r"], rel_fro=1e-4)
    assert_close_tiles("swiglu", O.decode_bf16(sw.reshape(M, F)), O.gemm_swiglu(ws["x"], ws["w"]))
    # the same calls through the binding: the same bits
    b = coda.coda_gemm_rmsnorm_fwd(*(to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")), wl["eps"])
    s = coda.coda_gemm_swiglu(to_dev_bf16(ws["x"]), to_dev_bf16(ws["w"]))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(b[0]).ravel(), h1) and np.array_equal(bf16_bits(b[1]).ravel(), h2)
    assert np.array_equal(b[2].cpu().numpy(), part) and np.array_equal(b[3].cpu().numpy(), r)
    assert np.array_equal(bf16_bits(b[4]).ravel(), y) and np.array_equal(bf16_bits(s).ravel(), sw)
