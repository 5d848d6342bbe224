"""The forward rewrite without allocation (coda_gemm_rmsnorm_fwd_noalloc), through the C
ABI: its outputs equal, bit for bit, those of coda_gemm_rmsnorm_fwd (same kernels, the
row partials in the library's fixed device array instead of a caller's buffer), on two
calls in a row, the second smaller than the first, so stale partials from the first
call would show. Torch allocates nothing during the calls (every output is passed in),
and sizes past the array's capacity are refused before anything runs. Captured in a HIP
graph (the use it exists for), its replays, with eager work and synchronisations between
them, equal the eager call bit for bit."""
import numpy as np
import pytest

import workloads as W
from gpu_util import bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def outputs(M, D, N1):
    import torch
    return (torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
            torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
            torch.empty((M,), dtype=torch.float32, device="cuda"),
            torch.empty((M, N1), dtype=torch.bfloat16, device="cuda"))


def test_noalloc_matches_allocating_entry_point_on_two_calls(coda):
    import torch
    cases = [(1000, 512, 1024, 264, 71), (300, 264, 520, 256, 72)]   # the second is smaller (and ragged)
    for M, K, D, N1, seed in cases:
        log(f"noalloc fwd M={M} K={K} D={D} N1={N1}")
        wl = W.gemm_rmsnorm_fwd_inputs(seed, M, K, D, N1, 1e-5)
        x, w0, z, g, w1 = (to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1"))
        ref = coda.coda_gemm_rmsnorm_fwd(x, w0, z, g, w1, wl["eps"])
        h1, h2, r, y = outputs(M, D, N1)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        coda.coda_gemm_rmsnorm_fwd_noalloc(x, w0, z, g, w1, wl["eps"], h1, h2, r, y)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        for a, b in ((h1, ref[0]), (h2, ref[1]), (y, ref[4])):
            assert np.array_equal(bf16_bits(a), bf16_bits(b))
        assert np.array_equal(r.cpu().numpy(), ref[3].cpu().numpy())
        assert np.all(np.isfinite(r.cpu().numpy()))


def test_noalloc_refuses_sizes_past_the_array(coda):
    import torch
    M, D = 65537, 4096       # M * 16 partials > 2^20
    x = torch.zeros((8, 8), dtype=torch.bfloat16, device="cuda")
    L = coda.lib()
    p = x.data_ptr()
    st = L.coda_gemm_rmsnorm_fwd_noalloc(p, p, p, p, p, M, 8, D, 8, 1e-5, p, p, p, p, None)
    assert st == 4    # CODA_ERR_WORKSPACE
    assert L.coda_gemm_rmsnorm_fwd_noalloc(p, p, p, p, p, 0, 8, D, 8, 1e-5, p, p, p, p, None) == 0


def test_noalloc_forward_replays_from_a_graph(coda):
    import torch
    M, K, D, N1 = 600, 512, 768, 264
    log(f"noalloc graph M={M} K={K} D={D} N1={N1}")
    wl = W.gemm_rmsnorm_fwd_inputs(73, M, K, D, N1, 1e-5)
    x, w0, z, g, w1 = (to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1"))
    h1, h2 = (torch.empty((M, D), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    r = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        coda.coda_gemm_rmsnorm_fwd_noalloc(x, w0, z, g, w1, wl["eps"], h1, h2, r, y)   # eager, also the lookup
    torch.cuda.synchronize()
    want = [bf16_bits(h1), bf16_bits(h2), r.cpu().numpy(), bf16_bits(y)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        coda.coda_gemm_rmsnorm_fwd_noalloc(x, w0, z, g, w1, wl["eps"], h1, h2, r, y)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (h1, h2, y):
            t.fill_(0)                       # eager work between replays: clear the outputs
        r.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bf16_bits(h1), bf16_bits(h2), r.cpu().numpy(), bf16_bits(y)]
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager call"
