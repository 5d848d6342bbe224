"""The forward rewrite under the split-depth schedule (coda_gemm_rmsnorm_fwd_ws), through
the C ABI: a GEMM whose output has fewer 256 x 256 tiles than the GPU has CUs cuts each
tile's depth into slices, stores fp32 partial tiles to the caller's workspace, and runs
the epilogue on their sum in slice order. Parity with the fp64 oracle on every element
(ragged shapes where both GEMMs split, slices of unequal length, a ragged last depth
step), determinism from call to call, bit-identity with coda_gemm_rmsnorm_fwd when no
GEMM splits, and the workspace's error paths."""
import ctypes

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu
TIGHT = 1e-4


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def dec(t):
    return O.decode_bf16(bf16_bits(t))


def dev_inputs(wl):
    return [to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")]


def check(got, ref):
    h1, h2, part, r, y = got
    assert_close_tiles("h1", dec(h1), ref["h1"])
    assert_close_tiles("h2", dec(h2), ref["h2"])
    assert_close_tiles("partials", part.cpu().numpy(), ref["partials"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("r", r.cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close_tiles("y", dec(y), ref["y"])


@pytest.mark.parametrize("shape", [
    (300, 1024, 1032, 264),   # both GEMMs split; GEMM2's slices are 18 and 15 steps, its last step ragged
    (513, 2048, 768, 1024),   # GEMM1 in 4 slices of 16 steps, GEMM2 one kernel
    (40, 4096, 520, 520),     # one token tile, ragged features
    (300, 4128, 264, 264),    # GEMM1 in 8 slices of 18 steps but the last of 3 (129 steps)
])
def test_split_depth_small_full_compare(coda, shape):
    import torch
    M, K, D, N1 = shape
    need = coda.coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1)
    log(f"split fwd M={M} K={K} D={D} N1={N1} workspace {need} B")
    assert need > 0
    wl = W.gemm_rmsnorm_fwd_inputs(60 + M % 11, M, K, D, N1, 1e-5)
    got = coda.coda_gemm_rmsnorm_fwd_ws(*dev_inputs(wl), wl["eps"])
    torch.cuda.synchronize()
    check(got, O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"]))


def test_split_depth_one_gpu_share_of_llama(coda):
    """The last of 8 token shards of the Llama-shaped forward (1024 rows: 64 GEMM1 tiles,
    96 GEMM2 tiles), the case the split-depth schedule is for."""
    import torch
    wl = W.llama_fwd()
    M = wl["M"]
    lo, hi = M - M // 8, M
    log(f"split fwd shard rows {lo}..{hi - 1} of {wl.name}")
    x = to_dev_bf16(np.ascontiguousarray(wl["x"][lo:hi]))
    z = to_dev_bf16(np.ascontiguousarray(wl["z"][lo:hi]))
    w0, g, w1 = (to_dev_bf16(wl[k]) for k in ("w0", "gamma", "w1"))
    assert coda.coda_gemm_rmsnorm_fwd_workspace_bytes(hi - lo, wl["K"], wl["D"], wl["N1"]) > 0
    got = coda.coda_gemm_rmsnorm_fwd_ws(x, w0, z, g, w1, wl["eps"])
    torch.cuda.synchronize()
    check(got, O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"],
                                  rows=np.arange(lo, hi)))


def test_split_depth_is_deterministic(coda):
    import torch
    wl = W.gemm_rmsnorm_fwd_inputs(71, 300, 1024, 1032, 264, 1e-5)
    a = coda.coda_gemm_rmsnorm_fwd_ws(*dev_inputs(wl), wl["eps"])
    b = coda.coda_gemm_rmsnorm_fwd_ws(*dev_inputs(wl), wl["eps"])
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        if u.dtype == torch.bfloat16:
            assert np.array_equal(bf16_bits(u), bf16_bits(v))
        else:
            assert np.array_equal(u.cpu().numpy(), v.cpu().numpy())


def test_no_split_equals_one_kernel_schedule(coda):
    import torch
    M, K, D, N1 = 4096, 512, 4096, 4096          # 256 tiles in each GEMM: nothing splits
    assert coda.coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1) == 0
    wl = W.gemm_rmsnorm_fwd_inputs(72, M, K, D, N1, 1e-5)
    dev = dev_inputs(wl)
    a = coda.coda_gemm_rmsnorm_fwd_ws(*dev, wl["eps"])
    b = coda.coda_gemm_rmsnorm_fwd(*dev, wl["eps"])
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        if u.dtype == torch.bfloat16:
            assert np.array_equal(bf16_bits(u), bf16_bits(v))
        else:
            assert np.array_equal(u.cpu().numpy(), v.cpu().numpy())


def test_split_depth_workspace_errors(coda):
    import torch
    M, K, D, N1 = 300, 1024, 1032, 264
    need = coda.coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1)
    wl = W.gemm_rmsnorm_fwd_inputs(73, M, K, D, N1, 1e-5)
    x, w0, z, g, w1 = dev_inputs(wl)
    h1, h2 = (torch.empty((M, D), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    part = torch.empty((M, coda.num_partials(D)), dtype=torch.float32, device="cuda")
    r = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    L = coda.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [p(x), p(w0), p(z), p(g), p(w1), M, K, D, N1, ctypes.c_float(1e-5), p(h1), p(h2), p(part), p(r), p(y)]
    assert L.coda_gemm_rmsnorm_fwd_ws(*args, p(ws), need - 16, None) == 4        # CODA_ERR_WORKSPACE
    assert L.coda_gemm_rmsnorm_fwd_ws(*args, None, 0, None) == 1                 # CODA_ERR_NULL
    assert L.coda_gemm_rmsnorm_fwd_ws(*args, p(ws), -1, None) == 6               # CODA_ERR_ARG
    big = torch.empty((need + M * D * 2,), dtype=torch.uint8, device="cuda")
    args_alias = list(args)
    args_alias[10] = ctypes.c_void_p(big.data_ptr() + need - 64)                 # h1 inside the workspace
    assert L.coda_gemm_rmsnorm_fwd_ws(*args_alias, p(big), need, None) == 6      # CODA_ERR_ARG
    assert L.coda_gemm_rmsnorm_fwd_ws(*args, p(ws), need, None) == 0
    torch.cuda.synchronize()


# ------------------------------------------------------------ RoPE and SwiGLU, split depth
def test_rope_split_depth_small(coda):
    import torch
    wl = W.rope_qkv(seed=31, M=300, K=1024, n_q=256, n_k=128, n_v=128, head_dim=128, seq_len=300, pos_offset=7)
    N = 512
    assert coda.coda_split_workspace_bytes(300, N, 1024) > 0
    log("rope split M=300 K=1024 N=512")
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    out = coda.coda_gemm_rope_ws(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, wl["n_q"], wl["n_k"], wl["n_v"],
                                 wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    torch.cuda.synchronize()
    ref = O.gemm_rope(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                      wl["pos_offset"], wl["theta"])
    assert_close_tiles("qkv", dec(out), ref)


def test_rope_split_depth_last_of_eight_shards(coda):
    """The last of 8 token shards of the RoPE workload (512 rows, 96 output tiles: two
    slices each), pos_offset = the shard's first row."""
    import torch
    wl = W.rope_qkv()
    M = wl["M"]
    lo, hi = M - M // 8, M
    N = wl["n_q"] + wl["n_k"] + wl["n_v"]
    assert coda.coda_split_workspace_bytes(hi - lo, N, wl["K"]) > 0
    log(f"rope split shard rows {lo}..{hi - 1}")
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    out = coda.coda_gemm_rope_ws(to_dev_bf16(np.ascontiguousarray(wl["x"][lo:hi])), to_dev_bf16(wl["w"]), c, s,
                                 wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                                 wl["pos_offset"] + lo)
    torch.cuda.synchronize()
    ref = O.gemm_rope(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                      wl["pos_offset"], wl["theta"], rows=np.arange(lo, hi))
    assert_close_tiles("qkv", dec(out), ref)


def test_rope_no_split_equals_one_kernel_schedule(coda):
    import torch
    wl = W.rope_qkv(seed=32, M=4096, K=256, n_q=2048, n_k=1024, n_v=1024, head_dim=128, seq_len=4096)
    assert coda.coda_split_workspace_bytes(4096, 4096, 256) == 0
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    args = (to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"],
            wl["seq_len"], wl["pos_offset"])
    a = coda.coda_gemm_rope_ws(*args)
    b = coda.coda_gemm_rope(*args)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(a), bf16_bits(b))


def test_swiglu_split_depth_small(coda):
    import torch
    M, K, F = 300, 1024, 264
    wl = W.swiglu(seed=33, M=M, K=K, F=F)
    assert coda.coda_split_workspace_bytes(M, 2 * F, K) > 0
    log(f"swiglu split M={M} K={K} F={F}")
    out = coda.coda_gemm_swiglu_ws(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]))
    torch.cuda.synchronize()
    assert_close_tiles("out", dec(out), O.gemm_swiglu(wl["x"], wl["w"]))


def test_rope_and_swiglu_workspace_errors(coda):
    import torch
    L = coda.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    M, K, F = 300, 1024, 264
    need = coda.coda_split_workspace_bytes(M, 2 * F, K)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((K, 2 * F), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    assert L.coda_gemm_swiglu_ws(p(x), p(w), M, K, F, p(out), p(ws), need - 16, None) == 4
    assert L.coda_gemm_swiglu_ws(p(x), p(w), M, K, F, p(out), None, 0, None) == 1
    assert L.coda_gemm_swiglu_ws(p(x), p(w), M, K, F, p(out), p(ws), -1, None) == 6
    assert L.coda_gemm_swiglu_ws(p(x), p(w), M, K, F, p(out), p(ws), need, None) == 0
    c = torch.zeros((300 * 64,), dtype=torch.float32, device="cuda")
    wr = torch.zeros((K, 512), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty((M, 512), dtype=torch.bfloat16, device="cuda")
    need2 = coda.coda_split_workspace_bytes(M, 512, K)
    ws2 = torch.empty((need2,), dtype=torch.uint8, device="cuda")
    args = [p(x), p(wr), p(c), p(c), M, K, 256, 128, 128, 128, 300, 0, p(o2)]
    assert L.coda_gemm_rope_ws(*args, p(ws2), need2 - 16, None) == 4
    assert L.coda_gemm_rope_ws(*args, p(o2), need2, None) == 6        # workspace on the output
    assert L.coda_gemm_rope_ws(*args, p(ws2), need2, None) == 0
    torch.cuda.synchronize()
