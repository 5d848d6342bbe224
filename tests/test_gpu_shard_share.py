"""One GPU's share of a token-sharded run. Every step of the path is row-independent
(the RMSNorm statistic, RoPE's position, SwiGLU and s are per row; weights are whole),
so G GPUs would each run the same kernels on M/G rows with no exchange, RoPE carrying
the shard's first global row as pos_offset. Here the last of 8 shards of the Llama-shaped
forward (rows 7168..8191) and the last of 4 shards of the RoPE workload (rows 3072..4095,
pos_offset 3072) run as calls of their own, and every element is compared with the
oracle's rows of the whole workload."""
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


def test_fwd_last_of_eight_shards(coda):
    import torch
    wl = W.llama_fwd()
    M = wl["M"]
    lo, hi = M - M // 8, M
    log(f"fwd shard rows {lo}..{hi - 1} of {wl.name}")
    x, z = to_dev_bf16(np.ascontiguousarray(wl["x"][lo:hi])), to_dev_bf16(np.ascontiguousarray(wl["z"][lo:hi]))
    w0, g, w1 = (to_dev_bf16(wl[k]) for k in ("w0", "gamma", "w1"))
    h1, h2, part, r, y = coda.coda_gemm_rmsnorm_fwd(x, w0, z, g, w1, wl["eps"])
    torch.cuda.synchronize()
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"], rows=np.arange(lo, hi))
    assert_close_tiles("h1", dec(h1), ref["h1"])
    assert_close_tiles("h2", dec(h2), ref["h2"])
    assert_close_tiles("r", r.cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close_tiles("y", dec(y), ref["y"])


def test_rope_last_of_four_shards(coda):
    import torch
    wl = W.rope_qkv()
    M = wl["M"]
    lo, hi = M - M // 4, M
    log(f"rope shard rows {lo}..{hi - 1} of {wl.name}, pos_offset {lo}")
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    out = coda.coda_gemm_rope(to_dev_bf16(np.ascontiguousarray(wl["x"][lo:hi])), to_dev_bf16(wl["w"]), c, s,
                              wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], wl["pos_offset"] + lo)
    torch.cuda.synchronize()
    ref = O.gemm_rope(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                      wl["pos_offset"], wl["theta"], rows=np.arange(lo, hi))
    assert_close_tiles("qkv", dec(out), ref)
