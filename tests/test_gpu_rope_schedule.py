"""GEMM + RoPE under both schedules, through the C ABI: the one-workgroup-per-tile
kernel and the persistent one (min(tiles, CUs) workgroups walking the tiles, the DMA
ring running on from one tile into the next). Parity with the fp64 oracle on every
element, bit-identity of the two schedules (same tile sums in the same order), and the
8192-class configuration at full size. Also the register-only MFMA probe the bench uses
for the power-limited ceiling (closed-form outputs)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def sync():
    import torch
    torch.cuda.synchronize()


def dec(t):
    return O.decode_bf16(bf16_bits(t))


def both_schedules(coda, wl):
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    x, w = to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"])
    args = (wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    a = coda.coda_gemm_rope(x, w, c, s, *args)
    b = coda.coda_gemm_rope_persistent(x, w, c, s, *args)
    sync()
    return a, b


def oracle_full(wl):
    return O.gemm_rope(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                       wl["pos_offset"], wl["theta"])


# More tiles than CUs, so persistent workgroups walk two or three tiles each. The loop
# runs ten depth steps per round and leaves 4 to 13 to the tail that loads the next
# tile's first steps: depth steps 4 .. 14 cover every tail length, both parities of the
# step that pairs the next tile's X loads (an odd count pairs across the two tiles) and
# every ring advance per tile (K/32 mod 5); 17 steps add a nonzero (even) depth
# rotation; ragged M and N; K below the persistent minimum.
@pytest.mark.parametrize("case", [
    dict(M=8192, K=128, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=0),
    dict(M=8192, K=160, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=4096, pos_offset=3),
    dict(M=8192, K=192, n_q=1536, n_k=1536, n_v=1536, head_dim=64, seq_len=8192, pos_offset=0),
    dict(M=8192, K=224, n_q=2048, n_k=1024, n_v=1024, head_dim=128, seq_len=8192, pos_offset=0),
    dict(M=8192, K=256, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=0),
    dict(M=8000, K=288, n_q=1000, n_k=1000, n_v=1000, head_dim=8, seq_len=5000, pos_offset=11),
    dict(M=8192, K=320, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=0),
    dict(M=8192, K=352, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=5),
    dict(M=8192, K=384, n_q=1536, n_k=1536, n_v=1536, head_dim=64, seq_len=8192, pos_offset=0),
    dict(M=8100, K=416, n_q=1024, n_k=1024, n_v=1024, head_dim=128, seq_len=8192, pos_offset=0),
    dict(M=8192, K=448, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=0),
    dict(M=8192, K=544, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=1),
    dict(M=8192, K=64, n_q=1536, n_k=1536, n_v=1536, head_dim=128, seq_len=8192, pos_offset=0),
])
def test_persistent_matches_per_tile_and_oracle(coda, case):
    log(f"rope schedules {case}")
    wl = W.rope_qkv(seed=21 + case["K"], **case)
    a, b = both_schedules(coda, wl)
    assert bool((a.view(-1) == b.view(-1)).all()), "persistent and per-tile schedules differ"
    assert_close_tiles("qkv (persistent)", dec(b), oracle_full(wl))


def test_rope_8192_full_size(coda):
    wl = W.rope_qkv_8k()
    log(f"rope {wl.name}")
    a, b = both_schedules(coda, wl)
    assert bool((a == b).all()), "persistent and per-tile schedules differ"
    got = dec(a)
    ref = oracle_full(wl)
    assert_close_tiles("qkv", got, ref)
    n_q, nqk = wl["n_q"], wl["n_q"] + wl["n_k"]
    assert_close("q", got[:, :n_q], ref[:, :n_q])
    assert_close("k", got[:, n_q:nqk], ref[:, n_q:nqk])
    assert_close("v", got[:, nqk:], ref[:, nqk:])


def test_mfma_probe_closed_form(coda):
    import torch
    # every operand 1.0: each accumulator element sums 32 products per round, so a
    # thread's 32 x 4 accumulator values add up to 128 * 32 * iters
    ones = torch.full((4096 * 8,), 1.0, dtype=torch.bfloat16, device="cuda")
    for iters in (1, 3, 10):
        out = coda.coda_baseline_mfma_loop(ones, iters, 2)
        sync()
        assert bool((out == 4096.0 * iters).all())
    zeros = torch.zeros((8,), dtype=torch.bfloat16, device="cuda")
    out = coda.coda_baseline_mfma_loop(zeros, 5, 1)
    sync()
    assert bool((out == 0).all())


def test_mfma_probe_rejects_bad_arguments(coda):
    import torch
    lib = coda.lib()
    ops = torch.zeros((64,), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((512,), dtype=torch.float32, device="cuda")
    import ctypes
    p, o = ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(out.data_ptr())
    assert lib.coda_baseline_mfma_loop(p, 0, 1, 1, o, None) != 0
    assert lib.coda_baseline_mfma_loop(p, 8, 0, 1, o, None) != 0
    assert lib.coda_baseline_mfma_loop(p, 8, 1, 0, o, None) != 0
    assert lib.coda_baseline_mfma_loop(p, 8, 1, 65536, o, None) != 0
    assert lib.coda_baseline_mfma_loop(None, 8, 1, 1, o, None) != 0
