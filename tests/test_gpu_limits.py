"""The documented size limits, through the C ABI: the most rows a call takes (2^24, here
2^24 - 5 for a ragged last tile), the widest output and the deepest depth (2^22 each),
with the other dimensions small so that the inputs stay small. They exercise the largest
grids (65536 and 16384 tiles), 131072 depth steps in one tile (and in 8 slices of the
split-depth schedule), the auxiliary reductions over 16384 partials per row, and the
byte offsets at those sizes. Outputs are compared with the oracle on sampled rows that
include the first and the last (most rows), or on every element (the others)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu
TIGHT = 1e-4
MAX_ROWS = 1 << 24
MAX_DIM = 1 << 22


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


def test_most_rows_forward(coda):
    import torch
    M, K, D, N1 = MAX_ROWS - 5, 8, 8, 8
    log(f"limits: forward M={M} K={K} D={D} N1={N1}")
    wl = W.gemm_rmsnorm_fwd_inputs(4100, M, K, D, N1, 1e-5)
    h1, h2, part, r, y = coda.coda_gemm_rmsnorm_fwd(*(to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")),
                                                    wl["eps"])
    sync()
    rng = np.random.default_rng(4101)
    rows = np.unique(np.r_[0:3, 255:258, rng.integers(0, M, 500), M - 300:M])
    idx = torch.from_numpy(rows).cuda()
    ref = O.gemm_rmsnorm_fwd(wl["x"][rows], wl["w0"], wl["z"][rows], wl["gamma"], wl["w1"], wl["eps"])
    assert_close("h1", dec(h1[idx]), ref["h1"])
    assert_close("h2", dec(h2[idx]), ref["h2"])
    assert_close("partials", part[idx].cpu().numpy(), ref["partials"], rel_fro=TIGHT)
    assert_close("r", r[idx].cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close("y", dec(y[idx]), ref["y"])


@pytest.mark.parametrize("split", [False, True])
def test_widest_output_and_deepest_depth_forward(coda, split):
    """GEMM1 writes 2^22 features per row (16384 tiles and partials per row); GEMM2 then
    walks a depth of 2^22 (131072 steps in one tile, or 8 slices)."""
    M, K, D, N1 = 40, 8, MAX_DIM, 8
    log(f"limits: forward split={split} M={M} K={K} D={D} N1={N1}")
    wl = W.gemm_rmsnorm_fwd_inputs(4200, M, K, D, N1, 1e-5)
    fn = coda.coda_gemm_rmsnorm_fwd_ws if split else coda.coda_gemm_rmsnorm_fwd
    h1, h2, part, r, y = fn(*(to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")), wl["eps"])
    sync()
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    assert_close_tiles("h1", dec(h1), ref["h1"])
    assert_close_tiles("h2", dec(h2), ref["h2"])
    assert_close_tiles("partials", part.cpu().numpy(), ref["partials"], rel_fro=TIGHT, tile_n=1)
    assert_close("r", r.cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close("y", dec(y), ref["y"])


@pytest.mark.parametrize("split", [False, True])
def test_deepest_depth_nk(coda, split):
    """The NK layout at a depth of 2^22: the SwiGLU backward's grad GEMM dY W_down^T."""
    M, Dm, F = 40, MAX_DIM, 8
    log(f"limits: swiglu_bwd split={split} M={M} Dm={Dm} F={F}")
    wl = W.swiglu_bwd(seed=4300, M=M, Dm=Dm, F=F)
    fn = coda.coda_gemm_swiglu_bwd_ws if split else coda.coda_gemm_swiglu_bwd
    dh = fn(to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w_down"]), to_dev_bf16(wl["h"]))
    sync()
    assert_close("dh", dec(dh), O.gemm_swiglu_bwd(wl["dy"], wl["w_down"], wl["h"])["dh"])


def test_widest_vocabulary_cross_entropy(coda):
    """2^22 logits per row: 16384 tile partials merged per row; every 5th label ignored."""
    import torch
    M, K, V = 40, 8, MAX_DIM
    log(f"limits: cross_entropy M={M} K={K} V={V}")
    wl = W.cross_entropy(seed=4400, M=M, K=K, V=V, ignore_every=5)
    loss, lse, target, tile = (t.cpu().numpy() for t in coda.coda_gemm_cross_entropy(
        to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), torch.from_numpy(wl["labels"]).cuda()))
    ref = O.gemm_cross_entropy(wl["x"], wl["w"], wl["labels"])
    assert_close("tile_lse", tile, ref["tile_lse"], rel_fro=TIGHT)
    assert_close("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close("target", target, ref["target"], rel_fro=TIGHT)
    assert_close("loss", loss, ref["loss"], rel_fro=TIGHT)
    assert np.all(loss[~ref["valid"]] == 0) and np.all(target[~ref["valid"]] == 0)


def test_widest_output_swiglu_and_rope(coda):
    """Output widths of 2^22: GEMM + SwiGLU with 2F = 2^22 (2^21 outputs per row) and
    GEMM + RoPE with 2^22 Q/K/V columns (32768 heads)."""
    M, K = 40, 8
    log(f"limits: swiglu M={M} K={K} F={MAX_DIM // 2}")
    wl = W.swiglu(seed=4500, M=M, K=K, F=MAX_DIM // 2)
    out = coda.coda_gemm_swiglu(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]))
    sync()
    assert_close_tiles("swiglu", dec(out), O.gemm_swiglu(wl["x"], wl["w"]))
    hd = 128
    n_q, n_k, n_v = MAX_DIM // 2, MAX_DIM // 4, MAX_DIM // 4
    log(f"limits: rope M={M} K={K} N={n_q + n_k + n_v}")
    wl = W.rope_qkv(seed=4600, M=M, K=K, n_q=n_q, n_k=n_k, n_v=n_v, head_dim=hd, seq_len=64, pos_offset=11)
    c, s = coda.coda_rope_tables(64, hd, wl["theta"])
    out = coda.coda_gemm_rope(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, n_q, n_k, n_v, hd, 64, 11)
    sync()
    assert_close_tiles("qkv", dec(out), O.gemm_rope(wl["x"], wl["w"], n_q, n_k, n_v, hd, 64, 11, wl["theta"]))
