"""Parity over a seeded sweep of ragged shapes, through the C ABI: every fused entry point
and its split-depth variant against the fp64 oracle on shapes drawn at random (rows
1..1300, depths and widths any multiple of 8 up to 2104 and 1400), so that ragged last
row, feature and depth tiles, a single depth step, a single row and one to several
depth slices all occur; the persistent RoPE schedule equals the per-tile one bit for bit. The shapes are fixed by the seed; each case prints its shape
before it runs."""
import os

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu
TIGHT = 1e-4


def _shapes(seed, n, max_rows=1300, max_width=1400, max_depth=2104):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, max_rows + 1))
        K = 8 * int(rng.integers(1, max_depth // 8 + 1))  # 8 .. 2104 (1 .. 66 depth steps) by default
        N = 8 * int(rng.integers(1, max_width // 8 + 1))  # 8 .. 1400 by default
        out.append((M, K, N))
    out[0] = (1, 8, 8)                                 # one row, one depth step, one ragged tile
    return out


# CODA_SWEEP_SEED, CODA_SWEEP_N and CODA_SWEEP_MAX_{ROWS,WIDTH,DEPTH} draw another, longer or
# larger sweep (the default is the committed one)
_env = os.environ.get
SHAPES = _shapes(int(_env("CODA_SWEEP_SEED", "2026")), int(_env("CODA_SWEEP_N", "12")),
                 int(_env("CODA_SWEEP_MAX_ROWS", "1300")), int(_env("CODA_SWEEP_MAX_WIDTH", "1400")),
                 int(_env("CODA_SWEEP_MAX_DEPTH", "2104")))
SPLIT = [False, True]


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


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("shape", SHAPES)
def test_sweep_forward(coda, shape, split):
    M, K, D = shape
    N1 = 8 * (1 + (M * 7 + K) % 97)
    log(f"sweep fwd split={split} M={M} K={K} D={D} N1={N1}")
    wl = W.gemm_rmsnorm_fwd_inputs(3000 + M, M, K, D, N1, 1e-5)
    args = [to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")]
    fn = coda.coda_gemm_rmsnorm_fwd_ws if split else coda.coda_gemm_rmsnorm_fwd
    h1, h2, part, r, y = fn(*args, wl["eps"])
    sync()
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    assert_close_tiles("h1", dec(h1), ref["h1"])
    assert_close_tiles("h2", dec(h2), ref["h2"])
    assert_close_tiles("partials", part.cpu().numpy(), ref["partials"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("r", r.cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close_tiles("y", dec(y), ref["y"])


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("shape", SHAPES)
def test_sweep_rope_and_backward(coda, shape, split):
    M, K, N = shape
    hd = 64 if N % 2 else 128
    n_q, n_k, n_v = hd * (1 + N % 3), hd, hd * (N % 2)
    pos = (M * 13) % 97
    for inverse in (False, True):
        log(f"sweep rope inverse={inverse} split={split} M={M} K={K} heads={n_q // hd},{n_k // hd},{n_v // hd} "
            f"head_dim={hd}")
        gen = W.rope_bwd if inverse else W.rope_qkv
        wl = gen(seed=3100 + M, M=M, K=K, n_q=n_q, n_k=n_k, n_v=n_v, head_dim=hd, seq_len=M + pos + 3,
                 pos_offset=pos)
        c, s = coda.coda_rope_tables(wl["seq_len"], hd, wl["theta"])
        name = ("coda_gemm_rope_bwd" if inverse else "coda_gemm_rope") + ("_ws" if split else "")
        out = getattr(coda, name)(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, n_q, n_k, n_v, hd,
                                  wl["seq_len"], pos)
        sync()
        oracle = O.gemm_rope_bwd if inverse else O.gemm_rope
        ref = oracle(wl["x"], wl["w"], n_q, n_k, n_v, hd, wl["seq_len"], pos, wl["theta"])
        assert_close_tiles("qkv", dec(out), ref)
        if not inverse and not split:   # the persistent schedule: the per-tile output, bit for bit
            per = coda.coda_gemm_rope_persistent(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, n_q, n_k, n_v,
                                                 hd, wl["seq_len"], pos)
            sync()
            assert np.array_equal(bf16_bits(per), bf16_bits(out))


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("shape", SHAPES)
def test_sweep_swiglu_and_backward(coda, shape, split):
    M, K, N = shape
    F = N
    log(f"sweep swiglu split={split} M={M} K={K} F={F}")
    wl = W.swiglu(seed=3200 + M, M=M, K=K, F=F)
    fn = coda.coda_gemm_swiglu_ws if split else coda.coda_gemm_swiglu
    out = fn(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]))
    sync()
    assert_close_tiles("out", dec(out), O.gemm_swiglu(wl["x"], wl["w"]))
    log(f"sweep swiglu_bwd split={split} M={M} Dm={K} F={F}")
    wb = W.swiglu_bwd(seed=3300 + M, M=M, Dm=K, F=F)
    fn = coda.coda_gemm_swiglu_bwd_ws if split else coda.coda_gemm_swiglu_bwd
    dh = fn(to_dev_bf16(wb["dy"]), to_dev_bf16(wb["w_down"]), to_dev_bf16(wb["h"]))
    sync()
    ref = O.gemm_swiglu_bwd(wb["dy"], wb["w_down"], wb["h"])["dh"]
    got = dec(dh)
    assert_close("dG", got[:, 0::2], ref[:, 0::2])
    assert_close("dU", got[:, 1::2], ref[:, 1::2])


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("shape", SHAPES)
def test_sweep_backward_statistic(coda, shape, split):
    M, N, D = shape
    log(f"sweep bwd_stats split={split} M={M} D={D} N={N}")
    wl = W.bwd_stats(seed=3400 + M, M=M, D=D, N=N)
    fn = coda.coda_gemm_rmsnorm_bwd_stats_ws if split else coda.coda_gemm_rmsnorm_bwd_stats
    dh2, part, s = fn(to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w1"]), to_dev_bf16(wl["h2"]))
    sync()
    ref = O.gemm_rmsnorm_bwd_stats(wl["dy"], wl["w1"], wl["h2"])
    assert_close_tiles("dh2", dec(dh2), ref["dh2"])
    assert_close_tiles("partials", part.cpu().numpy(), ref["partials"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("s", s.cpu().numpy(), ref["s_prime"], rel_fro=TIGHT)


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("shape", SHAPES)
def test_sweep_rmsnorm_backward(coda, shape, split):
    """dh1 and dgamma from the grad GEMM, with r, y and s as the GPU path has them."""
    import torch
    M, N, D = shape
    log(f"sweep rmsnorm_bwd split={split} M={M} D={D} N={N}")
    wl = W.rmsnorm_bwd_full(3500 + M, M, D, N)
    dev = {k: to_dev_bf16(wl[k]) for k in ("h1", "gamma", "w1", "dy", "g_res")}
    h = dev["h1"].float()
    r = torch.rsqrt((h * h).mean(dim=1) + wl["eps"]).contiguous()
    y = coda.coda_gemm_rowscale((h * dev["gamma"].float()).to(torch.bfloat16).contiguous(), dev["w1"], r)
    s = coda.coda_rowdot_stat(dev["dy"], y, D)
    fn = coda.coda_gemm_rmsnorm_bwd_dx_ws if split else coda.coda_gemm_rmsnorm_bwd_dx
    dh1, part = fn(dev["dy"], dev["w1"], dev["h1"], dev["gamma"], r, s, g_res=dev["g_res"])
    dgamma = coda.coda_colsum_reduce(part)
    sync()
    ref = O.rmsnorm_bwd(wl["h1"], wl["gamma"], wl["w1"], wl["dy"], wl["eps"], g_res=wl["g_res"])
    assert_close_tiles("dh1", dec(dh1), ref["dh1"])
    assert_close("dgamma", dgamma.cpu().numpy(), ref["dgamma"], rel_fro=TIGHT)


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("shape", SHAPES)
def test_sweep_cross_entropy(coda, shape, split):
    import torch
    M, K, V = shape
    log(f"sweep cross_entropy split={split} M={M} K={K} V={V}")
    wl = W.cross_entropy(seed=3600 + M, M=M, K=K, V=V, ignore_every=5)
    labels = torch.from_numpy(wl["labels"]).cuda()
    fn = coda.coda_gemm_cross_entropy_ws if split else coda.coda_gemm_cross_entropy
    loss, lse, target, tile = (t.cpu().numpy() for t in fn(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), labels))
    ref = O.gemm_cross_entropy(wl["x"], wl["w"], wl["labels"])
    assert_close_tiles("tile_lse", tile, ref["tile_lse"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close_tiles("target", target, ref["target"], rel_fro=TIGHT)
    assert_close_tiles("loss", loss, ref["loss"], rel_fro=TIGHT)
    assert np.all(loss[~ref["valid"]] == 0) and np.all(target[~ref["valid"]] == 0)
