"""Parity of the rest of the RMSNorm backward (the grad GEMM with the RMSNorm-backward
epilogue, the output-side statistic and the dgamma column reduction) with the fp64
oracle, through the C ABI.

The GPU path gets what a forward pass leaves behind: r from the normalised rows of h1
(torch, fp32) and y = r (h1 * gamma) W1 from the library's own row-scale GEMM (bf16).
The oracle computes everything exactly from the base inputs (h1, gamma, W1, dY, g_res),
so the comparison also covers the roundings of r and y that the GPU path carries.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu

TIGHT = 1e-4  # fp32 outputs against fp64: relative Frobenius bound


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


def gpu_inputs(coda, wl, with_gres=True):
    """Device tensors plus the forward's r (fp32) and y (bf16) as the GPU path gets them."""
    import torch
    dev = {k: to_dev_bf16(wl[k]) for k in ("h1", "gamma", "w1", "dy", "g_res")}
    if not with_gres:
        dev["g_res"] = None
    h = dev["h1"].float()
    r = torch.rsqrt((h * h).mean(dim=1) + wl["eps"]).contiguous()
    h2 = (h * dev["gamma"].float()).to(torch.bfloat16).contiguous()
    y = coda.coda_gemm_rowscale(h2, dev["w1"], r)
    sync()
    return dev, r, y


def run(coda, dev, r, y):
    out = coda.coda_rmsnorm_bwd(dev["dy"], dev["w1"], dev["h1"], dev["gamma"], r, y, g_res=dev["g_res"])
    sync()
    return out


def oracle(wl, with_gres=True, rows=None, cols=None):
    return O.rmsnorm_bwd(wl["h1"], wl["gamma"], wl["w1"], wl["dy"], wl["eps"],
                         g_res=wl["g_res"] if with_gres else None, rows=rows, cols=cols)


def s_from_gpu_y(wl, y, rows=None):
    """The output-side statistic from the y the GPU used, in fp64 (checks the row-dot)."""
    dy = O.decode_bf16(wl["dy"])
    yy = dec(y)
    if rows is not None:
        dy, yy = dy[rows], yy[rows]
    return (dy * yy).sum(axis=1) / wl["h1"].shape[1]


@pytest.mark.parametrize("shape,with_gres", [((517, 392, 264), True), ((256, 256, 256), False),
                                             ((700, 520, 328), True), ((3, 16, 8), True), ((1, 8, 8), False)])
def test_rmsnorm_bwd_small_full_compare(coda, shape, with_gres):
    M, D, N = shape
    log(f"rmsnorm_bwd M={M} D={D} N={N} g_res={with_gres}")
    wl = W.rmsnorm_bwd_full(50 + M % 11, M, D, N)
    dev, r, y = gpu_inputs(coda, wl, with_gres)
    s, dh1, part, dgamma = run(coda, dev, r, y)
    ref = oracle(wl, with_gres)
    assert_close("s (row-dot of the GPU's y)", s.cpu().numpy(), s_from_gpu_y(wl, y), rel_fro=TIGHT)
    assert_close("s", s.cpu().numpy(), ref["s"])
    assert_close("dh1", dec(dh1), ref["dh1"])
    assert_close("dgamma_partials", part.cpu().numpy(), ref["dgamma_partials"], rel_fro=TIGHT)
    assert_close("dgamma", dgamma.cpu().numpy(), ref["dgamma"], rel_fro=TIGHT)


def test_rmsnorm_bwd_zero_gradient_rows(coda):
    """Rows of dY that are zero: both forms of the row statistic (output side, and dH2 . h2
    from the grad GEMM's epilogue) are exactly zero, the dH2 row is zero, and dh1 reduces to
    the residual-stream gradient g_res exactly (every other term of the epilogue is an exact
    zero). Zero rows on a row-tile edge and in the ragged last tile; the rest matches the
    oracle."""
    import torch
    base = W.rmsnorm_bwd_full(31, 300, 256, 264)
    wl = {k: base[k].copy() for k in ("h1", "gamma", "w1", "dy", "g_res")}
    wl["eps"] = base["eps"]
    rows = [0, 255, 256, 299]
    wl["dy"][rows] = 0
    dev, r, y = gpu_inputs(coda, wl)
    s, dh1, part, dgamma = run(coda, dev, r, y)
    ref = oracle(wl)
    assert_close("dh1", dec(dh1), ref["dh1"])
    assert_close("dgamma", dgamma.cpu().numpy(), ref["dgamma"], rel_fro=TIGHT)
    assert np.all(s.cpu().numpy()[rows] == 0.0)
    assert np.array_equal(dec(dh1)[rows], O.decode_bf16(wl["g_res"])[rows])
    h2 = (dev["h1"].float() * dev["gamma"].float()).to(torch.bfloat16).contiguous()
    dh2, p2, s2 = coda.coda_gemm_rmsnorm_bwd_stats(dev["dy"], dev["w1"], h2)
    sync()
    assert not dec(dh2)[rows].any() and not p2.cpu().numpy()[rows].any()
    assert np.all(s2.cpu().numpy()[rows] == 0.0)


def test_rmsnorm_bwd_full_size(coda):
    wl = W.rmsnorm_bwd_full()
    log(f"rmsnorm_bwd {wl.name}")
    dev, r, y = gpu_inputs(coda, wl)
    s, dh1, part, dgamma = run(coda, dev, r, y)
    ref = oracle(wl)
    assert_close_tiles("s (row-dot of the GPU's y)", s.cpu().numpy(), s_from_gpu_y(wl, y), rel_fro=TIGHT)
    assert_close_tiles("s", s.cpu().numpy(), ref["s"])
    assert_close_tiles("dh1", dec(dh1), ref["dh1"])
    assert_close_tiles("dgamma", dgamma.cpu().numpy(), ref["dgamma"], rel_fro=TIGHT)
    assert_close_tiles("dgamma_partials", part.cpu().numpy(), ref["dgamma_partials"], rel_fro=TIGHT, tile_m=1)


def test_rmsnorm_bwd_stages_equal_composition_and_deterministic(coda):
    wl = W.rmsnorm_bwd_full(61, 600, 264, 392)
    dev, r, y = gpu_inputs(coda, wl)
    s, dh1, part, dgamma = run(coda, dev, r, y)
    s2 = coda.coda_rowdot_stat(dev["dy"], y, 264)
    dh1b, partb = coda.coda_gemm_rmsnorm_bwd_dx(dev["dy"], dev["w1"], dev["h1"], dev["gamma"], r, s2,
                                                g_res=dev["g_res"])
    dg2 = coda.coda_colsum_reduce(partb)
    s3, dh1c, partc, dg3 = run(coda, dev, r, y)
    sync()
    for a, b in ((s, s2), (dh1, dh1b), (part, partb), (dgamma, dg2), (s, s3), (dh1, dh1c), (dgamma, dg3)):
        assert bool((a == b).all())


def test_rmsnorm_bwd_residual_gradient_is_added(coda):
    wl = W.rmsnorm_bwd_full(62, 300, 136, 200)
    dev, r, y = gpu_inputs(coda, wl)
    _, with_g, _, dg1 = run(coda, dev, r, y)
    dev_ng = dict(dev, g_res=None)
    _, without_g, _, dg0 = run(coda, dev_ng, r, y)
    assert_close("dh1(g) - dh1(0)", dec(with_g) - dec(without_g), O.decode_bf16(wl["g_res"]), rel_fro=5e-2)
    assert bool((dg1 == dg0).all())   # the residual-stream gradient does not reach gamma


def test_colsum_reduce_order_and_empty(coda):
    import torch
    rng = np.random.default_rng(7)
    P = rng.standard_normal((37, 300)).astype(np.float32)
    out = coda.coda_colsum_reduce(torch.from_numpy(P).cuda())
    sync()
    want = np.zeros(300, dtype=np.float32)
    for t in range(37):      # the documented order t = 0, 1, ... in fp32
        want = want + P[t]
    assert np.array_equal(out.cpu().numpy(), want)
    empty = torch.empty((0, 300), dtype=torch.float32, device="cuda")
    z = coda.coda_colsum_reduce(empty, out=torch.full((300,), 5.0, device="cuda"))
    sync()
    assert bool((z == 0).all())


def test_rmsnorm_bwd_empty_batch(coda):
    import torch
    D, N = 64, 48
    bf = dict(dtype=torch.bfloat16, device="cuda")
    dy, y = torch.empty((0, N), **bf), torch.empty((0, N), **bf)
    w1, h1, g = torch.zeros((D, N), **bf), torch.empty((0, D), **bf), torch.ones((D,), **bf)
    r = torch.empty((0,), dtype=torch.float32, device="cuda")
    dgamma = torch.full((D,), 3.0, device="cuda")
    s, dh1, part, dg = coda.coda_rmsnorm_bwd(dy, w1, h1, g, r, y, dgamma=dgamma)
    sync()
    assert part.shape == (0, D) and dh1.shape == (0, D) and s.shape == (0,)
    assert bool((dg == 0).all())


# the column reduction keeps the order t = 0, 1, ..., tiles-1 (loads batched 16 at a time,
# adds in order): bit for bit a sequential fp32 sum, across batch boundaries and the tail
@pytest.mark.parametrize("tiles", [0, 1, 15, 16, 17, 33, 100])
def test_colsum_reduce_sum_order_is_sequential(coda, tiles):
    import torch
    rng = np.random.default_rng(100 + tiles)
    for width in (8, 1000, 4096):
        P = (rng.standard_normal((tiles, width)) * np.exp(rng.uniform(-8, 8, (tiles, 1)))).astype(np.float32)
        got = coda.coda_colsum_reduce(torch.from_numpy(P).cuda())
        sync()
        ref = np.zeros(width, dtype=np.float32)
        for t in range(tiles):
            ref = ref + P[t]  # fp32 adds in order
        assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
