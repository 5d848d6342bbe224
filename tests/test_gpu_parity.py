"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle on seeded inputs.

Small cases span several 256x256 tiles with ragged tails in every dimension and are
checked element by element in full. The five stated workloads run at full size in the
same launch configuration the bench times, and every element of every output is
compared with the oracle's full result, on the whole tensor and on each 256 x 256 output
tile on its own. Integer-valued inputs make the main loop's result exact, so those cases
are compared bit for bit.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import (assert_close, assert_close_tiles, bf16_bits, errors, log, to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu

TIGHT = 1e-4  # fp32 outputs (r, s, partials) against fp64: relative Frobenius bound


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


# ------------------------------------------------------------------ forward GEMM-RMSNorm-GEMM
def run_fwd(coda, wl):
    dev = {k: to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")}
    h1, h2, part, r, y = coda.coda_gemm_rmsnorm_fwd(dev["x"], dev["w0"], dev["z"], dev["gamma"], dev["w1"],
                                                    wl["eps"])
    sync()
    return h1, h2, part, r, y


def check_fwd(got, ref):
    h1, h2, part, r, y = got
    assert_close_tiles("h1", dec(h1), ref["h1"])
    assert_close_tiles("h2", dec(h2), ref["h2"])
    assert_close_tiles("partials", part.cpu().numpy(), ref["partials"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("r", r.cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close_tiles("y", dec(y), ref["y"])


@pytest.mark.parametrize("shape", [(256, 256, 256, 256), (700, 328, 520, 264), (37, 64, 256, 8), (1, 8, 8, 8)])
def test_fwd_small_full_compare(coda, shape):
    M, K, D, N1 = shape
    log(f"fwd M={M} K={K} D={D} N1={N1}")
    wl = (W.tiny_fwd(0) if shape == (256, 256, 256, 256)
          else W.gemm_rmsnorm_fwd_inputs(40 + M % 7, M, K, D, N1, 1e-5))
    got = run_fwd(coda, wl)
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    check_fwd(got, ref)


def test_fwd_degenerate_rows(coda):
    """Rows whose residual-stream value h1 is exactly zero (x and z zero) have a zero mean
    square, so r = 1/sqrt(eps) and every output of the row is exactly zero; a row with x
    zero and z constant c has h1 = c, r = 1/sqrt(c^2 + eps) in closed form and h2 = c gamma
    exactly (c a power of two). Zero rows sit at tile edges and in the ragged last tile."""
    M, K, D, N1 = 300, 64, 512, 264
    base = W.gemm_rmsnorm_fwd_inputs(77, M, K, D, N1, 1e-5)
    wl = {k: base[k].copy() for k in ("x", "w0", "z", "gamma", "w1")}
    wl["eps"] = base["eps"]
    zero_rows, const_row = [0, 5, 255, 256, M - 1], 130
    for m in zero_rows + [const_row]:
        wl["x"][m] = 0
        wl["z"][m] = 0
    wl["z"][const_row] = 0x4000  # bf16 bits of 2.0
    got = run_fwd(coda, wl)
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    check_fwd(got, ref)
    h1, h2, part, r, y = (dec(got[0]), dec(got[1]), got[2].cpu().numpy(), got[3].cpu().numpy(), dec(got[4]))
    for m in zero_rows:
        assert not h1[m].any() and not h2[m].any() and not part[m].any() and not y[m].any(), m
        assert abs(r[m] * np.sqrt(wl["eps"]) - 1.0) <= 1e-6, (m, r[m])
    assert np.all(h1[const_row] == 2.0)
    assert np.array_equal(h2[const_row], 2.0 * O.decode_bf16(wl["gamma"]))
    assert abs(r[const_row] * np.sqrt(4.0 + wl["eps"]) - 1.0) <= 1e-6, r[const_row]


def test_fwd_llama_full_size(coda):
    wl = W.llama_fwd()
    log(f"fwd {wl.name}")
    got = run_fwd(coda, wl)
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    check_fwd(got, ref)
    r = got[3].cpu().numpy()
    assert np.all(np.isfinite(r)) and np.all(r > 0)


def test_fwd_stages_equal_composition(coda):
    """coda_gemm_residual_rmsnorm_partials + coda_rowstat_reduce + coda_gemm_rowscale
    give bit-identical results to coda_gemm_rmsnorm_fwd."""
    wl = W.gemm_rmsnorm_fwd_inputs(7, 520, 256, 512, 264, 1e-5)
    dev = {k: to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")}
    h1, h2, part, r, y = coda.coda_gemm_rmsnorm_fwd(dev["x"], dev["w0"], dev["z"], dev["gamma"], dev["w1"],
                                                    wl["eps"])
    h1b, h2b, partb = coda.coda_gemm_residual_rmsnorm_partials(dev["x"], dev["w0"], dev["z"], dev["gamma"])
    rb = coda.coda_rowstat_reduce(partb, 512, wl["eps"], coda.ROWSTAT_RSQRT_MEAN_EPS)
    yb = coda.coda_gemm_rowscale(h2b, dev["w1"], rb)
    sync()
    for a, b in ((h1, h1b), (h2, h2b), (y, yb)):
        assert np.array_equal(bf16_bits(a), bf16_bits(b))
    assert np.array_equal(part.cpu().numpy(), partb.cpu().numpy())
    assert np.array_equal(r.cpu().numpy(), rb.cpu().numpy())


def test_fwd_deterministic(coda):
    wl = W.gemm_rmsnorm_fwd_inputs(8, 600, 512, 768, 256, 1e-5)
    a = run_fwd(coda, wl)
    b = run_fwd(coda, wl)
    for i in (0, 1, 4):
        assert np.array_equal(bf16_bits(a[i]), bf16_bits(b[i]))
    for i in (2, 3):
        assert np.array_equal(a[i].cpu().numpy(), b[i].cpu().numpy())


def test_fused_error_not_above_unfused_path(coda):
    """Numerics of the rewrite: applying r after GEMM2 keeps y at least as close to the
    exact result as the operator-by-operator bf16 path (GEMM, residual, RMSNorm, GEMM
    with bf16 intermediates)."""
    wl = W.llama_fwd(seed=3, M=512)
    dev = {k: to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")}
    _, _, _, _, y = coda.coda_gemm_rmsnorm_fwd(dev["x"], dev["w0"], dev["z"], dev["gamma"], dev["w1"], wl["eps"])
    h0 = coda.coda_baseline_gemm(dev["x"], dev["w0"])
    _, _, o = coda.coda_baseline_residual_rmsnorm(h0, dev["z"], dev["gamma"], wl["eps"])
    y_unf = coda.coda_baseline_gemm(o, dev["w1"])
    sync()
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])["y"]
    e_f = errors(dec(y), ref)[0]
    e_u = errors(dec(y_unf), ref)[0]
    log(f"  y rel_fro fused={e_f:.4e} unfused={e_u:.4e}")
    assert_close("y_unfused", dec(y_unf), ref)
    assert e_f <= e_u * 1.02


# ------------------------------------------------------------------------------ row reduce
@pytest.mark.parametrize("nb", [1, 3, 16, 40, 100])
def test_rowstat_reduce(coda, nb):
    rng = np.random.default_rng(nb)
    M = 1000
    P = (rng.standard_normal((M, nb)) ** 2).astype(np.float32)
    Pd = to_dev_f32(P)
    d = 256 * nb - 17
    r = coda.coda_rowstat_reduce(Pd, d, 1e-5, coda.ROWSTAT_RSQRT_MEAN_EPS)
    s = coda.coda_rowstat_reduce(Pd, d, 0.0, coda.ROWSTAT_MEAN)
    sync()
    assert_close("r", r.cpu().numpy(), O.rowstat_reduce(P, d, 1e-5, "rsqrt_mean_eps"), rel_fro=1e-6)
    assert_close("s", s.cpu().numpy(), O.rowstat_reduce(P, d, 0.0, "mean"), rel_fro=1e-6)


@pytest.mark.parametrize("nb,M", [(4, 1), (4, 1031), (8, 777), (16, 8192), (16, 4099), (32, 300), (64, 1000),
                                  (12, 513)])
def test_rowstat_reduce_sum_order_is_sequential(coda, nb, M):
    """Every load layout sums a row in the order t = 0, 1, ..., nb-1 in fp32 (the
    contiguous-load form passes the running sum lane to lane): compared bit for bit with
    that sequential fp32 sum, here on the host; ragged M past a block."""
    rng = np.random.default_rng(100 + nb + M)
    P = (rng.standard_normal((M, nb)) ** 2).astype(np.float32)
    s = coda.coda_rowstat_reduce(to_dev_f32(P), 4096, 0.0, coda.ROWSTAT_MEAN)
    sync()
    acc = np.zeros(M, dtype=np.float32)
    for t in range(nb):
        acc = (acc + P[:, t]).astype(np.float32)
    want = (acc / np.float32(4096)).astype(np.float32)
    assert np.array_equal(s.cpu().numpy(), want)


def test_rowstat_reduce_ragged_partial_buffer_offset(coda):
    """A partials view that is only 4-byte aligned takes the scalar-load path."""
    import torch
    rng = np.random.default_rng(5)
    P = rng.random((130, 17)).astype(np.float32)
    buf = torch.zeros(130 * 17 + 1, dtype=torch.float32, device="cuda")
    buf[1:] = to_dev_f32(P.reshape(-1))
    view = buf[1:].view(130, 17)
    s = coda.coda_rowstat_reduce(view, 17, 0.0, coda.ROWSTAT_MEAN)
    sync()
    assert_close("s", s.cpu().numpy(), O.rowstat_reduce(P, 17, 0.0, "mean"), rel_fro=1e-6)


# ------------------------------------------------------------------------------------ RoPE
def test_rope_tables(coda):
    seq, hd, theta = 4096, 128, 10000.0
    c, s = coda.coda_rope_tables(seq, hd, theta)
    sync()
    ang = np.arange(seq)[:, None] * theta ** (-2.0 * np.arange(hd // 2)[None, :] / hd)
    assert np.max(np.abs(c.cpu().numpy() - np.cos(ang))) < 1e-7
    assert np.max(np.abs(s.cpu().numpy() - np.sin(ang))) < 1e-7


def run_rope(coda, wl):
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    out = coda.coda_gemm_rope(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, wl["n_q"], wl["n_k"], wl["n_v"],
                              wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    sync()
    return dec(out)


def oracle_rope(wl, rows=None):
    return O.gemm_rope(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                       wl["pos_offset"], wl["theta"], rows=rows)


@pytest.mark.parametrize("case", [
    dict(M=600, K=200, n_q=256, n_k=128, n_v=128, head_dim=128, seq_len=300, pos_offset=7),
    dict(M=70, K=64, n_q=64, n_k=64, n_v=64, head_dim=64, seq_len=70, pos_offset=0),
    dict(M=300, K=136, n_q=0, n_k=0, n_v=264, head_dim=8, seq_len=16, pos_offset=0),
])
def test_rope_small_full_compare(coda, case):
    log(f"rope {case}")
    wl = W.rope_qkv(seed=11, **case)
    assert_close("qkv", run_rope(coda, wl), oracle_rope(wl))


def test_rope_full_size(coda):
    wl = W.rope_qkv()
    log(f"rope {wl.name}")
    got = run_rope(coda, wl)
    ref = oracle_rope(wl)
    assert_close_tiles("qkv", got, ref)
    nqk = wl["n_q"] + wl["n_k"]
    assert_close("q", got[:, :wl["n_q"]], ref[:, :wl["n_q"]])
    assert_close("k", got[:, wl["n_q"]:nqk], ref[:, wl["n_q"]:nqk])
    assert_close("v", got[:, nqk:], ref[:, nqk:])


# ---------------------------------------------------------------------------------- SwiGLU
@pytest.mark.parametrize("shape", [(333, 136, 200), (256, 256, 128), (5, 64, 8)])
def test_swiglu_small_full_compare(coda, shape):
    M, K, F = shape
    log(f"swiglu M={M} K={K} F={F}")
    wl = W.swiglu(seed=12, M=M, K=K, F=F)
    out = coda.coda_gemm_swiglu(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]))
    sync()
    assert_close("swiglu", dec(out), O.gemm_swiglu(wl["x"], wl["w"]))


def test_swiglu_zero_gate_or_up_columns(coda):
    """A gate column of W that is zero gives G = 0 and silu(0) = 0; an up column that is
    zero gives U = 0: either way the output feature is exactly zero for every row. The
    features sit at both edges of an output tile (128 features per 256-column GEMM tile)
    and in the ragged last one; the rest matches the oracle."""
    M, K, F = 333, 136, 200
    wl = W.swiglu(seed=13, M=M, K=K, F=F)
    w = wl["w"].copy()
    gate_zero, up_zero = [0, 127, 128, F - 1], [5, 130]
    w[:, [2 * j for j in gate_zero]] = 0
    w[:, [2 * j + 1 for j in up_zero]] = 0
    out = dec(coda.coda_gemm_swiglu(to_dev_bf16(wl["x"]), to_dev_bf16(w)))
    sync()
    assert_close("swiglu", out, O.gemm_swiglu(wl["x"], w))
    assert not out[:, gate_zero + up_zero].any()


def test_swiglu_full_size(coda):
    wl = W.swiglu()
    log(f"swiglu {wl.name}")
    out = coda.coda_gemm_swiglu(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]))
    sync()
    # a 256-column GEMM tile gives 128 output features
    assert_close_tiles("swiglu", dec(out), O.gemm_swiglu(wl["x"], wl["w"]), tile_n=128)


def test_swiglu_4096_full_size(coda):
    wl = W.swiglu_4k()
    log(f"swiglu {wl.name}")
    out = coda.coda_gemm_swiglu(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]))
    sync()
    assert_close_tiles("swiglu", dec(out), O.gemm_swiglu(wl["x"], wl["w"]), tile_n=128)


# ----------------------------------------------------------------------- backward statistic
def run_bwd(coda, wl):
    dh2, part, s = coda.coda_gemm_rmsnorm_bwd_stats(to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w1"]),
                                                    to_dev_bf16(wl["h2"]))
    sync()
    return dec(dh2), part.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("shape", [(517, 392, 264), (256, 256, 256), (3, 16, 8)])
def test_bwd_small_full_compare(coda, shape):
    M, D, N = shape
    log(f"bwd M={M} D={D} N={N}")
    wl = W.bwd_stats(seed=13, M=M, D=D, N=N)
    dh2, part, s = run_bwd(coda, wl)
    ref = O.gemm_rmsnorm_bwd_stats(wl["dy"], wl["w1"], wl["h2"])
    assert_close("dh2", dh2, ref["dh2"])
    assert_close("partials", part, ref["partials"], rel_fro=TIGHT)
    assert_close("s", s, ref["s_prime"], rel_fro=TIGHT)


def test_bwd_full_size(coda):
    wl = W.bwd_stats()
    log(f"bwd {wl.name}")
    dh2, part, s = run_bwd(coda, wl)
    ref = O.gemm_rmsnorm_bwd_stats(wl["dy"], wl["w1"], wl["h2"])
    assert_close_tiles("dh2", dh2, ref["dh2"])
    assert_close_tiles("partials", part, ref["partials"], rel_fro=TIGHT, tile_n=1)
    # graded against (1/d) sum(dY * (h2 W1)), the right-hand form of the identity
    assert_close_tiles("s", s, ref["s_prime"], rel_fro=TIGHT)


# ------------------------------------------------------------------- exact integer results
def test_kn_large_weight_takes_per_step_descriptors(coda):
    """A KN weight with (K + 32) N >= 2^30 elements (2.1 GB here) is loaded through one W
    descriptor per depth step (one descriptor over the whole depth would need offsets past
    2^31). Ragged last depth step (K mod 32 = 8) and ragged last column tile (N mod 256 =
    8); sampled rows and columns against the oracle. The weight is drawn on the GPU from a
    seeded generator and only the sampled columns are brought to the host."""
    import torch
    M, K, N = 300, 32776, 32776
    assert (K + 32) * N >= 1 << 30
    gen = torch.Generator(device="cuda").manual_seed(1234)
    x = (torch.randn((M, K), generator=gen, device="cuda")).to(torch.bfloat16)
    w = (torch.randn((K, N), generator=gen, device="cuda") * K ** -0.5).to(torch.bfloat16)
    out = dec(coda.coda_baseline_gemm(x, w))
    sync()
    assert np.all(np.isfinite(out))
    rows = np.array([0, 1, 255, 256, M - 1])
    cols = np.array([0, 1, 255, 256, 16384, N - 9, N - 8, N - 1])
    ref = O.matmul(O.decode_bf16(bf16_bits(x[torch.from_numpy(rows).cuda()])),
                   O.decode_bf16(bf16_bits(w[:, torch.from_numpy(cols).cuda()])))
    assert_close("sampled", out[np.ix_(rows, cols)], ref)
    del w


def test_integer_inputs_are_bit_exact(coda):
    """Small integers (|v| <= 2, K <= 256) make every product and fp32 partial sum exact,
    so the bf16 outputs must equal the round-to-nearest-even of the exact result."""
    rng = np.random.default_rng(100)
    M, K, N = 300, 136, 264
    x = W.small_int_bf16(rng, (M, K), -2, 2)
    w = W.small_int_bf16(rng, (K, N), -2, 2)
    z = W.small_int_bf16(rng, (M, N), -3, 3)
    exact = O.matmul(x, w)
    want = W.f32_to_bf16_bits(exact.astype(np.float32))
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    kn = coda.coda_baseline_gemm(xd, wd, b_kn=True)
    nk = coda.coda_baseline_gemm(xd, to_dev_bf16(np.ascontiguousarray(w.T)), b_kn=False)
    c, s = coda.coda_rope_tables(16, 8)
    v_only = coda.coda_gemm_rope(xd, wd, c, s, 0, 0, N, 8, 16)
    gamma = W.small_int_bf16(rng, (N,), 1, 1)
    h1, h2, part = coda.coda_gemm_residual_rmsnorm_partials(xd, wd, to_dev_bf16(z), to_dev_bf16(gamma))
    sync()
    assert np.array_equal(bf16_bits(kn), want)
    assert np.array_equal(bf16_bits(nk), want)
    assert np.array_equal(bf16_bits(v_only), want)
    h1_exact = exact + O.decode_bf16(z)
    assert np.array_equal(bf16_bits(h1), W.f32_to_bf16_bits(h1_exact.astype(np.float32)))
    assert np.array_equal(bf16_bits(h2), W.f32_to_bf16_bits(h1_exact.astype(np.float32)))
    # the partial sums of squares of integers below 2^24 are exact in fp32 as well
    assert np.array_equal(part.cpu().numpy().astype(np.float64), O.tile_row_sums(h1_exact ** 2))


def test_integer_inputs_bwd_bit_exact(coda):
    rng = np.random.default_rng(101)
    M, D, N = 280, 264, 136
    dy = W.small_int_bf16(rng, (M, N), -2, 2)
    w1 = W.small_int_bf16(rng, (D, N), -2, 2)
    h2 = W.small_int_bf16(rng, (M, D), -2, 2)
    dh2, part, s = coda.coda_gemm_rmsnorm_bwd_stats(to_dev_bf16(dy), to_dev_bf16(w1), to_dev_bf16(h2))
    sync()
    ref = O.gemm_rmsnorm_bwd_stats(dy, w1, h2)
    assert np.array_equal(bf16_bits(dh2), W.f32_to_bf16_bits(ref["dh2"].astype(np.float32)))
    assert np.array_equal(part.cpu().numpy().astype(np.float64), ref["partials"])


# ----------------------------------------------------------------------------- error paths
def test_misaligned_pointer_is_rejected_and_writes_nothing(coda):
    import torch
    x = torch.zeros((64, 72), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.full((64, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        coda.coda_gemm_swiglu(x[:, 8:], w, out=out)   # non-contiguous view: rejected by the binding
    flat = torch.zeros(64 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    xm = flat[1:].view(64, 64)                          # contiguous but 2-byte aligned
    with pytest.raises(coda.CodaError) as e:
        coda.coda_gemm_swiglu(xm, w, out=out)
    assert e.value.status == 3
    sync()
    assert torch.all(out == 7.0)


def test_adjacent_outputs_and_aliased_inputs_are_accepted(coda):
    """Buffers that touch but do not overlap pass the overlap rule: h1, h2 and y carved
    back to back out of one allocation (and the partials and r likewise). Inputs may
    alias each other: the residual z is the same buffer as the GEMM1 input x (K = D).
    Results match the oracle."""
    import torch
    M, K, D, N1 = 300, 256, 256, 264
    wl = W.gemm_rmsnorm_fwd_inputs(61, M, K, D, N1, 1e-5)
    x = to_dev_bf16(wl["x"])
    w0, g, w1 = to_dev_bf16(wl["w0"]), to_dev_bf16(wl["gamma"]), to_dev_bf16(wl["w1"])
    big = torch.empty(2 * M * D + M * N1, dtype=torch.bfloat16, device="cuda")
    h1, h2, y = big[:M * D].view(M, D), big[M * D:2 * M * D].view(M, D), big[2 * M * D:].view(M, N1)
    fbuf = torch.empty(M * coda.num_partials(D) + M, dtype=torch.float32, device="cuda")
    part, r = fbuf[:M * coda.num_partials(D)].view(M, -1), fbuf[M * coda.num_partials(D):]
    coda.coda_gemm_rmsnorm_fwd(x, w0, x, g, w1, wl["eps"], h1=h1, h2=h2, partials=part, r=r, y=y)
    sync()
    check_fwd((h1, h2, part, r, y), O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["x"], wl["gamma"], wl["w1"], wl["eps"]))


def test_overlapping_output_is_rejected_and_writes_nothing(coda):
    import torch
    x = torch.ones((64, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((64, 64), dtype=torch.bfloat16, device="cuda")
    out = x.view(-1)[:64 * 32].view(64, 32)  # the output would overwrite the input
    with pytest.raises(coda.CodaError) as e:
        coda.coda_gemm_swiglu(x, w, out=out)
    assert e.value.status == 6
    sync()
    assert bool((x == 1).all())


def test_empty_batch_is_a_noop(coda):
    import torch
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 16), dtype=torch.bfloat16, device="cuda")
    out = coda.coda_gemm_swiglu(x, w)
    sync()
    assert out.shape == (0, 8)
