"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties one oracle function to something other than its own formula: a
library routine computing the same textbook operation by a different route (torch's
rms_norm and autograd, scipy's logistic, numpy complex arithmetic), brute force on
tiny inputs, closed forms, invariants, or an identity the pages state. The last
section plants plausible mistakes into copies of oracle functions and checks that the
pins reject them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from workloads import f32_to_bf16_bits, gemm_rmsnorm_fwd_inputs, normal_bf16


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------------------- bf16
def test_decode_bf16_known_patterns():
    # Values fixed by the bf16 format (sign | 8-bit exponent, bias 127 | 7-bit fraction).
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0x3F00, 0x4049, 0x0001,
                     0x7F7F, 0x7F80, 0xFF80, 0x3C00], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, 0.5, 3.140625, 2.0 ** -133,
            (2 - 2.0 ** -7) * 2.0 ** 127, math.inf, -math.inf, 2.0 ** -7]
    got = O.decode_bf16(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[1]) == -1.0


def test_decode_bf16_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                       # drop inf/NaN patterns
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(O.decode_bf16(bits), t)


def test_input_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: RNE keeps the even mantissa (1.0).
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -9], np.float32)
    assert list(O.decode_bf16(f32_to_bf16_bits(v))) == [1.0, 1 + 2 * 2.0 ** -7 * 1, -1.0, 1.0]
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(v), t)


# ----------------------------------------------------------------------------- GEMM
def brute_matmul(a, b):
    M, K = a.shape
    K2, N = b.shape
    assert K == K2
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(a[i, k]) * float(b[k, j])
            out[i][j] = acc
    return np.array(out)


def test_matmul_brute_force():
    rng = np.random.default_rng(0)
    a = normal_bf16(rng, (5, 7), 1.0)
    b = normal_bf16(rng, (7, 3), 1.0)
    got = O.matmul(a, b)
    want = brute_matmul(O.decode_bf16(a), O.decode_bf16(b))
    assert got.shape == (5, 3)
    assert rel(got, want) < 1e-14


def test_matmul_shape_check():
    with pytest.raises(ValueError):
        O.matmul(np.zeros((4, 3)), np.zeros((4, 3)))


# ----------------------------------------------------------------- RMSNorm forward
def _small_fwd(seed=11, M=37, K=48, D=40, N1=24, eps=1e-5):
    return gemm_rmsnorm_fwd_inputs(seed, M, K, D, N1, eps)


def test_fwd_matches_torch_rms_norm():
    wl = _small_fwd()
    res = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    x, w0, z, g, w1 = (torch.from_numpy(O.decode_bf16(wl[k])) for k in ("x", "w0", "z", "gamma", "w1"))
    h1 = x @ w0 + z
    y = torch.nn.functional.rms_norm(h1, (h1.shape[1],), weight=g, eps=wl["eps"]) @ w1
    assert rel(res["h1"], h1.numpy()) < 1e-15
    assert rel(res["y"], y.numpy()) < 1e-13
    r_t = torch.rsqrt(h1.pow(2).mean(dim=1) + wl["eps"])
    assert rel(res["r"], r_t.numpy()) < 1e-14


def test_fwd_deferred_r_identity():
    # [notes] key design 1: the row scale commutes with the right matmul.
    wl = _small_fwd(seed=12, M=64, K=32, D=96, N1=80)
    res = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    assert rel(res["y_deferred"], res["y"]) < 1e-12
    # and the aux reduction of the partials reproduces r
    r2 = O.rowstat_reduce(res["partials"], 96, wl["eps"], "rsqrt_mean_eps")
    assert rel(r2, res["r"]) < 1e-14


def test_rmsnorm_closed_forms():
    eps = 1e-5
    g = np.ones(8)
    for c in (0.0, 0.25, 3.0, -7.5):
        r, out = O.rmsnorm_rows(np.full((1, 8), c), g, eps)
        assert r[0] == pytest.approx(1.0 / math.sqrt(c * c + eps), rel=1e-15)
    a = 2.5
    row = np.array([[a, -a, a, -a, -a, a, a, -a]])
    r, out = O.rmsnorm_rows(row, g, eps)
    assert r[0] == pytest.approx(1.0 / math.sqrt(a * a + eps), rel=1e-15)
    # eps = 0: every normalised row has unit RMS
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 33))
    _, out = O.rmsnorm_rows(h, np.ones(33), 0.0)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, rtol=1e-14)


@pytest.mark.parametrize("tile", [1, 7, 64, 256, 1000])
def test_partials_sum_to_full_row(tile):
    rng = np.random.default_rng(2)
    v = rng.standard_normal((9, 300)) ** 2
    P = O.tile_row_sums(v, tile)
    assert P.shape == (9, -(-300 // tile))
    assert np.allclose(P.sum(axis=1), v.sum(axis=1), rtol=1e-13)
    # last ragged tile holds exactly the remaining columns
    last = (P.shape[1] - 1) * tile
    assert np.allclose(P[:, -1], v[:, last:].sum(axis=1), rtol=1e-14)


def test_rowstat_reduce_closed_form():
    P = np.array([[1.0, 2.0, 3.0, 4.0], [0.0, 0.0, 0.0, 0.0]])
    r = O.rowstat_reduce(P, d=5, eps=0.5, mode="rsqrt_mean_eps")
    assert r[0] == pytest.approx(1 / math.sqrt(10 / 5 + 0.5), rel=1e-15)
    assert r[1] == pytest.approx(1 / math.sqrt(0.5), rel=1e-15)
    s = O.rowstat_reduce(P, d=4, mode="mean")
    assert list(s) == [2.5, 0.0]


def test_row_sampling_equals_full():
    wl = _small_fwd(seed=13, M=50)
    full = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    rows = np.array([0, 7, 49, 23])
    part = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"], rows=rows)
    for k in ("h1", "h2", "partials", "r", "y"):
        assert np.allclose(part[k], full[k][rows], rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------- RoPE
def _rope_case(seed=3, M=20, K=16, n_q=16, n_k=8, n_v=8, head_dim=8):
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    w = normal_bf16(rng, (K, n_q + n_k + n_v), 0.25)
    return x, w, dict(n_q=n_q, n_k=n_k, n_v=n_v, head_dim=head_dim)


def test_rope_matches_complex_form():
    # RoFormer's complex form: (e + i o) * exp(i * pos * theta^(-2p/d)).
    x, w, p = _rope_case()
    seq_len, off, theta = 13, 5, 10000.0
    out = O.gemm_rope(x, w, seq_len=seq_len, pos_offset=off, theta=theta, **p)
    h = O.matmul(x, w)
    hd = p["head_dim"]
    pos = (np.arange(h.shape[0]) + off) % seq_len
    for c0 in range(0, p["n_q"] + p["n_k"], hd):
        for q in range(hd // 2):
            zc = h[:, c0 + 2 * q] + 1j * h[:, c0 + 2 * q + 1]
            rot = zc * np.exp(1j * pos * theta ** (-2.0 * q / hd))
            assert np.allclose(out[:, c0 + 2 * q], rot.real, rtol=0, atol=1e-13)
            assert np.allclose(out[:, c0 + 2 * q + 1], rot.imag, rtol=0, atol=1e-13)


def test_rope_invariants():
    x, w, p = _rope_case(seed=4)
    out = O.gemm_rope(x, w, seq_len=1000, **p)
    h = O.matmul(x, w)
    nqk = p["n_q"] + p["n_k"]
    # V passes through, row 0 (pos 0) is the identity
    assert np.array_equal(out[:, nqk:], h[:, nqk:])
    assert np.allclose(out[0], h[0], rtol=0, atol=1e-15)
    # pair norms are preserved
    e, o = out[:, 0:nqk:2], out[:, 1:nqk:2]
    he, ho = h[:, 0:nqk:2], h[:, 1:nqk:2]
    assert np.allclose(e ** 2 + o ** 2, he ** 2 + ho ** 2, rtol=1e-12)


def test_rope_relative_position():
    # <R_m q, R_n k> depends only on m - n.
    hd, theta = 16, 10000.0
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, hd))
    k = rng.standard_normal((1, hd))
    def rot(v, pos):
        return O.rope_rotate(v, np.array([pos]), hd, 0, 0, hd, theta)
    base = (rot(q, 9) @ rot(k, 4).T).item()
    for shift in (1, 17, 300):
        assert (rot(q, 9 + shift) @ rot(k, 4 + shift).T).item() == pytest.approx(base, rel=1e-11)
    assert (rot(q, 9) @ rot(k, 5).T).item() != pytest.approx(base, rel=1e-6)


def test_rope_frequency_per_pair():
    # Pair p at position 1 turns the unit vector (1, 0) by exactly theta^(-2p/d) rad.
    hd, theta = 128, 10000.0
    v = np.zeros((1, hd))
    v[0, 0::2] = 1.0
    out = O.rope_rotate(v, np.array([1]), hd, 0, 0, hd, theta)
    ang = np.arctan2(out[0, 1::2], out[0, 0::2])
    want = theta ** (-np.arange(hd // 2) * 2.0 / hd)
    assert np.allclose(ang, want, rtol=1e-14, atol=0)
    assert ang[0] == pytest.approx(1.0, rel=1e-15)       # pair 0 turns by 1 rad


# --------------------------------------------------------------------------- SwiGLU
def test_silu_pins():
    g = np.linspace(-30, 30, 601)
    assert np.allclose(O.silu(g), g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-15)
    assert abs(O.silu(np.array([-60.0]))[0]) < 1e-24
    assert O.silu(np.array([-1e6]))[0] == 0.0


def test_swiglu_compaction_one_hot():
    # W's column 2j picks x[:, a_j] (gate) and 2j+1 picks x[:, b_j] (up).
    rng = np.random.default_rng(7)
    M, K, F = 6, 10, 4
    x = normal_bf16(rng, (M, K), 1.0)
    a = [3, 0, 9, 3]
    b = [1, 1, 4, 8]
    W = np.zeros((K, 2 * F))
    for j in range(F):
        W[a[j], 2 * j] = 1.0
        W[b[j], 2 * j + 1] = 1.0
    out = O.gemm_swiglu(x, W)
    xf = O.decode_bf16(x)
    assert out.shape == (M, F)
    for j in range(F):
        g = xf[:, a[j]]
        assert np.allclose(out[:, j], g * scipy.special.expit(g) * xf[:, b[j]], rtol=1e-14)


# --------------------------------------------------------------- backward statistic
def _bwd_case(seed=8, M=24, D=40, N=36):
    rng = np.random.default_rng(seed)
    return (normal_bf16(rng, (M, N), 0.1), normal_bf16(rng, (D, N), 1 / math.sqrt(D)),
            normal_bf16(rng, (M, D), 1.0))


def test_bwd_three_forms_equal():
    dy, w1, h2 = _bwd_case()
    res = O.gemm_rmsnorm_bwd_stats(dy, w1, h2)
    assert rel(res["s_prime"], res["s"]) < 1e-12
    assert rel(res["s_diag"], res["s"]) < 1e-12
    assert np.allclose(res["partials"].sum(axis=1) / 40, res["s"], rtol=1e-13)


def test_bwd_matches_autograd():
    dy, w1, h2 = _bwd_case(seed=9)
    res = O.gemm_rmsnorm_bwd_stats(dy, w1, h2)
    H2 = torch.from_numpy(O.decode_bf16(h2)).requires_grad_(True)
    W1 = torch.from_numpy(O.decode_bf16(w1))
    (H2 @ W1).backward(torch.from_numpy(O.decode_bf16(dy)))
    assert rel(res["dh2"], H2.grad.numpy()) < 1e-14
    s_t = (H2.grad * H2.detach()).sum(dim=1) / H2.shape[1]
    assert rel(res["s"], s_t.numpy()) < 1e-13


def test_s_is_the_rmsnorm_backward_statistic():
    # With o = RMSNorm(h1, gamma) = r h1 * gamma, autograd's input gradient must equal
    # r (gamma * g) - r^2 s h1, where g = dY W1^T is the gradient reaching o and
    # s = (1/d) sum(g * o) is the oracle's statistic with h2 := o.
    rng = np.random.default_rng(10)
    M, D, N, eps = 8, 16, 12, 1e-5
    h1 = torch.from_numpy(rng.standard_normal((M, D))).requires_grad_(True)
    gamma = torch.from_numpy(1 + 0.1 * rng.standard_normal(D))
    w1 = rng.standard_normal((D, N)) / 4
    dy = rng.standard_normal((M, N)) * 0.1
    o = torch.nn.functional.rms_norm(h1, (D,), weight=gamma, eps=eps)
    g = torch.from_numpy(dy) @ torch.from_numpy(w1).T
    o.backward(g)
    res = O.gemm_rmsnorm_bwd_stats(dy, w1, o.detach().numpy())
    r = 1 / torch.sqrt(h1.detach().pow(2).mean(dim=1) + eps)
    s = torch.from_numpy(res["s"])
    want = r[:, None] * (gamma * g) - (r * r * s)[:, None] * h1.detach()
    assert rel(h1.grad.numpy(), want.numpy()) < 1e-12
    assert rel(res["dh2"], g.numpy()) < 1e-14


# ---------------------------------------------------- planted mistakes are rejected
def _fwd_pin_holds(fwd) -> bool:
    wl = _small_fwd(seed=21, M=16, K=24, D=40, N1=8)
    res = fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    x, w0, z, g, w1 = (torch.from_numpy(O.decode_bf16(wl[k])) for k in ("x", "w0", "z", "gamma", "w1"))
    h1 = x @ w0 + z
    y = torch.nn.functional.rms_norm(h1, (h1.shape[1],), weight=g, eps=wl["eps"]) @ w1
    return rel(res["y"], y.numpy()) < 1e-10 and rel(res["y_deferred"], y.numpy()) < 1e-10


def test_planted_fwd_mistakes_fail_pin():
    assert _fwd_pin_holds(O.gemm_rmsnorm_fwd)

    def eps_outside(x, w0, z, gamma, w1, eps):
        h1 = O.matmul(x, w0) + O.decode_bf16(z)
        r = 1 / (np.sqrt(np.mean(h1 ** 2, axis=1)) + eps * 1e3)
        y = O.matmul((r[:, None] * h1) * O.decode_bf16(gamma), w1)
        return dict(y=y, y_deferred=y)

    def gamma_twice(x, w0, z, gamma, w1, eps):
        res = O.gemm_rmsnorm_fwd(x, w0, z, gamma, w1, eps)
        g = O.decode_bf16(gamma)
        return dict(y=O.matmul(res["h2"] * g * res["r"][:, None], w1), y_deferred=res["y_deferred"])

    def no_residual(x, w0, z, gamma, w1, eps):
        return O.gemm_rmsnorm_fwd(x, w0, np.zeros_like(z), gamma, w1, eps)

    for bad in (eps_outside, gamma_twice, no_residual):
        assert not _fwd_pin_holds(bad), bad.__name__


def test_planted_rope_sign_flip_fails_pin():
    x, w, p = _rope_case(seed=22)
    good = O.gemm_rope(x, w, seq_len=50, **p)
    flipped = O.rope_rotate(O.matmul(x, w), -np.arange(x.shape[0]), p["n_q"], p["n_k"], p["n_v"],
                            p["head_dim"], 10000.0)
    h = O.matmul(x, w)
    pos = np.arange(h.shape[0])
    zc = h[:, 0] + 1j * h[:, 1]
    rot = zc * np.exp(1j * pos)
    assert np.allclose(good[:, 0], rot.real, atol=1e-13)
    assert not np.allclose(flipped[:, 0], rot.real, atol=1e-6)


def test_planted_bwd_transpose_fails_pin():
    dy, w1, h2 = _bwd_case(seed=23, M=12, D=20, N=20)   # square W1 so a transpose still runs
    H2 = torch.from_numpy(O.decode_bf16(h2)).requires_grad_(True)
    W1 = torch.from_numpy(O.decode_bf16(w1))
    (H2 @ W1).backward(torch.from_numpy(O.decode_bf16(dy)))
    wrong = O.matmul(dy, O.decode_bf16(w1))        # dY W1 instead of dY W1^T
    assert rel(O.gemm_rmsnorm_bwd_stats(dy, w1, h2)["dh2"], H2.grad.numpy()) < 1e-14
    assert rel(wrong, H2.grad.numpy()) > 0.1


# ------------------------------------------- rest of the RMSNorm backward (reading R8)
def _rbwd_case(seed=30, M=40, D=48, N=36):
    rng = np.random.default_rng(seed)
    return dict(h1=normal_bf16(rng, (M, D), 1.0), gamma=normal_bf16(rng, (D,), 0.1, 1.0),
                w1=normal_bf16(rng, (D, N), 1 / math.sqrt(D)), dy=normal_bf16(rng, (M, N), 0.1),
                g_res=normal_bf16(rng, (M, D), 0.1), eps=1e-5)


def _rbwd(c, **kw):
    return O.rmsnorm_bwd(c["h1"], c["gamma"], c["w1"], c["dy"], c["eps"], g_res=c["g_res"], **kw)


def _autograd_rmsnorm_bwd(c):
    # torch's rms_norm (a library routine) then the GEMM; the residual stream adds
    # g_res . h1 to the loss, so its gradient reaches h1 unchanged.
    h1 = torch.from_numpy(O.decode_bf16(c["h1"])).requires_grad_(True)
    g = torch.from_numpy(O.decode_bf16(c["gamma"])).requires_grad_(True)
    w1 = torch.from_numpy(O.decode_bf16(c["w1"]))
    y = torch.nn.functional.rms_norm(h1, (h1.shape[1],), weight=g, eps=c["eps"]) @ w1
    loss = (y * torch.from_numpy(O.decode_bf16(c["dy"]))).sum() + \
        (h1 * torch.from_numpy(O.decode_bf16(c["g_res"]))).sum()
    loss.backward()
    return h1.grad.numpy(), g.grad.numpy(), y.detach().numpy()


def test_rmsnorm_bwd_matches_autograd():
    c = _rbwd_case()
    dh1, dg, y = _autograd_rmsnorm_bwd(c)
    res = _rbwd(c)
    assert rel(res["dh1"], dh1) < 1e-12
    assert rel(res["dgamma"], dg) < 1e-12
    assert rel(res["y"], y) < 1e-13
    assert rel(res["s_out"], res["s"]) < 1e-12   # key design 3: the statistic from dY . y


def test_rmsnorm_bwd_row_col_sampling_and_tile_partials():
    c = _rbwd_case(seed=31, M=600, D=24, N=20)
    full = _rbwd(c)
    rows = np.array([0, 5, 255, 256, 599])
    sub = _rbwd(c, rows=rows)
    for k in ("r", "s", "s_out", "dh1"):
        assert np.allclose(sub[k], full[k][rows], rtol=1e-13, atol=0), k
    cols = np.array([0, 7, 23])
    sc = _rbwd(c, cols=cols)
    assert np.allclose(sc["dgamma"], full["dgamma"][cols], rtol=1e-13, atol=1e-15)
    # 3 row tiles of 256 (the last one ragged, 88 rows) add up to dgamma
    assert full["dgamma_partials"].shape == (3, 24)
    assert np.allclose(full["dgamma_partials"].sum(axis=0), full["dgamma"], rtol=1e-13, atol=1e-15)
    # brute force of the ragged tile: plain Python loops over rows 512..599, column 7
    H1, G, W1, DY = (O.decode_bf16(c[k]) for k in ("h1", "gamma", "w1", "dy"))
    acc = 0.0
    for m in range(512, 600):
        ms = sum(float(v) * float(v) for v in H1[m]) / 24
        r = 1.0 / math.sqrt(ms + c["eps"])
        dO = sum(float(DY[m, j]) * float(W1[7, j]) for j in range(20))
        acc += dO * r * float(H1[m, 7])
    assert abs(full["dgamma_partials"][2, 7] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_planted_rmsnorm_bwd_mistakes_fail_pin():
    c = _rbwd_case(seed=32)
    dh1, dg, _ = _autograd_rmsnorm_bwd(c)
    res = _rbwd(c)
    r, s, dO = res["r"], res["s"], res["dO"]
    H1, G, GR = (O.decode_bf16(c[k]) for k in ("h1", "gamma", "g_res"))
    assert rel(res["dh1"], dh1) < 1e-12
    planted = {
        "r^3 in the statistic term": r[:, None] * G * dO - (r ** 3 * s)[:, None] * H1 + GR,
        "gamma dropped": r[:, None] * dO - (r * r * s)[:, None] * H1 + GR,
        "residual gradient dropped": r[:, None] * G * dO - (r * r * s)[:, None] * H1,
    }
    for name, bad in planted.items():
        assert rel(bad, dh1) > 1e-3, name
    assert rel((dO * H1).sum(axis=0), dg) > 1e-3          # dgamma without r


# ------------------------------------------------------- SwiGLU and RoPE backward (R9, R10)
def _swiglu_bwd_case(seed=40, M=24, Dm=20, F=18):
    rng = np.random.default_rng(seed)
    return (normal_bf16(rng, (M, Dm), 0.1), normal_bf16(rng, (F, Dm), 1 / math.sqrt(F)),
            normal_bf16(rng, (M, 2 * F), 1.0))


def _swiglu_autograd(dy, w_down, h):
    # torch's silu (a library routine): out = silu(G) U, then the down projection
    H = torch.from_numpy(O.decode_bf16(h)).requires_grad_(True)
    out = torch.nn.functional.silu(H[:, 0::2]) * H[:, 1::2]
    y = out @ torch.from_numpy(O.decode_bf16(w_down))
    y.backward(torch.from_numpy(O.decode_bf16(dy)))
    return H.grad.numpy()


def test_swiglu_bwd_matches_autograd():
    dy, w_down, h = _swiglu_bwd_case()
    res = O.gemm_swiglu_bwd(dy, w_down, h)
    assert rel(res["dh"], _swiglu_autograd(dy, w_down, h)) < 1e-13


def test_silu_grad_pins():
    g = np.array([-30.0, -2.5, -1e-3, 0.0, 1e-3, 0.7, 3.0, 30.0])
    # central difference of scipy's logistic-based silu
    e = 1e-6
    fd = ((g + e) * scipy.special.expit(g + e) - (g - e) * scipy.special.expit(g - e)) / (2 * e)
    assert np.allclose(O.silu_grad(g), fd, rtol=1e-7, atol=1e-9)
    assert O.silu_grad(np.array([0.0]))[0] == 0.5        # s(0) = 1/2
    assert abs(O.silu_grad(np.array([40.0]))[0] - 1.0) < 1e-12 and abs(O.silu_grad(np.array([-40.0]))[0]) < 1e-12


def test_swiglu_bwd_rows_and_planted_mistakes():
    dy, w_down, h = _swiglu_bwd_case(seed=41, M=30)
    full = O.gemm_swiglu_bwd(dy, w_down, h)
    rows = np.array([0, 7, 29])
    sub = O.gemm_swiglu_bwd(dy, w_down, h, rows=rows)
    assert np.allclose(sub["dh"], full["dh"][rows], rtol=1e-13, atol=0)
    want = _swiglu_autograd(dy, w_down, h)
    G, U = O.decode_bf16(h)[:, 0::2], O.decode_bf16(h)[:, 1::2]
    d = full["dout"]
    sig = scipy.special.expit(G)
    for name, dG, dU in (("silu' = s(g) only", d * U * sig, d * G * sig),
                         ("gate and up swapped", d * G * O.silu_grad(U), d * O.silu(U))):
        bad = np.empty_like(full["dh"])
        bad[:, 0::2], bad[:, 1::2] = dG, dU
        assert rel(bad, want) > 1e-3, name


def _torch_rope(h, pos, head_dim, theta):
    # RoPE as a complex multiplication built from torch.polar (library routines)
    M, W_ = h.shape
    half = head_dim // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / head_dim)
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)                      # e^{i a}
    z = torch.view_as_complex(h.reshape(M, W_ // head_dim, half, 2).contiguous())
    return torch.view_as_real(z * rot[:, None, :]).reshape(M, W_)


def test_rope_bwd_matches_autograd_and_inverts_forward():
    rng = np.random.default_rng(42)
    M, hd, nq, nk, nv = 9, 8, 16, 8, 8
    h = rng.standard_normal((M, nq + nk + nv))
    pos = (np.arange(M) + 3) % 7
    H = torch.from_numpy(h).requires_grad_(True)
    qk = _torch_rope(H[:, :nq + nk], pos, hd, 10000.0)
    g = torch.from_numpy(rng.standard_normal((M, nq + nk + nv)))
    (torch.cat([qk, H[:, nq + nk:]], dim=1) * g).sum().backward()
    # the oracle's backward with the identity as GEMM operand reproduces autograd
    got = O.gemm_rope_bwd(f32_to_bf16_bits(np.eye(M, dtype=np.float32)), g.numpy(), nq, nk, nv, hd, seq_len=7,
                          pos_offset=3)
    assert rel(got, H.grad.numpy()) < 1e-13
    # backward after forward is the identity on every pair (an orthogonal rotation)
    fwd = O.rope_rotate(h, pos, nq, nk, nv, hd, 10000.0)
    assert rel(O.rope_rotate(fwd, -pos, nq, nk, nv, hd, 10000.0), h) < 1e-14
    # planted: the forward sign in the backward is rejected
    wrong = O.rope_rotate(g.numpy(), pos, nq, nk, nv, hd, 10000.0)
    assert rel(wrong, H.grad.numpy()) > 1e-2


# ------------------------------------------------------------- GEMM + cross-entropy (R11)
def _ce_case(seed=50, M=30, K=24, V=600):
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    w = normal_bf16(rng, (K, V), 1 / math.sqrt(K))
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[3] = -1          # ignored
    labels[4] = V           # out of range: ignored
    return x, w, labels


def test_cross_entropy_matches_torch_and_scipy():
    x, w, labels = _ce_case()
    res = O.gemm_cross_entropy(x, w, labels)
    z = O.matmul(x, w)
    assert rel(res["lse"], scipy.special.logsumexp(z, axis=1)) < 1e-14
    lab = torch.from_numpy(labels.astype(np.int64))
    want = torch.nn.functional.cross_entropy(torch.from_numpy(z), lab.clamp(0, z.shape[1] - 1), reduction="none")
    valid = (labels >= 0) & (labels < z.shape[1])
    assert rel(res["loss"][valid], want.numpy()[valid]) < 1e-14
    assert np.all(res["loss"][~valid] == 0) and np.all(res["target"][~valid] == 0)


def test_cross_entropy_tile_partials_merge_and_closed_forms():
    x, w, labels = _ce_case(seed=51, M=12, V=600)   # 3 tiles of 256, the last ragged (88)
    res = O.gemm_cross_entropy(x, w, labels)
    assert res["tile_lse"].shape == (12, 3)
    z = O.matmul(x, w)
    for t, (a, b) in enumerate(((0, 256), (256, 512), (512, 600))):
        assert rel(res["tile_lse"][:, t], scipy.special.logsumexp(z[:, a:b], axis=1)) < 1e-14
    assert rel(scipy.special.logsumexp(res["tile_lse"], axis=1), res["lse"]) < 1e-14
    # constant logits c over V columns: lse = c + log V, loss = log V
    const = np.full((2, 600), 3.25)
    assert np.allclose(O.logsumexp_rows(const), 3.25 + math.log(600), rtol=1e-15)
    # row sampling equals slicing
    sub = O.gemm_cross_entropy(x, w, labels, rows=np.array([0, 5, 11]))
    assert np.allclose(sub["loss"], res["loss"][[0, 5, 11]], rtol=1e-13, atol=0)


def test_planted_cross_entropy_mistakes_fail_pin():
    x, w, labels = _ce_case(seed=52)
    z = O.matmul(x, w)
    valid = (labels >= 0) & (labels < z.shape[1])
    lab = torch.from_numpy(np.clip(labels, 0, z.shape[1] - 1).astype(np.int64))
    want = torch.nn.functional.cross_entropy(torch.from_numpy(z), lab, reduction="none").numpy()[valid]
    res = O.gemm_cross_entropy(x, w, labels)
    idx = np.arange(z.shape[0])
    off_by_one = res["lse"] - z[idx, np.clip(labels + 1, 0, z.shape[1] - 1)]
    no_log = np.exp(res["lse"]) - res["target"]
    tiles_summed = res["tile_lse"].sum(axis=1) - res["target"]      # adding tile lse instead of merging
    for bad in (off_by_one, no_log, tiles_summed):
        assert rel(bad[valid], want) > 1e-3
