"""Parity of the pairwise backward epilogues (SwiGLU backward on the down projection's
grad GEMM, RoPE backward as the inverse rotation) with the fp64 oracle, through the C
ABI: small ragged cases element by element, the full-size workloads on sampled rows."""
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


# ----------------------------------------------------------------------- SwiGLU backward
def run_swiglu_bwd(coda, wl):
    dh = coda.coda_gemm_swiglu_bwd(to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w_down"]), to_dev_bf16(wl["h"]))
    sync()
    return dec(dh)


@pytest.mark.parametrize("shape", [(333, 200, 136), (256, 256, 128), (5, 64, 8), (700, 328, 264)])
def test_swiglu_bwd_small_full_compare(coda, shape):
    M, Dm, F = shape
    log(f"swiglu_bwd M={M} Dm={Dm} F={F}")
    wl = W.swiglu_bwd(seed=70 + M % 13, M=M, Dm=Dm, F=F)
    got = run_swiglu_bwd(coda, wl)
    ref = O.gemm_swiglu_bwd(wl["dy"], wl["w_down"], wl["h"])["dh"]
    assert_close("dG", got[:, 0::2], ref[:, 0::2])
    assert_close("dU", got[:, 1::2], ref[:, 1::2])


def test_swiglu_bwd_zero_rows_and_gates(coda):
    """Zero rows of dY give exactly zero gradient rows; a saved gate G = 0 has silu(G) = 0,
    so the up-gradient dU = dOut silu(G) of that feature is exactly zero in every row (and
    dG = dOut U / 2 is the oracle's). Zero rows on a row-tile edge and in the ragged last
    tile; zero gates at both ends of the ragged feature tile and inside it."""
    M, Dm, F = 333, 200, 136
    wl0 = W.swiglu_bwd(seed=78, M=M, Dm=Dm, F=F)
    wl = {k: wl0[k].copy() for k in ("dy", "w_down", "h")}
    zero_rows, zero_gates = [0, 255, 256, M - 1], [0, 127, 128, F - 1]
    wl["dy"][zero_rows] = 0
    wl["h"][:, [2 * j for j in zero_gates]] = 0
    got = run_swiglu_bwd(coda, wl)
    ref = O.gemm_swiglu_bwd(wl["dy"], wl["w_down"], wl["h"])["dh"]
    assert_close("dG", got[:, 0::2], ref[:, 0::2])
    assert_close("dU", got[:, 1::2], ref[:, 1::2])
    assert not got[zero_rows].any()
    assert not got[:, [2 * j + 1 for j in zero_gates]].any()


def test_swiglu_bwd_saturated_gates(coda):
    # gates far into both tails of the logistic (|G| up to ~40): finite, and still the oracle's values
    wl = W.swiglu_bwd(seed=77, M=300, Dm=64, F=128)
    h = O.decode_bf16(wl["h"]) * 12.0
    from workloads import f32_to_bf16_bits
    hb = f32_to_bf16_bits(h.astype(np.float32))
    wl2 = dict(dy=wl["dy"], w_down=wl["w_down"], h=hb)
    got = run_swiglu_bwd(coda, wl2)
    ref = O.gemm_swiglu_bwd(wl2["dy"], wl2["w_down"], wl2["h"])["dh"]
    assert np.all(np.isfinite(got))
    assert_close("dh", got, ref)


def test_swiglu_bwd_full_size(coda):
    wl = W.swiglu_bwd()
    log(f"swiglu_bwd {wl.name}")
    got = run_swiglu_bwd(coda, wl)
    ref = O.gemm_swiglu_bwd(wl["dy"], wl["w_down"], wl["h"])["dh"]
    # a 256-feature GEMM tile of dOut gives 512 interleaved (dG, dU) columns
    assert_close_tiles("dh", got, ref, tile_n=512)


# ------------------------------------------------------------------------- RoPE backward
def run_rope_bwd(coda, wl):
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    out = coda.coda_gemm_rope_bwd(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, wl["n_q"], wl["n_k"], wl["n_v"],
                                  wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    sync()
    return dec(out)


def oracle_rope_bwd(wl, rows=None):
    return O.gemm_rope_bwd(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                           wl["pos_offset"], wl["theta"], rows=rows)


@pytest.mark.parametrize("case", [
    dict(M=600, K=200, n_q=256, n_k=128, n_v=128, head_dim=128, seq_len=300, pos_offset=7),
    dict(M=70, K=64, n_q=64, n_k=64, n_v=64, head_dim=64, seq_len=70, pos_offset=5),
])
def test_rope_bwd_small_full_compare(coda, case):
    log(f"rope_bwd {case}")
    wl = W.rope_bwd(seed=13, **case)
    assert_close("dqkv", run_rope_bwd(coda, wl), oracle_rope_bwd(wl))


def test_rope_bwd_full_size(coda):
    wl = W.rope_bwd()
    log(f"rope_bwd {wl.name}")
    got = run_rope_bwd(coda, wl)
    ref = oracle_rope_bwd(wl)
    nqk = wl["n_q"] + wl["n_k"]
    assert_close_tiles("dqkv", got, ref)
    assert_close("dq", got[:, :wl["n_q"]], ref[:, :wl["n_q"]])
    assert_close("dk", got[:, wl["n_q"]:nqk], ref[:, wl["n_q"]:nqk])
    assert_close("dv", got[:, nqk:], ref[:, nqk:])


def test_rope_bwd_rotation_properties(coda):
    # the forward and backward epilogues of the same GEMM: both keep every pair's norm,
    # and they differ (the angle's sign)
    wl = W.rope_bwd(seed=14, M=256, K=64, n_q=128, n_k=128, n_v=0, head_dim=64, seq_len=256, pos_offset=3)
    import transformer_gemm_epilogue_amd as c
    cos_t, sin_t = c.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    x, w = to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"])
    args = (wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    fwd = dec(c.coda_gemm_rope(x, w, cos_t, sin_t, *args))
    bwd = dec(c.coda_gemm_rope_bwd(x, w, cos_t, sin_t, *args))
    plain = O.matmul(wl["x"], wl["w"])
    # each pair keeps its norm under both rotations
    for out in (fwd, bwd):
        n_out = out[:, 0::2] ** 2 + out[:, 1::2] ** 2
        n_ref = plain[:, 0::2] ** 2 + plain[:, 1::2] ** 2
        assert np.allclose(n_out, n_ref, rtol=2e-2, atol=1e-4)
    assert not np.allclose(fwd, bwd, atol=1e-3)


def test_rope_position_zero_is_identity(coda):
    """At position 0 every pair's angle is zero (the table holds cos 1 and sin 0 exactly),
    so those rows of the fused output, forward and backward, equal the plain-store GEMM of
    the same main loop bit for bit; the V block passes through unrotated at every row."""
    c = coda
    wl = W.rope_qkv(seed=21, M=600, K=128, n_q=256, n_k=128, n_v=128, head_dim=64, seq_len=256, pos_offset=0)
    cos_t, sin_t = c.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    assert np.all(cos_t[0].cpu().numpy() == 1.0) and np.all(sin_t[0].cpu().numpy() == 0.0)
    x, w = to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"])
    args = (wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    fwd = bf16_bits(c.coda_gemm_rope(x, w, cos_t, sin_t, *args))
    bwd = bf16_bits(c.coda_gemm_rope_bwd(x, w, cos_t, sin_t, *args))
    plain = bf16_bits(c.coda_baseline_gemm(x, w))
    rows = [0, 256, 512]  # (m + pos_offset) mod seq_len == 0, one in the ragged last row tile
    qk = wl["n_q"] + wl["n_k"]
    for out in (fwd, bwd):
        assert np.array_equal(out[rows], plain[rows])
        assert np.array_equal(out[:, qk:], plain[:, qk:])
        assert not np.array_equal(out[1:256, :qk], plain[1:256, :qk])  # other positions do rotate
