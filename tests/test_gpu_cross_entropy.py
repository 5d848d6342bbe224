"""Parity of GEMM + cross-entropy (logits never stored; per-tile log-sum-exp partials,
the label logit, the auxiliary merge) with the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, log, to_dev_bf16

pytestmark = pytest.mark.gpu

TIGHT = 1e-4  # fp32 outputs against fp64: relative Frobenius bound


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def run(coda, wl):
    import torch
    labels = torch.from_numpy(wl["labels"]).cuda()
    loss, lse, target, tile = coda.coda_gemm_cross_entropy(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), labels)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), target.cpu().numpy(), tile.cpu().numpy()


@pytest.mark.parametrize("shape", [(300, 64, 600), (256, 256, 512), (517, 136, 1000), (3, 8, 8)])
def test_cross_entropy_small_full_compare(coda, shape):
    M, K, V = shape
    log(f"cross_entropy M={M} K={K} V={V}")
    wl = W.cross_entropy(seed=80 + M % 7, M=M, K=K, V=V, ignore_every=5)
    loss, lse, target, tile = run(coda, wl)
    ref = O.gemm_cross_entropy(wl["x"], wl["w"], wl["labels"])
    assert_close("tile_lse", tile, ref["tile_lse"], rel_fro=TIGHT)
    assert_close("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close("target", target, ref["target"], rel_fro=TIGHT)
    assert_close("loss", loss, ref["loss"], rel_fro=TIGHT)
    assert np.all(loss[~ref["valid"]] == 0) and np.all(target[~ref["valid"]] == 0)


def check_full(wl, got):
    loss, lse, target, tile = got
    ref = O.gemm_cross_entropy(wl["x"], wl["w"], wl["labels"])
    assert_close_tiles("tile_lse", tile, ref["tile_lse"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close_tiles("target", target, ref["target"], rel_fro=TIGHT)
    assert_close_tiles("loss", loss, ref["loss"], rel_fro=TIGHT)
    assert np.all(loss[~ref["valid"]] == 0) and np.all(target[~ref["valid"]] == 0)
    assert np.all(np.isfinite(loss)) and np.all(loss >= 0)


# the kernel table's two cross-entropy shapes (M x vocab x K), every row compared; every
# 97th row's label is ignored
def test_cross_entropy_full_size(coda):
    wl = W.cross_entropy(ignore_every=97)
    log(f"cross_entropy {wl.name}")
    check_full(wl, run(coda, wl))


def test_cross_entropy_8192_full_size(coda):
    wl = W.cross_entropy_8k(ignore_every=97)
    log(f"cross_entropy {wl.name}")
    check_full(wl, run(coda, wl))


def test_cross_entropy_deterministic_and_stages(coda):
    import torch
    wl = W.cross_entropy(seed=88, M=600, K=200, V=2056, ignore_every=9)
    a = run(coda, wl)
    b = run(coda, wl)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    # the merge entry point alone reproduces the loss from the epilogue's outputs
    loss, lse, target, tile = a
    t_target = torch.from_numpy(target).cuda()
    l2, lse2 = coda.coda_lse_reduce(torch.from_numpy(tile).cuda(), torch.from_numpy(wl["labels"]).cuda(), 2056,
                                    t_target)
    torch.cuda.synchronize()
    assert np.array_equal(l2.cpu().numpy(), loss) and np.array_equal(lse2.cpu().numpy(), lse)


def test_cross_entropy_large_logits(coda):
    # logits with sigma ~16 (row maxima near 50, exp would overflow-prone unshifted): finite, fp32-exact
    wl = W.cross_entropy(seed=89, M=256, K=64, V=512)
    from workloads import f32_to_bf16_bits
    x = O.decode_bf16(wl["x"]) * 16.0
    wl2 = dict(x=f32_to_bf16_bits(x.astype(np.float32)), w=wl["w"], labels=wl["labels"])
    loss, lse, target, tile = run(coda, wl2)
    ref = O.gemm_cross_entropy(wl2["x"], wl2["w"], wl2["labels"])
    assert np.all(np.isfinite(lse)) and np.max(np.abs(ref["lse"])) > 40
    assert_close("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close("loss", loss, ref["loss"], rel_fro=TIGHT)


# the merge alone, over widths that take every lane-chain instance (1 .. 32 partials per
# lane) and the thread-per-row form beyond 512 tiles, with row counts that leave partial
# 16-row groups; ignored labels on both sides of [0, V)
@pytest.mark.parametrize("nb", [1, 5, 16, 17, 32, 100, 128, 129, 256, 512, 513, 700])
def test_lse_merge_widths(coda, nb):
    import torch
    rng = np.random.default_rng(nb)
    V = 256 * nb - 8
    for M in (1, 37, 1000):
        log(f"lse merge nb={nb} M={M}")
        P = (rng.standard_normal((M, nb)) * 3.0).astype(np.float32)
        labels = rng.integers(-V // 2, V + V // 2, size=M).astype(np.int32)
        target = rng.standard_normal(M).astype(np.float32)
        t_target = torch.from_numpy(target.copy()).cuda()
        loss, lse = coda.coda_lse_reduce(torch.from_numpy(P).cuda(), torch.from_numpy(labels).cuda(), V, t_target)
        torch.cuda.synchronize()
        ref_lse = O.logsumexp_rows(P.astype(np.float64))
        valid = (labels >= 0) & (labels < V)
        assert_close("lse", lse.cpu().numpy(), ref_lse, rel_fro=2e-6)
        assert_close("loss", loss.cpu().numpy(), np.where(valid, ref_lse - target, 0.0), rel_fro=2e-6)
        assert np.array_equal(t_target.cpu().numpy(), np.where(valid, target, np.float32(0)))


def test_cross_entropy_zero_rows_closed_form(coda):
    """A row of x that is zero makes every logit of the row zero, so lse = log V, the label
    logit is 0 and the loss is log V (an ignored label: loss 0); the other rows match the
    oracle. Zero rows sit on a row-tile edge and in the ragged last tile; V spans a ragged
    last column tile."""
    M, K, V = 300, 64, 1000
    wl = W.cross_entropy(seed=91, M=M, K=K, V=V, ignore_every=0)
    x, labels = wl["x"].copy(), wl["labels"].copy()
    zero_rows = [0, 255, 256, M - 1]
    x[zero_rows] = 0
    labels[M - 1] = -1  # ignored
    loss, lse, target, _ = run(coda, dict(x=x, w=wl["w"], labels=labels))
    ref = O.gemm_cross_entropy(x, wl["w"], labels)
    assert_close("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close("loss", loss, ref["loss"], rel_fro=TIGHT)
    for m in zero_rows:
        assert abs(lse[m] - np.log(V)) <= 1e-6 * np.log(V), (m, lse[m])
        assert target[m] == 0.0
    for m in zero_rows[:-1]:
        assert abs(loss[m] - np.log(V)) <= 1e-6 * np.log(V), (m, loss[m])
    assert loss[M - 1] == 0.0
