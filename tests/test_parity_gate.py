"""The parity gate itself (host logic, no GPU): the per-tile bound of assert_close_tiles
catches an error confined to one output tile that the whole-tensor bound misses, and a
tile whose reference is exactly zero must come out (near) zero."""
import numpy as np
import pytest

from gpu_util import assert_close, assert_close_tiles


def _pair(seed=0, shape=(700, 600), rel=1e-3):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal(shape)
    return ref * (1 + rel * rng.standard_normal(shape)), ref


def test_clean_result_passes_both_bounds():
    got, ref = _pair()
    assert_close_tiles("clean", got, ref)
    assert_close_tiles("clean rows", got[:, 0], ref[:, 0])


def test_one_bad_tile_fails_only_the_per_tile_bound():
    got, ref = _pair()
    bad = got.copy()
    bad[256:512, 256:512] *= 1.012     # one tile of nine 1.2% off
    assert_close("whole tensor", bad, ref)          # the whole-tensor bound misses it
    with pytest.raises(AssertionError, match="tiles above"):
        assert_close_tiles("one bad tile", bad, ref)


def test_zero_reference_tile_must_stay_zero():
    got, ref = _pair()
    ref[:256] = 0.0
    got[:256] = 0.0
    assert_close_tiles("zero rows", got, ref)
    got[3, 3] = 1.0
    with pytest.raises(AssertionError):
        assert_close_tiles("zero rows, one wrong", got, ref)
