"""Helpers shared by the GPU tests: host<->device marshalling of bf16 bit arrays and the
parity gate. Test infrastructure: it may use both the oracle and the HIP binding."""
from __future__ import annotations

import sys

import numpy as np

# Parity gate for bf16-in / fp32-accumulate results against the fp64 oracle: relative
# Frobenius error <= 5e-3 and max abs error <= 2e-2 * max |ref|. One bf16 rounding costs
# about 2^-9 / sqrt(3) ~ 1.1e-3 relative RMS, and the deepest output (y) carries two
# roundings plus fp32 accumulation, ~2.5e-3: the gate leaves ~2x headroom.
REL_FRO = 5e-3
MAX_ABS = 2e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_dev_f32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def bf16_bits(t) -> np.ndarray:
    """Device bf16 tensor -> host uint16 bit patterns."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    rel_fro = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    max_ref = float(np.max(np.abs(ref))) if ref.size else 0.0
    return rel_fro, max_abs, max_ref


def assert_close(name: str, got, ref, rel_fro=REL_FRO, max_abs_frac=MAX_ABS):
    rf, ma, mr = errors(got, ref)
    log(f"  {name}: rel_fro={rf:.3e} max_abs={ma:.3e} max_ref={mr:.3e}")
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite output"
    assert rf <= rel_fro, f"{name}: relative Frobenius error {rf:.3e} > {rel_fro:.1e}"
    assert ma <= max_abs_frac * mr, f"{name}: max abs error {ma:.3e} > {max_abs_frac:.1e} * {mr:.3e}"


def _block_reduce(ufunc, a: np.ndarray, tile_m: int, tile_n: int) -> np.ndarray:
    """ufunc.reduceat of a 1-D or 2-D array over blocks of tile_m rows (x tile_n columns)."""
    s = ufunc.reduceat(a, np.arange(0, a.shape[0], tile_m), axis=0)
    return s if a.ndim == 1 else ufunc.reduceat(s, np.arange(0, a.shape[1], tile_n), axis=1)


def assert_close_tiles(name: str, got, ref, rel_fro=REL_FRO, max_abs_frac=MAX_ABS, tile_m=256, tile_n=256):
    """The gate on the whole tensor, then on every output tile of the GEMM on its own.

    A kernel computes each 256 x 256 output tile independently (its own depth loop, its
    own epilogue), so a fault confined to one tile (a dropped or repeated depth step, a
    misplaced side input) can stay below the whole-tensor relative error of thousands of
    tiles. The same relative bound therefore applies per tile (per 256-row block for 1-D
    outputs); a tile whose reference is exactly zero must come out within the max-abs
    bound of the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert_close(name, got, ref, rel_fro, max_abs_frac)
    if ref.size == 0:
        return
    diff = got - ref
    num = _block_reduce(np.add, diff * diff, tile_m, tile_n)
    den = _block_reduce(np.add, ref * ref, tile_m, tile_n)
    nz = den > 0
    rel = np.zeros_like(num)
    rel[nz] = np.sqrt(num[nz] / den[nz])
    worst = float(rel.max())
    log(f"  {name}: {num.size} tiles, worst tile rel_fro={worst:.3e}")
    bad = np.argwhere(rel > rel_fro)
    assert bad.size == 0, f"{name}: {len(bad)} tiles above {rel_fro:.1e}, first at block {bad[0].tolist()}"
    if not nz.all():
        dmax = _block_reduce(np.maximum, np.abs(diff), tile_m, tile_n)
        limit = max_abs_frac * float(np.max(np.abs(ref)))
        assert float(dmax[~nz].max()) <= limit, f"{name}: a tile with an all-zero reference is off by more than {limit}"
