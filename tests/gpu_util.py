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


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    """Rows to check at full size: the first and last rows of the batch, rows at tile
    edges, and random rows."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 255, 256, M // 2, M - 257, M - 256, M - 1}
    fixed = {r for r in fixed if 0 <= r < M}
    rnd = rng.choice(M, size=max(0, n - len(fixed)), replace=False)
    return np.array(sorted(fixed | set(int(r) for r in rnd)))
