"""Seeded synthetic inputs for the GEMM-epilogue workloads.

This module holds none of the method's arithmetic. It only draws Gaussian numbers
from a seeded PCG64 generator, scales them to the stated standard deviation and packs
the fp32 draws into bf16 bit patterns with round-to-nearest-even. The HIP path (through
its tests and the bench) and the CPU oracle both consume exactly these arrays; neither
side generates its own inputs.

Notation: a workload "N(0, v)" names a normal law of *variance* v, so its draws are
scaled by sqrt(v) (e.g. N(0, 1/4096) has standard deviation 1/64 and N(0, 1e-2) has
standard deviation 0.1).

Every tensor is a C-contiguous row-major numpy array: bf16 tensors as ``uint16`` bit
patterns, scalars as Python floats/ints.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "normal_bf16",
    "small_int_bf16",
    "Workload",
    "tiny_fwd",
    "rope_qkv",
    "swiglu",
    "llama_fwd",
    "bwd_stats",
    "WORKLOADS",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the bits.

    The inputs here are finite Gaussian draws, so NaN handling is not needed; a NaN
    or infinity input raises instead of being silently mangled.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    """Draw fp32 standard normals, form ``mean + std * g`` in fp32, round to bf16 bits."""
    g = rng.standard_normal(size=shape, dtype=np.float32)
    v = np.float32(mean) + np.float32(std) * g
    return f32_to_bf16_bits(v)


def small_int_bf16(rng: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 bits (exact: |v| <= 256 is representable)."""
    assert -256 <= lo <= hi <= 256
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


@dataclass
class Workload:
    """One seeded problem instance: its tensors (bf16 bits) and scalar parameters."""

    name: str
    seed: int
    tensors: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)

    def __getitem__(self, k):
        if k in self.tensors:
            return self.tensors[k]
        return self.params[k]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def gemm_rmsnorm_fwd_inputs(seed: int, M: int, K: int, D: int, N1: int, eps: float,
                            name: str = "gemm_rmsnorm_fwd") -> Workload:
    """x[M,K] ~ N(0,1); W0[K,D] ~ N(0,1/K); z[M,D] ~ N(0,1); gamma[D] = 1 + 0.1 N(0,1);
    W1[D,N1] ~ N(0,1/D); drawn in that order from one seed."""
    rng = _rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    w0 = normal_bf16(rng, (K, D), 1.0 / np.sqrt(K))
    z = normal_bf16(rng, (M, D), 1.0)
    gamma = normal_bf16(rng, (D,), 0.1, mean=1.0)
    w1 = normal_bf16(rng, (D, N1), 1.0 / np.sqrt(D))
    return Workload(name, seed, dict(x=x, w0=w0, z=z, gamma=gamma, w1=w1),
                    dict(M=M, K=K, D=D, N1=N1, eps=eps))


def tiny_fwd(seed: int = 0) -> Workload:
    """Tiny GEMM-RMSNorm-GEMM forward: 256x256x256 twice, eps = 1e-6."""
    return gemm_rmsnorm_fwd_inputs(seed, 256, 256, 256, 256, 1e-6, name="tiny_gemm_rmsnorm_gemm_256")


def llama_fwd(seed: int = 3, M: int = 8192, K: int = 14336, D: int = 4096, N1: int = 6144,
              eps: float = 1e-5) -> Workload:
    """Llama-3-8B-shaped GEMM-RMSNorm-GEMM forward: FFN down-projection (K=14336 -> D=4096),
    residual add, RMSNorm, then the GQA QKV projection (D -> 4096 + 2*1024)."""
    return gemm_rmsnorm_fwd_inputs(seed, M, K, D, N1, eps,
                                   name=f"llama3_8b_gemm_rmsnorm_gemm_M{M}")


def rope_qkv(seed: int = 1, M: int = 4096, K: int = 4096, n_q: int = 4096, n_k: int = 4096,
             n_v: int = 4096, head_dim: int = 128, seq_len: int = 4096, pos_offset: int = 0,
             theta: float = 10000.0) -> Workload:
    """QKV projection with RoPE: x[M,K] ~ N(0,1); W[K, n_q+n_k+n_v] ~ N(0,1/K)."""
    rng = _rng(seed)
    N = n_q + n_k + n_v
    x = normal_bf16(rng, (M, K), 1.0)
    w = normal_bf16(rng, (K, N), 1.0 / np.sqrt(K))
    return Workload(f"gemm_rope_qkv_M{M}_K{K}_N{N}", seed, dict(x=x, w=w),
                    dict(M=M, K=K, n_q=n_q, n_k=n_k, n_v=n_v, head_dim=head_dim,
                         seq_len=seq_len, pos_offset=pos_offset, theta=theta))


def rope_qkv_8k(seed: int = 9) -> Workload:
    """The 8192-class GEMM + RoPE: M = K = 8192, QKV width 3 x 8192, head_dim 128, the
    positions of one 8192-token sequence; same distributions as rope_qkv."""
    return rope_qkv(seed=seed, M=8192, K=8192, n_q=8192, n_k=8192, n_v=8192, head_dim=128, seq_len=8192)


def swiglu(seed: int = 2, M: int = 8192, K: int = 8192, F: int = 4096) -> Workload:
    """GEMM+SwiGLU: x[M,K] ~ N(0,1); W[K,2F] ~ N(0,1/K) with interleaved columns
    (even = gate, odd = up)."""
    rng = _rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    w = normal_bf16(rng, (K, 2 * F), 1.0 / np.sqrt(K))
    return Workload(f"gemm_swiglu_M{M}_K{K}_F{F}", seed, dict(x=x, w=w), dict(M=M, K=K, F=F))


def swiglu_4k(seed: int = 10) -> Workload:
    """GEMM+SwiGLU at the pages' 4096 shape: M = K = 4096, interleaved width 2F = 4096."""
    return swiglu(seed=seed, M=4096, K=4096, F=2048)


def bwd_stats(seed: int = 4, M: int = 8192, D: int = 4096, N: int = 6144) -> Workload:
    """RMSNorm-backward statistic through the grad GEMM: h2[M,D] ~ N(0,1);
    W1[D,N] ~ N(0,1/D); dY[M,N] ~ N(0,1e-2), drawn in that order."""
    rng = _rng(seed)
    h2 = normal_bf16(rng, (M, D), 1.0)
    w1 = normal_bf16(rng, (D, N), 1.0 / np.sqrt(D))
    dy = normal_bf16(rng, (M, N), 0.1)
    return Workload(f"gemm_rmsnorm_bwd_stats_M{M}_D{D}_N{N}", seed, dict(h2=h2, w1=w1, dy=dy),
                    dict(M=M, D=D, N=N))


def rmsnorm_bwd_full(seed: int = 5, M: int = 8192, D: int = 4096, N: int = 6144) -> Workload:
    """Rest of the RMSNorm backward at the backward workload's shapes: h1[M,D] ~ N(0,1);
    gamma = 1 + 0.1 N(0,1); W1[D,N] ~ N(0,1/D); dY[M,N] ~ N(0,1e-2); residual-stream
    gradient g_res[M,D] ~ N(0,1e-2); eps = 1e-5; drawn in that order."""
    rng = _rng(seed)
    h1 = normal_bf16(rng, (M, D), 1.0)
    gamma = normal_bf16(rng, (D,), 0.1, 1.0)
    w1 = normal_bf16(rng, (D, N), 1.0 / np.sqrt(D))
    dy = normal_bf16(rng, (M, N), 0.1)
    g_res = normal_bf16(rng, (M, D), 0.1)
    return Workload(f"rmsnorm_bwd_M{M}_D{D}_N{N}", seed, dict(h1=h1, gamma=gamma, w1=w1, dy=dy, g_res=g_res),
                    dict(M=M, D=D, N=N, eps=1e-5))


def swiglu_bwd(seed: int = 6, M: int = 8192, Dm: int = 8192, F: int = 4096) -> Workload:
    """SwiGLU backward through the down projection's grad GEMM: saved interleaved
    pre-activations h[M, 2F] ~ N(0,1); W_down[F, Dm] ~ N(0,1/F); dY[M, Dm] ~ N(0,1e-2),
    drawn in that order."""
    rng = _rng(seed)
    h = normal_bf16(rng, (M, 2 * F), 1.0)
    w_down = normal_bf16(rng, (F, Dm), 1.0 / np.sqrt(F))
    dy = normal_bf16(rng, (M, Dm), 0.1)
    return Workload(f"gemm_swiglu_bwd_M{M}_Dm{Dm}_F{F}", seed, dict(h=h, w_down=w_down, dy=dy),
                    dict(M=M, Dm=Dm, F=F))


def rope_bwd(seed: int = 7, M: int = 4096, K: int = 4096, n_q: int = 4096, n_k: int = 4096,
             n_v: int = 4096, head_dim: int = 128, seq_len: int = 4096, pos_offset: int = 0,
             theta: float = 10000.0) -> Workload:
    """RoPE backward in the epilogue of the GEMM producing the rotated Q/K/V gradient, at
    the RoPE workload's shapes: a[M,K] ~ N(0,1e-2); W[K, n_q+n_k+n_v] ~ N(0,1/K)."""
    rng = _rng(seed)
    N = n_q + n_k + n_v
    x = normal_bf16(rng, (M, K), 0.1)
    w = normal_bf16(rng, (K, N), 1.0 / np.sqrt(K))
    return Workload(f"gemm_rope_bwd_M{M}_K{K}_N{N}", seed, dict(x=x, w=w),
                    dict(M=M, K=K, n_q=n_q, n_k=n_k, n_v=n_v, head_dim=head_dim,
                         seq_len=seq_len, pos_offset=pos_offset, theta=theta))


def cross_entropy(seed: int = 8, M: int = 4096, K: int = 4096, V: int = 32768, ignore_every: int = 0) -> Workload:
    """GEMM + cross-entropy at the pages' M x vocab x K shapes: hidden x[M,K] ~ N(0,1);
    W[K,V] ~ N(0,1/K) (logits ~ N(0,1)); labels uniform in [0, V); with ignore_every = k,
    every k-th row's label is -1 (ignored). Drawn in that order."""
    rng = _rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    w = normal_bf16(rng, (K, V), 1.0 / np.sqrt(K))
    labels = rng.integers(0, V, size=M, dtype=np.int64).astype(np.int32)
    if ignore_every:
        labels[::ignore_every] = -1
    return Workload(f"gemm_cross_entropy_M{M}_K{K}_V{V}", seed, dict(x=x, w=w, labels=labels),
                    dict(M=M, K=K, V=V))


def cross_entropy_8k(seed: int = 8, ignore_every: int = 0) -> Workload:
    """GEMM + cross-entropy at the larger of the kernel table's two shapes: 8192 tokens,
    vocabulary 32768, hidden 8192; same distributions as cross_entropy."""
    return cross_entropy(seed=seed, M=8192, K=8192, V=32768, ignore_every=ignore_every)


# The five workloads at their stated sizes (seed i for workload i).
WORKLOADS = {
    "tiny_fwd": tiny_fwd,
    "rope_qkv": rope_qkv,
    "swiglu": swiglu,
    "llama_fwd": llama_fwd,
    "bwd_stats": bwd_stats,
}
