"""Python binding of libcoda.so: gfx950 bf16 GEMMs with Transformer epilogues.

Argument marshalling only. Every step of the computation runs in the HIP kernels of
libcoda.so; torch is used for device memory (output allocation) and for the current
HIP stream. There is no CPU fallback: if the library is missing or a tensor is not
on the GPU, the call raises.

Function names match the C ABI in include/coda.h. bf16 tensors are torch.bfloat16
CUDA tensors (their storage holds the bf16 bit patterns the C ABI takes as uint16).
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH, ROOT, source_hash

__all__ = [
    "CodaError",
    "StaleLibraryError",
    "check_source_hash",
    "lib",
    "PARTIAL_TILE_N",
    "ROWSTAT_RSQRT_MEAN_EPS",
    "ROWSTAT_MEAN",
    "num_partials",
    "coda_gemm_rmsnorm_fwd",
    "coda_gemm_rmsnorm_fwd_noalloc",
    "coda_gemm_rmsnorm_fwd_ws",
    "coda_gemm_rmsnorm_fwd_workspace_bytes",
    "NOALLOC_SCRATCH_FLOATS",
    "coda_gemm_residual_rmsnorm_partials",
    "coda_gemm_rowscale",
    "coda_rowstat_reduce",
    "coda_rope_tables",
    "coda_gemm_rope",
    "coda_gemm_rope_persistent",
    "coda_gemm_swiglu",
    "coda_gemm_swiglu_ws",
    "coda_gemm_rope_ws",
    "coda_split_workspace_bytes",
    "coda_split_plan",
    "coda_gemm_rmsnorm_bwd_stats",
    "coda_gemm_rmsnorm_bwd_stats_ws",
    "num_row_tiles",
    "coda_rowdot_stat",
    "coda_gemm_rmsnorm_bwd_dx",
    "coda_gemm_rmsnorm_bwd_dx_ws",
    "coda_colsum_reduce",
    "coda_rmsnorm_bwd",
    "coda_gemm_rope_bwd",
    "coda_gemm_rope_bwd_ws",
    "coda_gemm_swiglu_bwd",
    "coda_gemm_swiglu_bwd_ws",
    "coda_gemm_cross_entropy",
    "coda_gemm_cross_entropy_ws",
    "coda_lse_reduce",
    "coda_baseline_gemm",
    "coda_baseline_residual_rmsnorm",
    "coda_baseline_rope",
    "coda_baseline_swiglu",
    "coda_baseline_rowdot",
    "coda_baseline_copy",
    "coda_baseline_mfma_loop",
    "coda_baseline_schedule_probe",
]

PARTIAL_TILE_N = 256
ROWSTAT_RSQRT_MEAN_EPS = 0
ROWSTAT_MEAN = 1
NOALLOC_SCRATCH_FLOATS = 1 << 20

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_D = ctypes.c_double
_I64 = ctypes.c_int64

# name -> argument types (every entry point returns int status)
SIGNATURES = {
    "coda_abi_version": [],
    "coda_rowstat_num_partials": [_I, ctypes.POINTER(_I)],
    "coda_gemm_rmsnorm_fwd": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P],
    "coda_gemm_rmsnorm_fwd_noalloc": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P],
    "coda_gemm_rmsnorm_fwd_ws": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _I64, _P],
    "coda_gemm_rmsnorm_fwd_workspace_bytes": [_I, _I, _I, _I, ctypes.POINTER(_I64)],
    "coda_gemm_residual_rmsnorm_partials": [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P],
    "coda_gemm_rowscale": [_P, _P, _P, _I, _I, _I, _P, _P],
    "coda_rowstat_reduce": [_P, _I, _I, _I, _F, _I, _P, _P],
    "coda_rope_tables": [_P, _P, _I, _I, _D, _P],
    "coda_gemm_rope": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P],
    "coda_gemm_rope_persistent": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P],
    "coda_gemm_rope_ws": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I64, _P],
    "coda_gemm_swiglu": [_P, _P, _I, _I, _I, _P, _P],
    "coda_gemm_swiglu_ws": [_P, _P, _I, _I, _I, _P, _P, _I64, _P],
    "coda_split_workspace_bytes": [_I, _I, _I, ctypes.POINTER(_I64)],
    "coda_split_plan": [_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I),
                        ctypes.POINTER(_I64)],
    "coda_gemm_rope_bwd": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P],
    "coda_gemm_rope_bwd_ws": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I64, _P],
    "coda_gemm_swiglu_bwd": [_P, _P, _P, _I, _I, _I, _P, _P],
    "coda_gemm_swiglu_bwd_ws": [_P, _P, _P, _I, _I, _I, _P, _P, _I64, _P],
    "coda_gemm_cross_entropy": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P],
    "coda_gemm_cross_entropy_ws": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _I64, _P],
    "coda_lse_reduce": [_P, _P, _I, _I, _I, _P, _P, _P, _P],
    "coda_gemm_rmsnorm_bwd_stats": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P],
    "coda_gemm_rmsnorm_bwd_stats_ws": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _I64, _P],
    "coda_colstat_num_partials": [_I, _P],
    "coda_rowdot_stat": [_P, _P, _I, _I, _I, _P, _P],
    "coda_colsum_reduce": [_P, _I, _I, _P, _P],
    "coda_gemm_rmsnorm_bwd_dx": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P],
    "coda_gemm_rmsnorm_bwd_dx_ws": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _I64, _P],
    "coda_rmsnorm_bwd": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P],
    "coda_baseline_gemm": [_P, _P, _I, _I, _I, _I, _P, _P],
    "coda_baseline_residual_rmsnorm": [_P, _P, _P, _I, _I, _F, _P, _P, _P, _P],
    "coda_baseline_rope": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P],
    "coda_baseline_swiglu": [_P, _I, _I, _P, _P],
    "coda_baseline_rowdot": [_P, _P, _I, _I, _P, _P],
    "coda_baseline_copy": [_P, _P, _I64, _P],
    "coda_baseline_mfma_loop": [_P, _I, _I, _I, _P, _P],
    "coda_baseline_schedule_probe": [_I, _I, _I, _F, ctypes.c_uint32, _P, _P, _P],
}


class CodaError(RuntimeError):
    def __init__(self, name: str, status: int, message: str):
        super().__init__(f"{name} failed: status {status} ({message})")
        self.status = status


_lib = None


class StaleLibraryError(RuntimeError):
    """libcoda.so was built from sources other than those next to it."""


def check_source_hash(L: ctypes.CDLL, root: str = ROOT) -> None:
    """Raise StaleLibraryError unless the library's embedded source hash equals the hash
    of the sources under `root`."""
    built = L.coda_build_source_hash().decode()
    here = source_hash(root)
    if built != here:
        raise StaleLibraryError(f"{LIB_PATH} was built from other sources (built {built[:16]}, sources "
                                f"{here[:16]}): rebuild it with transformer_gemm_epilogue_amd.build.build()")


def lib() -> ctypes.CDLL:
    """Load libcoda.so (built in-tree by build.py), check that it was built from the
    sources next to it, and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run transformer_gemm_epilogue_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.coda_build_source_hash.argtypes = []
        L.coda_build_source_hash.restype = ctypes.c_char_p
        check_source_hash(L)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _I
        L.coda_status_string.argtypes = [_I]
        L.coda_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _call(name: str, *args) -> None:
    L = lib()
    st = getattr(L, name)(*args)
    if st != 0:
        raise CodaError(name, st, L.coda_status_string(st).decode())


def _torch():
    import torch  # imported lazily: the library itself does not need it
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (there is no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _bf16(t, name):
    return _dev(t, _torch().bfloat16, name)


def _f32(t, name):
    return _dev(t, _torch().float32, name)


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


def num_partials(width: int) -> int:
    nb = ctypes.c_int(0)
    _call("coda_rowstat_num_partials", int(width), ctypes.byref(nb))
    return nb.value


# ------------------------------------------------------------------ fused entry points
def coda_gemm_rmsnorm_fwd(x, w0, z, gamma, w1, eps, h1=None, h2=None, partials=None, r=None, y=None,
                          stream=None):
    """y = RMSNorm(x w0 + z, gamma) w1 via GEMM1-epilogue / row reduce / GEMM2-epilogue.
    Returns (h1, h2, partials, r, y)."""
    torch = _torch()
    M, K = x.shape
    D = w0.shape[1]
    N1 = w1.shape[1]
    if w0.shape[0] != K or z.shape != (M, D) or gamma.shape != (D,) or w1.shape[0] != D:
        raise ValueError("coda_gemm_rmsnorm_fwd: inconsistent shapes")
    h1 = _empty((M, D), torch.bfloat16, x) if h1 is None else h1
    h2 = _empty((M, D), torch.bfloat16, x) if h2 is None else h2
    partials = _empty((M, num_partials(D)), torch.float32, x) if partials is None else partials
    r = _empty((M,), torch.float32, x) if r is None else r
    y = _empty((M, N1), torch.bfloat16, x) if y is None else y
    _call("coda_gemm_rmsnorm_fwd", _bf16(x, "x"), _bf16(w0, "w0"), _bf16(z, "z"), _bf16(gamma, "gamma"),
          _bf16(w1, "w1"), M, K, D, N1, float(eps), _bf16(h1, "h1"), _bf16(h2, "h2"),
          _f32(partials, "partials"), _f32(r, "r"), _bf16(y, "y"), _stream(stream))
    return h1, h2, partials, r, y


def coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1):
    """Bytes of workspace coda_gemm_rmsnorm_fwd_ws needs on the current device."""
    out = ctypes.c_int64(0)
    _call("coda_gemm_rmsnorm_fwd_workspace_bytes", int(M), int(K), int(D), int(N1), ctypes.byref(out))
    return out.value


def coda_gemm_rmsnorm_fwd_ws(x, w0, z, gamma, w1, eps, h1=None, h2=None, partials=None, r=None, y=None,
                             workspace=None, stream=None):
    """coda_gemm_rmsnorm_fwd with the split-depth schedule for GEMMs with fewer tiles than
    CUs; `workspace` is a uint8 GPU tensor of at least coda_gemm_rmsnorm_fwd_workspace_bytes
    bytes (allocated here when None). Returns (h1, h2, partials, r, y)."""
    torch = _torch()
    M, K = x.shape
    D = w0.shape[1]
    N1 = w1.shape[1]
    if w0.shape[0] != K or z.shape != (M, D) or gamma.shape != (D,) or w1.shape[0] != D:
        raise ValueError("coda_gemm_rmsnorm_fwd_ws: inconsistent shapes")
    h1 = _empty((M, D), torch.bfloat16, x) if h1 is None else h1
    h2 = _empty((M, D), torch.bfloat16, x) if h2 is None else h2
    partials = _empty((M, num_partials(D)), torch.float32, x) if partials is None else partials
    r = _empty((M,), torch.float32, x) if r is None else r
    y = _empty((M, N1), torch.bfloat16, x) if y is None else y
    if workspace is None:
        need = coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1)
        workspace = _empty((max(need, 16),), torch.uint8, x)
    ws = _dev(workspace, torch.uint8, "workspace")
    _call("coda_gemm_rmsnorm_fwd_ws", _bf16(x, "x"), _bf16(w0, "w0"), _bf16(z, "z"), _bf16(gamma, "gamma"),
          _bf16(w1, "w1"), M, K, D, N1, float(eps), _bf16(h1, "h1"), _bf16(h2, "h2"),
          _f32(partials, "partials"), _f32(r, "r"), _bf16(y, "y"), ws, int(workspace.numel()), _stream(stream))
    return h1, h2, partials, r, y


def coda_gemm_rmsnorm_fwd_noalloc(x, w0, z, gamma, w1, eps, h1, h2, r, y, stream=None):
    """coda_gemm_rmsnorm_fwd with the row partials in the library's fixed device array:
    nothing is allocated, by the library or here, so every output is the caller's."""
    M, K = x.shape
    D = w0.shape[1]
    N1 = w1.shape[1]
    if (w0.shape[0] != K or z.shape != (M, D) or gamma.shape != (D,) or w1.shape[0] != D or h1.shape != (M, D)
            or h2.shape != (M, D) or r.shape != (M,) or y.shape != (M, N1)):
        raise ValueError("coda_gemm_rmsnorm_fwd_noalloc: inconsistent shapes")
    _call("coda_gemm_rmsnorm_fwd_noalloc", _bf16(x, "x"), _bf16(w0, "w0"), _bf16(z, "z"), _bf16(gamma, "gamma"),
          _bf16(w1, "w1"), M, K, D, N1, float(eps), _bf16(h1, "h1"), _bf16(h2, "h2"), _f32(r, "r"), _bf16(y, "y"),
          _stream(stream))
    return h1, h2, r, y


def coda_gemm_residual_rmsnorm_partials(x, w0, z, gamma, h1=None, h2=None, partials=None, stream=None):
    torch = _torch()
    M, K = x.shape
    D = w0.shape[1]
    if w0.shape[0] != K or z.shape != (M, D) or gamma.shape != (D,):
        raise ValueError("coda_gemm_residual_rmsnorm_partials: inconsistent shapes")
    h1 = _empty((M, D), torch.bfloat16, x) if h1 is None else h1
    h2 = _empty((M, D), torch.bfloat16, x) if h2 is None else h2
    partials = _empty((M, num_partials(D)), torch.float32, x) if partials is None else partials
    _call("coda_gemm_residual_rmsnorm_partials", _bf16(x, "x"), _bf16(w0, "w0"), _bf16(z, "z"),
          _bf16(gamma, "gamma"), M, K, D, _bf16(h1, "h1"), _bf16(h2, "h2"), _f32(partials, "partials"),
          _stream(stream))
    return h1, h2, partials


def coda_gemm_rowscale(h2, w1, r, y=None, stream=None):
    torch = _torch()
    M, D = h2.shape
    N1 = w1.shape[1]
    if w1.shape[0] != D or r.shape != (M,):
        raise ValueError("coda_gemm_rowscale: inconsistent shapes")
    y = _empty((M, N1), torch.bfloat16, h2) if y is None else y
    _call("coda_gemm_rowscale", _bf16(h2, "h2"), _bf16(w1, "w1"), _f32(r, "r"), M, D, N1, _bf16(y, "y"),
          _stream(stream))
    return y


def coda_rowstat_reduce(partials, d, eps=0.0, mode=ROWSTAT_RSQRT_MEAN_EPS, out=None, stream=None):
    torch = _torch()
    M, nb = partials.shape
    out = _empty((M,), torch.float32, partials) if out is None else out
    _call("coda_rowstat_reduce", _f32(partials, "partials"), M, nb, int(d), float(eps), int(mode),
          _f32(out, "out"), _stream(stream))
    return out


def coda_rope_tables(seq_len, head_dim, theta=10000.0, device="cuda", stream=None):
    """Returns (cos_t, sin_t), each [seq_len, head_dim // 2] fp32, built on the GPU."""
    torch = _torch()
    cos_t = torch.empty((seq_len, head_dim // 2), dtype=torch.float32, device=device)
    sin_t = torch.empty_like(cos_t)
    _call("coda_rope_tables", _f32(cos_t, "cos_t"), _f32(sin_t, "sin_t"), int(seq_len), int(head_dim),
          float(theta), _stream(stream))
    return cos_t, sin_t


def _split_args(split, need, like, workspace):
    """The (workspace, bytes) arguments of a split-depth entry point (none otherwise)."""
    if not split:
        return ()
    return _workspace(need() if workspace is None else 0, like, workspace)


def _gemm_rope(name, x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out, stream, split=False,
               workspace=None):
    torch = _torch()
    M, K = x.shape
    N = n_q + n_k + n_v
    if w.shape != (K, N):
        raise ValueError(f"{name}: w must be [K, n_q + n_k + n_v]")
    out = _empty((M, N), torch.bfloat16, x) if out is None else out
    ws = _split_args(split, lambda: coda_split_workspace_bytes(M, N, K), x, workspace)
    _call(name, _bf16(x, "x"), _bf16(w, "w"), _f32(cos_t, "cos_t"), _f32(sin_t, "sin_t"), M, K,
          n_q, n_k, n_v, head_dim, seq_len, pos_offset, _bf16(out, "out"), *ws, _stream(stream))
    return out


def coda_gemm_rope(x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset=0, out=None, stream=None):
    return _gemm_rope("coda_gemm_rope", x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out,
                      stream)


def coda_split_workspace_bytes(M, N, K):
    """Bytes of split-depth workspace one GEMM with output [M, N] and depth K needs."""
    out = ctypes.c_int64(0)
    _call("coda_split_workspace_bytes", int(M), int(N), int(K), ctypes.byref(out))
    return out.value


def coda_split_plan(M, N, K, cus):
    """The split-depth plan of one GEMM on a device of `cus` CUs (host only): (slices per
    split tile, depth steps per slice, first split tile, workspace bytes)."""
    s, st, t0, b = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int64(0)
    _call("coda_split_plan", int(M), int(N), int(K), int(cus), ctypes.byref(s), ctypes.byref(st), ctypes.byref(t0),
          ctypes.byref(b))
    return s.value, st.value, t0.value, b.value


def _workspace(need, like, workspace):
    if workspace is None:
        workspace = _empty((max(int(need), 16),), _torch().uint8, like)
    return _dev(workspace, _torch().uint8, "workspace"), int(workspace.numel())


def coda_gemm_rope_ws(x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset=0, out=None, workspace=None,
                      stream=None):
    """coda_gemm_rope with the split-depth schedule for outputs with fewer tiles than CUs
    (`workspace`: uint8 GPU tensor, allocated here when None)."""
    return _gemm_rope("coda_gemm_rope_ws", x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out,
                      stream, True, workspace)


def coda_gemm_rope_persistent(x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset=0, out=None,
                              stream=None):
    """coda_gemm_rope under the persistent schedule (same output, bit for bit)."""
    return _gemm_rope("coda_gemm_rope_persistent", x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset,
                      out, stream)


def coda_gemm_rope_bwd(x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset=0, out=None, stream=None):
    """x w with every Q and K pair rotated by the negated angle (the RoPE backward)."""
    return _gemm_rope("coda_gemm_rope_bwd", x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out,
                      stream)


def coda_gemm_rope_bwd_ws(x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset=0, out=None,
                          workspace=None, stream=None):
    """coda_gemm_rope_bwd with the split-depth schedule."""
    return _gemm_rope("coda_gemm_rope_bwd_ws", x, w, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset,
                      out, stream, True, workspace)


def coda_gemm_swiglu(x, w, out=None, stream=None):
    torch = _torch()
    M, K = x.shape
    if w.shape[0] != K or w.shape[1] % 2:
        raise ValueError("coda_gemm_swiglu: w must be [K, 2F]")
    F = w.shape[1] // 2
    out = _empty((M, F), torch.bfloat16, x) if out is None else out
    _call("coda_gemm_swiglu", _bf16(x, "x"), _bf16(w, "w"), M, K, F, _bf16(out, "out"), _stream(stream))
    return out


def coda_gemm_swiglu_ws(x, w, out=None, workspace=None, stream=None):
    """coda_gemm_swiglu with the split-depth schedule for outputs with fewer tiles than CUs."""
    torch = _torch()
    M, K = x.shape
    if w.shape[0] != K or w.shape[1] % 2:
        raise ValueError("coda_gemm_swiglu_ws: w must be [K, 2F]")
    F = w.shape[1] // 2
    out = _empty((M, F), torch.bfloat16, x) if out is None else out
    ws, nbytes = _workspace(coda_split_workspace_bytes(M, 2 * F, K) if workspace is None else 0, x, workspace)
    _call("coda_gemm_swiglu_ws", _bf16(x, "x"), _bf16(w, "w"), M, K, F, _bf16(out, "out"), ws, nbytes,
          _stream(stream))
    return out


def _swiglu_bwd(name, dy, w_down, h, dh, stream, split=False, workspace=None):
    torch = _torch()
    M, Dm = dy.shape
    F = w_down.shape[0]
    if w_down.shape[1] != Dm or h.shape != (M, 2 * F):
        raise ValueError(f"{name}: inconsistent shapes")
    dh = _empty((M, 2 * F), torch.bfloat16, dy) if dh is None else dh
    ws = _split_args(split, lambda: coda_split_workspace_bytes(M, F, Dm), dy, workspace)
    _call(name, _bf16(dy, "dy"), _bf16(w_down, "w_down"), _bf16(h, "h"), M, Dm, F, _bf16(dh, "dh"), *ws,
          _stream(stream))
    return dh


def coda_gemm_swiglu_bwd(dy, w_down, h, dh=None, stream=None):
    """dOut = dy w_down^T mapped in the epilogue to the interleaved (gate, up) gradients
    of the saved pre-activations h [M, 2F]. Returns dh [M, 2F]."""
    return _swiglu_bwd("coda_gemm_swiglu_bwd", dy, w_down, h, dh, stream)


def coda_gemm_swiglu_bwd_ws(dy, w_down, h, dh=None, workspace=None, stream=None):
    """coda_gemm_swiglu_bwd with the split-depth schedule (output width F, depth Dm)."""
    return _swiglu_bwd("coda_gemm_swiglu_bwd_ws", dy, w_down, h, dh, stream, True, workspace)


def _i32(t, name):
    return _dev(t, _torch().int32, name)


def _cross_entropy(name, x, w, labels, tile_lse, target, lse, loss, stream, split=False, workspace=None):
    torch = _torch()
    M, K = x.shape
    V = w.shape[1]
    if w.shape[0] != K or labels.shape != (M,):
        raise ValueError(f"{name}: inconsistent shapes")
    tile_lse = _empty((M, num_partials(V)), torch.float32, x) if tile_lse is None else tile_lse
    target = _empty((M,), torch.float32, x) if target is None else target
    lse = _empty((M,), torch.float32, x) if lse is None else lse
    loss = _empty((M,), torch.float32, x) if loss is None else loss
    ws = _split_args(split, lambda: coda_split_workspace_bytes(M, V, K), x, workspace)
    _call(name, _bf16(x, "x"), _bf16(w, "w"), _i32(labels, "labels"), M, K, V, _f32(tile_lse, "tile_lse"),
          _f32(target, "target"), _f32(lse, "lse"), _f32(loss, "loss"), *ws, _stream(stream))
    return loss, lse, target, tile_lse


def coda_gemm_cross_entropy(x, w, labels, tile_lse=None, target=None, lse=None, loss=None, stream=None):
    """Cross-entropy of the logits x w (never stored) against int32 labels (outside
    [0, V): ignored, loss 0). Returns (loss, lse, target, tile_lse)."""
    return _cross_entropy("coda_gemm_cross_entropy", x, w, labels, tile_lse, target, lse, loss, stream)


def coda_gemm_cross_entropy_ws(x, w, labels, tile_lse=None, target=None, lse=None, loss=None, workspace=None,
                               stream=None):
    """coda_gemm_cross_entropy with the split-depth schedule."""
    return _cross_entropy("coda_gemm_cross_entropy_ws", x, w, labels, tile_lse, target, lse, loss, stream, True,
                          workspace)


def coda_lse_reduce(tile_lse, labels, V, target, lse=None, loss=None, stream=None):
    """The auxiliary merge of per-tile log-sum-exp partials. Returns (loss, lse)."""
    torch = _torch()
    M, nb = tile_lse.shape
    lse = _empty((M,), torch.float32, tile_lse) if lse is None else lse
    loss = _empty((M,), torch.float32, tile_lse) if loss is None else loss
    _call("coda_lse_reduce", _f32(tile_lse, "tile_lse"), _i32(labels, "labels"), M, nb, int(V),
          _f32(target, "target"), _f32(lse, "lse"), _f32(loss, "loss"), _stream(stream))
    return loss, lse


def _bwd_stats(name, dy, w1, h2, dh2, partials, s, stream, split=False, workspace=None):
    torch = _torch()
    M, N = dy.shape
    D = w1.shape[0]
    if w1.shape[1] != N or h2.shape != (M, D):
        raise ValueError(f"{name}: inconsistent shapes")
    dh2 = _empty((M, D), torch.bfloat16, dy) if dh2 is None else dh2
    partials = _empty((M, num_partials(D)), torch.float32, dy) if partials is None else partials
    s = _empty((M,), torch.float32, dy) if s is None else s
    ws = _split_args(split, lambda: coda_split_workspace_bytes(M, D, N), dy, workspace)
    _call(name, _bf16(dy, "dy"), _bf16(w1, "w1"), _bf16(h2, "h2"), M, D, N, _bf16(dh2, "dh2"),
          _f32(partials, "partials"), _f32(s, "s"), *ws, _stream(stream))
    return dh2, partials, s


def coda_gemm_rmsnorm_bwd_stats(dy, w1, h2, dh2=None, partials=None, s=None, stream=None):
    """dh2 = dy w1^T with row partials of dh2 * h2 in the epilogue, then s = mean.
    Returns (dh2, partials, s)."""
    return _bwd_stats("coda_gemm_rmsnorm_bwd_stats", dy, w1, h2, dh2, partials, s, stream)


def coda_gemm_rmsnorm_bwd_stats_ws(dy, w1, h2, dh2=None, partials=None, s=None, workspace=None, stream=None):
    """coda_gemm_rmsnorm_bwd_stats with the split-depth schedule (output width D, depth N)."""
    return _bwd_stats("coda_gemm_rmsnorm_bwd_stats_ws", dy, w1, h2, dh2, partials, s, stream, True, workspace)


def num_row_tiles(rows: int) -> int:
    """Row tiles (of 256) of the column-partial workspace [tiles, D] of dgamma."""
    t = ctypes.c_int(0)
    _call("coda_colstat_num_partials", int(rows), ctypes.byref(t))
    return t.value


def _opt_bf16(t, name):
    return ctypes.c_void_p(None) if t is None else _bf16(t, name)


def coda_rowdot_stat(dy, y, d, s=None, stream=None):
    """s[m] = (1/d) sum_j dy[m, j] y[m, j] (the statistic from the output side)."""
    torch = _torch()
    M, N = dy.shape
    if y.shape != (M, N):
        raise ValueError("coda_rowdot_stat: inconsistent shapes")
    s = _empty((M,), torch.float32, dy) if s is None else s
    _call("coda_rowdot_stat", _bf16(dy, "dy"), _bf16(y, "y"), M, N, int(d), _f32(s, "s"), _stream(stream))
    return s


def coda_colsum_reduce(partials, out=None, stream=None):
    """out[n] = sum_t partials[t, n] in the order t = 0, 1, ..."""
    torch = _torch()
    T, W = partials.shape
    out = _empty((W,), torch.float32, partials) if out is None else out
    _call("coda_colsum_reduce", _f32(partials, "partials"), T, W, _f32(out, "out"), _stream(stream))
    return out


def _bwd_dx(name, dy, w1, h1, gamma, r, s, g_res, dh1, dgamma_partials, stream, split=False, workspace=None):
    torch = _torch()
    M, N = dy.shape
    D = w1.shape[0]
    if w1.shape[1] != N or h1.shape != (M, D) or gamma.shape != (D,) or r.shape != (M,) or s.shape != (M,) \
            or (g_res is not None and g_res.shape != (M, D)):
        raise ValueError(f"{name}: inconsistent shapes")
    dh1 = _empty((M, D), torch.bfloat16, dy) if dh1 is None else dh1
    dgamma_partials = _empty((num_row_tiles(M), D), torch.float32, dy) if dgamma_partials is None else dgamma_partials
    ws = _split_args(split, lambda: coda_split_workspace_bytes(M, D, N), dy, workspace)
    _call(name, _bf16(dy, "dy"), _bf16(w1, "w1"), _bf16(h1, "h1"), _bf16(gamma, "gamma"), _f32(r, "r"),
          _f32(s, "s"), _opt_bf16(g_res, "g_res"), M, D, N, _bf16(dh1, "dh1"),
          _f32(dgamma_partials, "dgamma_partials"), *ws, _stream(stream))
    return dh1, dgamma_partials


def coda_gemm_rmsnorm_bwd_dx(dy, w1, h1, gamma, r, s, g_res=None, dh1=None, dgamma_partials=None, stream=None):
    """Grad GEMM dO = dy w1^T whose epilogue stores dh1 = r gamma dO - r^2 s h1 (+ g_res)
    and the dgamma column partials. Returns (dh1, dgamma_partials)."""
    return _bwd_dx("coda_gemm_rmsnorm_bwd_dx", dy, w1, h1, gamma, r, s, g_res, dh1, dgamma_partials, stream)


def coda_gemm_rmsnorm_bwd_dx_ws(dy, w1, h1, gamma, r, s, g_res=None, dh1=None, dgamma_partials=None, workspace=None,
                                stream=None):
    """coda_gemm_rmsnorm_bwd_dx with the split-depth schedule (output width D, depth N)."""
    return _bwd_dx("coda_gemm_rmsnorm_bwd_dx_ws", dy, w1, h1, gamma, r, s, g_res, dh1, dgamma_partials, stream, True,
                   workspace)


def coda_rmsnorm_bwd(dy, w1, h1, gamma, r, y, g_res=None, s=None, dh1=None, dgamma_partials=None, dgamma=None,
                     stream=None):
    """The rest of the RMSNorm backward: s from (dy, y), the grad GEMM with the
    RMSNorm-backward epilogue, and dgamma. Returns (s, dh1, dgamma_partials, dgamma)."""
    torch = _torch()
    M, N = dy.shape
    D = w1.shape[0]
    if w1.shape[1] != N or h1.shape != (M, D) or gamma.shape != (D,) or r.shape != (M,) or y.shape != (M, N) \
            or (g_res is not None and g_res.shape != (M, D)):
        raise ValueError("coda_rmsnorm_bwd: inconsistent shapes")
    s = _empty((M,), torch.float32, dy) if s is None else s
    dh1 = _empty((M, D), torch.bfloat16, dy) if dh1 is None else dh1
    dgamma_partials = _empty((num_row_tiles(M), D), torch.float32, dy) if dgamma_partials is None else dgamma_partials
    dgamma = _empty((D,), torch.float32, dy) if dgamma is None else dgamma
    _call("coda_rmsnorm_bwd", _bf16(dy, "dy"), _bf16(w1, "w1"), _bf16(h1, "h1"), _bf16(gamma, "gamma"),
          _f32(r, "r"), _bf16(y, "y"), _opt_bf16(g_res, "g_res"), M, D, N, _f32(s, "s"), _bf16(dh1, "dh1"),
          _f32(dgamma_partials, "dgamma_partials"), _f32(dgamma, "dgamma"), _stream(stream))
    return s, dh1, dgamma_partials, dgamma


# ------------------------------------------------------------------- unfused baselines
def coda_baseline_gemm(a, b, b_kn=True, c=None, stream=None):
    torch = _torch()
    M, K = a.shape
    N = b.shape[1] if b_kn else b.shape[0]
    if (b.shape[0] if b_kn else b.shape[1]) != K:
        raise ValueError("coda_baseline_gemm: inconsistent shapes")
    c = _empty((M, N), torch.bfloat16, a) if c is None else c
    _call("coda_baseline_gemm", _bf16(a, "a"), _bf16(b, "b"), M, K, N, 1 if b_kn else 0, _bf16(c, "c"),
          _stream(stream))
    return c


def coda_baseline_residual_rmsnorm(h0, z, gamma, eps, h1=None, r=None, o=None, stream=None):
    torch = _torch()
    M, D = h0.shape
    h1 = _empty((M, D), torch.bfloat16, h0) if h1 is None else h1
    o = _empty((M, D), torch.bfloat16, h0) if o is None else o
    r = _empty((M,), torch.float32, h0) if r is None else r
    _call("coda_baseline_residual_rmsnorm", _bf16(h0, "h0"), _bf16(z, "z"), _bf16(gamma, "gamma"), M, D,
          float(eps), _bf16(h1, "h1"), _f32(r, "r"), _bf16(o, "o"), _stream(stream))
    return h1, r, o


def coda_baseline_rope(h, cos_t, sin_t, n_q, n_k, n_v, head_dim, seq_len, pos_offset=0, out=None, stream=None):
    torch = _torch()
    M = h.shape[0]
    out = _empty(h.shape, torch.bfloat16, h) if out is None else out
    _call("coda_baseline_rope", _bf16(h, "h"), _f32(cos_t, "cos_t"), _f32(sin_t, "sin_t"), M, n_q, n_k, n_v,
          head_dim, seq_len, pos_offset, _bf16(out, "out"), _stream(stream))
    return out


def coda_baseline_swiglu(h, out=None, stream=None):
    torch = _torch()
    M, N2 = h.shape
    F = N2 // 2
    out = _empty((M, F), torch.bfloat16, h) if out is None else out
    _call("coda_baseline_swiglu", _bf16(h, "h"), M, F, _bf16(out, "out"), _stream(stream))
    return out


def coda_baseline_rowdot(a, b, s=None, stream=None):
    torch = _torch()
    M, D = a.shape
    s = _empty((M,), torch.float32, a) if s is None else s
    _call("coda_baseline_rowdot", _bf16(a, "a"), _bf16(b, "b"), M, D, _f32(s, "s"), _stream(stream))
    return s


def coda_baseline_copy(src, dst, stream=None):
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("coda_baseline_copy: size mismatch")
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("coda_baseline_copy: contiguous GPU tensors required")
    _call("coda_baseline_copy", ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
          src.numel() * src.element_size(), _stream(stream))
    return dst


def coda_baseline_mfma_loop(operands, iters, grid, out=None, stream=None):
    """Register-only MFMA loop over bf16 `operands` (numel a multiple of 8); returns the
    per-thread sums [grid * 512] fp32. FLOPs = grid * 8 * iters * 32 * 16384."""
    torch = _torch()
    if operands.numel() % 8:
        raise ValueError("coda_baseline_mfma_loop: operands must hold whole 8-element fragments")
    out = _empty((grid * 512,), torch.float32, operands) if out is None else out
    _call("coda_baseline_mfma_loop", _bf16(operands, "operands"), operands.numel() // 8, int(iters), int(grid),
          _f32(out, "out"), _stream(stream))
    return out


def coda_baseline_schedule_probe(kind, steps, grid, fill=0.125, seed=0, out=None, cycles=None, device="cuda",
                                 stream=None):
    """The main loop's LDS reads and MFMAs on a fixed LDS image (every element `fill`, or
    hashed bits when seed != 0; kind 0: KN-W reads with the per-step barrier, 1: without
    it, 2: NK-W reads, 3: the reads of kind 0 alone, 4: its MFMAs alone);
    returns (out [grid * 512] fp32, cycles [grid * 8] int64 per wave over `steps` steps)."""
    torch = _torch()
    out = torch.empty((grid * 512,), dtype=torch.float32, device=device) if out is None else out
    cycles = torch.empty((grid * 8,), dtype=torch.int64, device=device) if cycles is None else cycles
    if out.numel() < grid * 512 or cycles.numel() < grid * 8:
        raise ValueError("coda_baseline_schedule_probe: out or cycles too small for the grid")
    _call("coda_baseline_schedule_probe", int(kind), int(steps), int(grid), float(fill), int(seed), _f32(out, "out"),
          _dev(cycles, torch.int64, "cycles"), _stream(stream))
    return out, cycles
