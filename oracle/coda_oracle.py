"""Plain, slow, obviously correct fp64 CPU oracle of the GEMM-epilogue hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path. It shares no code,
header, table or constant generator with the HIP library.

Sources (the paper is "CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs",
arXiv 2605.19269; two web pages about it are used):
  [notes]  papernotes.org notes page, section "方法详解" (method), "关键设计" 1-4
           (key designs 1-4) and their displayed equations;
  [pith]   pith.science page: Figure 4 and Figure 5 captions (two-level reduction and
           the formula for r), Figure 7 caption (pairwise activations), and the
           fragments of Appendix A.1 / Listing 2 (the epilogue visitor list
           EVTResidual, EVTColBlockReductionStore, EVTRowVecMulPostAct).

Conventions
  * Every input is taken as bf16 bit patterns (``uint16``) and decoded *exactly* to
    fp64 by :func:`decode_bf16`. fp32 inputs (RoPE tables are never used here) stay
    fp32 -> fp64. Nothing is rounded afterwards: all arithmetic is fp64.
  * Every operation on the path is independent across rows (tokens), so every
    function takes an optional ``rows`` index array and then computes exactly those
    rows of the full result (row sampling for large workloads).
  * Matrix products use ``numpy.matmul`` in float64, a library primitive; nothing is
    blocked, fused or reordered beyond the definitions below.

Readings where the pages are silent, garbled or inconsistent (each is also listed in
the design notes of the repository):
  R1  eps sits inside the square root: r = 1 / sqrt(mean(h1^2) + eps) ([pith] Fig. 5
      caption prints the formula with the radical sign lost; the standard RMSNorm).
  R2  The tile partial is a *sum* of squares over a 256-column tile; the reduction
      divides by the full width d. (The listing stores a block mean with
      inv_block_size = 1/tile_N; both agree when the tile divides d, and the sum is
      right for a ragged last tile.)
  R3  The square is taken of h1 = x W0 + z before gamma and before any rounding
      ([notes] key design 1: r = 1/rms(x W0 + z); Listing 2: the partial is taken on
      the unscaled D, the main output D stays unscaled).
  R4  GEMM2 consumes h2 = h1 * gamma (not normalised) and r multiplies its
      accumulator: y[i, j] = r[i] * h3[i, j], h3 = h2 W1 ([notes] key design 1).
  R5  RoPE: theta_p = theta^(-2p/head_dim) for the pair p of adjacent columns
      (2p, 2p+1) inside a head; the pair is rotated by [[cos a, -sin a],
      [sin a, cos a]] with a = pos * theta_p, pos = (row + pos_offset) mod seq_len;
      the output is [Q | K | V] in contiguous blocks, V unrotated.
  R6  SwiGLU: even accumulator column = gate G, odd = up U, out = silu(G) * U with
      silu(g) = g / (1 + exp(-g)); the output width is half the accumulator width.
  R7  Backward statistic: h2 is the GEMM2 input and y = h2 W1 ([notes] key design 3);
      s = (1/d) sum_cols(dY W1^T * h2), also computed as (1/d) sum(dY * y).
  R8  Rest of the RMSNorm backward ([notes] key design 3 and the duality paragraph
      before its statistic; [pith] Fig. 9): the forward is o = r h1 gamma (the GEMM2
      input of R7, normalised), y = o W1. With dO = dY W1^T the chain rule gives
      dh1 = r gamma dO - r^2 s h1 with s = (1/d) sum_cols(dO * o), plus the gradient
      g_res that reaches h1 through the residual stream; dgamma = sum_rows(dO r h1).
      Column partials of dgamma are sums over 256-row tiles, like R2's row partials.
  R9  SwiGLU backward ([notes] key design 2, last item; [pith] Fig. 7: the backward
      maps one incoming gradient into gradients for both paired inputs): the grad GEMM
      dOut = dY W_down^T (W_down [F, Dm] is the forward down projection) meets the
      saved interleaved pre-activations h = [G_0, U_0, G_1, U_1, ...]; out =
      silu(G) U gives dG = dOut U silu'(G), dU = dOut silu(G) with
      silu'(g) = s(g) (1 + g (1 - s(g))), s the logistic function; dh is interleaved
      like h.
  R10 RoPE backward: the rotation is orthogonal, so the gradient through it is the
      rotation by the negated angle (R5 with -pos); fused into the GEMM that produces
      the gradient of the rotated Q and K, it is that GEMM's epilogue.
  R11 GEMM + cross-entropy ([notes] method overview: the cross-entropy log-sum-exp is a
      cross-tile statistic produced as tile partials and reduced by an auxiliary
      kernel; the five primitives, (5) stateful transforms such as an online
      log-sum-exp): logits = x W are never stored; each 256-column tile yields, per row,
      the log-sum-exp of its columns; the auxiliary step merges them,
      lse = log sum_t exp(lse_t), and loss = lse - logits[label]. A label outside
      [0, V) marks an ignored row: loss 0.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "PARTIAL_TILE_N",
    "decode_bf16",
    "matmul",
    "tile_row_sums",
    "rowstat_reduce",
    "gemm_rmsnorm_fwd",
    "rmsnorm_rows",
    "rope_rotate",
    "gemm_rope",
    "silu",
    "gemm_swiglu",
    "gemm_rmsnorm_bwd_stats",
    "rmsnorm_bwd",
    "silu_grad",
    "gemm_swiglu_bwd",
    "gemm_rope_bwd",
    "logsumexp_rows",
    "gemm_cross_entropy",
    "flops_gemm_rmsnorm_fwd",
]

# Width of one column tile of the partial-statistic workspace [M, nb]: tile t covers
# columns [t*256, (t+1)*256) (the last tile may be ragged). This is the layout
# contract of the workspace, stated by the library's interface documentation.
PARTIAL_TILE_N = 256
# Height of one row tile of the column-partial workspace [ceil(M/256), D] of dgamma.
PARTIAL_TILE_M = 256


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values.

    bf16 is the upper half of an IEEE-754 binary32: placing the 16 bits in the high
    half of a 32-bit word gives the fp32 number exactly, which widens exactly to fp64.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("decode_bf16 expects uint16 bit patterns")
    u32 = b.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return decode_bf16(a)
    return a.astype(np.float64)


def _take_rows(a: np.ndarray, rows):
    return a if rows is None else a[np.asarray(rows)]


def matmul(a, b) -> np.ndarray:
    """fp64 matrix product a @ b (a: [M, K], b: [K, N])."""
    a = _as_f64(a)
    b = _as_f64(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"matmul shape mismatch {a.shape} @ {b.shape}")
    return np.matmul(a, b)


def tile_row_sums(v: np.ndarray, tile_n: int = PARTIAL_TILE_N) -> np.ndarray:
    """Per-row sums of ``v`` over consecutive column tiles of width ``tile_n``.

    Returns P[m, t] = sum_{n in [t*tile_n, (t+1)*tile_n) and n < width} v[m, n]
    ([pith] Listing 2, EVTColBlockReductionStore: one value per row and N-block;
    reading R2: sums, not means).
    """
    M, W = v.shape
    nb = -(-W // tile_n) if W else 0
    P = np.zeros((M, nb), dtype=np.float64)
    for t in range(nb):
        P[:, t] = v[:, t * tile_n:min((t + 1) * tile_n, W)].sum(axis=1)
    return P


def rowstat_reduce(partials, d: int, eps: float = 0.0, mode: str = "rsqrt_mean_eps") -> np.ndarray:
    """The auxiliary row reduction over tile partials ([pith] Fig. 4 and Fig. 5).

    mode "rsqrt_mean_eps": r[m] = 1 / sqrt(sum_t P[m, t] / d + eps)   (forward r)
    mode "mean":           s[m] = sum_t P[m, t] / d                   (backward s)
    """
    P = _as_f64(partials)
    total = P.sum(axis=1)
    if mode == "rsqrt_mean_eps":
        return 1.0 / np.sqrt(total / d + eps)
    if mode == "mean":
        return total / d
    raise ValueError(mode)


def rmsnorm_rows(h: np.ndarray, gamma: np.ndarray, eps: float):
    """Textbook RMSNorm of each row: returns (r, r * h * gamma) with
    r = 1 / sqrt(mean(h^2) + eps) (reading R1)."""
    ms = np.mean(h * h, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    return r, (r[:, None] * h) * gamma[None, :]


def gemm_rmsnorm_fwd(x, w0, z, gamma, w1, eps: float, rows=None,
                     tile_n: int = PARTIAL_TILE_N) -> dict:
    """y = RMSNorm(x W0 + z, gamma) W1, unfused, plus the rewrite's intermediates.

    Follows [notes] key design 1 (both displayed equations) and [pith] Fig. 4:
      h0 = x W0;  h1 = h0 + z;  r = 1/rms(h1);  y = (r h1 * gamma) W1     (direct)
      h2 = h1 * gamma;  h3 = h2 W1;  y_deferred[i, j] = r[i] h3[i, j]      (deferred r)
      partials = per-tile row sums of h1^2                                 (two-level r)
    Returns fp64 arrays h1, h2, partials, r, y, y_deferred for the selected rows.
    """
    xr = _take_rows(_as_f64(x), rows)
    zr = _take_rows(_as_f64(z), rows)
    W0 = _as_f64(w0)
    W1 = _as_f64(w1)
    g = _as_f64(gamma)
    h0 = matmul(xr, W0)
    h1 = h0 + zr
    r, normed = rmsnorm_rows(h1, g, eps)
    y = matmul(normed, W1)
    h2 = h1 * g[None, :]
    h3 = matmul(h2, W1)
    y_def = r[:, None] * h3
    partials = tile_row_sums(h1 * h1, tile_n)
    return dict(h1=h1, h2=h2, partials=partials, r=r, y=y, y_deferred=y_def)


def rope_rotate(h: np.ndarray, positions: np.ndarray, n_q: int, n_k: int, n_v: int,
                head_dim: int, theta: float) -> np.ndarray:
    """Rotary position embedding of the Q and K blocks of h = [Q | K | V] (reading R5).

    Each head's adjacent columns (2p, 2p+1) form one 2-D vector that is rotated by the
    angle pos * theta^(-2p/head_dim) ([notes] key design 2; [pith] Fig. 7: RoPE
    rotates each feature pair and returns two outputs). V is returned unchanged.
    """
    assert h.shape[1] == n_q + n_k + n_v
    assert head_dim % 2 == 0 and n_q % head_dim == 0 and n_k % head_dim == 0
    out = h.copy()
    half = head_dim // 2
    p = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * p / head_dim)              # [half]
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]   # [rows, half]
    c, s = np.cos(ang), np.sin(ang)
    for base, width in ((0, n_q), (n_q, n_k)):
        for h0 in range(base, base + width, head_dim):
            e = h[:, h0:h0 + head_dim:2]
            o = h[:, h0 + 1:h0 + head_dim:2]
            out[:, h0:h0 + head_dim:2] = e * c - o * s
            out[:, h0 + 1:h0 + head_dim:2] = e * s + o * c
    return out


def gemm_rope(x, w, n_q: int, n_k: int, n_v: int, head_dim: int, seq_len: int,
              pos_offset: int = 0, theta: float = 10000.0, rows=None) -> np.ndarray:
    """QKV projection followed by RoPE on Q and K: out = rope(x W).

    The position of row i is (i + pos_offset) mod seq_len. The angles come from fp64
    trigonometry directly, not from any precomputed table.
    """
    M = np.asarray(x).shape[0]
    idx = np.arange(M) if rows is None else np.asarray(rows)
    h = matmul(_take_rows(_as_f64(x), rows), w)
    pos = (idx + pos_offset) % seq_len
    return rope_rotate(h, pos, n_q, n_k, n_v, head_dim, theta)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in fp64 (exp overflow for g << 0 gives -0)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gemm_swiglu(x, w, rows=None) -> np.ndarray:
    """h = x W with interleaved columns; out[m, j] = silu(h[m, 2j]) * h[m, 2j+1]
    ([notes] key design 2: even channel G, odd channel U, width halved; reading R6)."""
    h = matmul(_take_rows(_as_f64(x), rows), w)
    if h.shape[1] % 2:
        raise ValueError("SwiGLU needs an even accumulator width")
    G = h[:, 0::2]
    U = h[:, 1::2]
    return silu(G) * U


def gemm_rmsnorm_bwd_stats(dy, w1, h2, rows=None, tile_n: int = PARTIAL_TILE_N) -> dict:
    """Grad GEMM dH2 = dY W1^T and the RMSNorm-backward row statistic s.

    [notes] key design 3: with grad_h2 = dY W1^T and y = h2 W1,
        s = (1/d) sum_cols(grad_h2 * h2) = (1/d) diag(dY (h2 W1)^T) = (1/d) sum(dY * y).
    Returns dh2, partials (per-tile row sums of dH2 * h2), s (first form) and
    s_prime (last form), for the selected rows; d is the width of h2.
    """
    dyr = _take_rows(_as_f64(dy), rows)
    h2r = _take_rows(_as_f64(h2), rows)
    W1 = _as_f64(w1)
    d = h2r.shape[1]
    dh2 = matmul(dyr, W1.T)
    prod = dh2 * h2r
    s = prod.sum(axis=1) / d
    y = matmul(h2r, W1)
    s_prime = (dyr * y).sum(axis=1) / d
    s_diag = np.diag(matmul(dyr, y.T)) / d if dyr.shape[0] <= 512 else None
    return dict(dh2=dh2, partials=tile_row_sums(prod, tile_n), s=s, s_prime=s_prime,
                s_diag=s_diag)


def rmsnorm_bwd(h1, gamma, w1, dy, eps: float, g_res=None, rows=None, cols=None,
                tile_m: int = PARTIAL_TILE_M) -> dict:
    """Rest of the RMSNorm backward around the grad GEMM (reading R8).

    Forward, non-deferred form of [notes] key design 1: r = 1/sqrt(mean(h1^2) + eps),
    o = r * h1 * gamma (GEMM2 input), y = o W1. With upstream gradient dY [M, N]:
        dO     = dY W1^T                                  (the grad GEMM)
        s      = (1/d) sum_cols(dO * o) = (1/d) sum(dY * y)  (key design 3)
        dh1    = r * gamma * dO - r^2 * s * h1  (+ g_res)
        dgamma = sum_rows(dO * r * h1)
    Derivation: o_k = r h1_k gamma_k and dr/dh1_j = -r^3 h1_j / d, so
    dh1_j = r gamma_j dO_j - (r^3 h1_j / d) sum_k dO_k gamma_k h1_k = r gamma_j dO_j -
    r^2 s h1_j.

    Row outputs (r, y, s, s_out, dh1) are for the selected ``rows`` (all by default).
    ``dgamma`` sums over all rows of the input (or only the selected rows when ``rows``
    is given); ``cols`` limits the dgamma / dgamma_partials columns (cheap at full size:
    only those columns of dO are formed). ``dgamma_partials[t, c]`` sums rows
    [t*tile_m, (t+1)*tile_m) of the selected rows' order.
    """
    H1 = _as_f64(h1)
    G = _as_f64(gamma)
    W1 = _as_f64(w1)
    DY = _as_f64(dy)
    d = H1.shape[1]
    h1r = _take_rows(H1, rows)
    dyr = _take_rows(DY, rows)
    r = 1.0 / np.sqrt((h1r * h1r).sum(axis=1) / d + eps)
    o = r[:, None] * h1r * G[None, :]
    y = matmul(o, W1)
    dO = matmul(dyr, W1.T)
    s = (dO * o).sum(axis=1) / d
    s_out = (dyr * y).sum(axis=1) / d
    dh1 = r[:, None] * G[None, :] * dO - (r * r * s)[:, None] * h1r
    if g_res is not None:
        dh1 = dh1 + _take_rows(_as_f64(g_res), rows)
    c = np.arange(d) if cols is None else np.asarray(cols)
    dO_c = dO[:, c] if cols is None else matmul(dyr, W1[c, :].T)
    contrib = dO_c * r[:, None] * h1r[:, c]
    nt = (contrib.shape[0] + tile_m - 1) // tile_m
    parts = np.stack([contrib[t * tile_m:(t + 1) * tile_m].sum(axis=0) for t in range(nt)])
    return dict(r=r, y=y, dO=dO, s=s, s_out=s_out, dh1=dh1, dgamma=contrib.sum(axis=0),
                dgamma_partials=parts, cols=c)


def silu_grad(g: np.ndarray) -> np.ndarray:
    """d/dg of g / (1 + exp(-g)) = s(g) + g s(g) (1 - s(g)), s the logistic function."""
    sig = 1.0 / (1.0 + np.exp(-g))
    return sig * (1.0 + g * (1.0 - sig))


def gemm_swiglu_bwd(dy, w_down, h, rows=None) -> dict:
    """SwiGLU backward through the grad GEMM of the down projection (reading R9).

    dOut = dY W_down^T (dY [M, Dm], W_down [F, Dm]); with G = h[:, 0::2], U = h[:, 1::2]
    the saved pre-activations, dG = dOut U silu'(G) and dU = dOut silu(G), returned
    interleaved as dh [M, 2F] (dh[:, 2j] = dG_j, dh[:, 2j+1] = dU_j).
    """
    dout = matmul(_take_rows(_as_f64(dy), rows), _as_f64(w_down).T)
    H = _take_rows(_as_f64(h), rows)
    if H.shape[1] != 2 * dout.shape[1]:
        raise ValueError("h must be [M, 2F] for dOut [M, F]")
    G = H[:, 0::2]
    U = H[:, 1::2]
    dh = np.empty_like(H)
    dh[:, 0::2] = dout * U * silu_grad(G)
    dh[:, 1::2] = dout * silu(G)
    return dict(dout=dout, dh=dh)


def gemm_rope_bwd(x, w, n_q: int, n_k: int, n_v: int, head_dim: int, seq_len: int,
                  pos_offset: int = 0, theta: float = 10000.0, rows=None) -> np.ndarray:
    """The GEMM x W followed by the RoPE backward on Q and K (reading R10): each pair is
    rotated by -pos * theta_p, the transpose of the forward rotation; V is unchanged."""
    M = np.asarray(x).shape[0]
    idx = np.arange(M) if rows is None else np.asarray(rows)
    h = matmul(_take_rows(_as_f64(x), rows), w)
    pos = (idx + pos_offset) % seq_len
    return rope_rotate(h, -pos, n_q, n_k, n_v, head_dim, theta)


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """log sum_j exp(z[i, j]) per row, shifted by the row maximum (exact in fp64 for the
    ranges here); rows of -inf only give -inf."""
    mx = z.max(axis=1)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    return safe + np.log(np.exp(z - safe[:, None]).sum(axis=1))


def gemm_cross_entropy(x, w, labels, rows=None, tile_n: int = PARTIAL_TILE_N) -> dict:
    """Cross-entropy of the logits x W against integer labels (reading R11).

    Returns, for the selected rows: the per-tile log-sum-exp partials [rows, nb] over
    256-column tiles, the full lse, the target logit (0 for ignored rows), and
    loss = lse - target (0 for ignored rows: label outside [0, V)).
    """
    z = matmul(_take_rows(_as_f64(x), rows), w)
    V = z.shape[1]
    lab = _take_rows(np.asarray(labels).astype(np.int64), rows)
    nb = (V + tile_n - 1) // tile_n
    tile_lse = np.stack([logsumexp_rows(z[:, t * tile_n:(t + 1) * tile_n]) for t in range(nb)], axis=1)
    lse = logsumexp_rows(z)
    valid = (lab >= 0) & (lab < V)
    target = np.where(valid, z[np.arange(z.shape[0]), np.clip(lab, 0, V - 1)], 0.0)
    loss = np.where(valid, lse - target, 0.0)
    return dict(tile_lse=tile_lse, lse=lse, target=target, loss=loss, valid=valid)


def flops_gemm_rmsnorm_fwd(M: int, K: int, D: int, N1: int) -> int:
    """Algorithmic flops of the forward rewrite: the two GEMMs (2MKD + 2MDN1)."""
    return 2 * M * K * D + 2 * M * D * N1
