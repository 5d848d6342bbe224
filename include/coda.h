/*
 * coda.h -- C ABI of libcoda.so: bf16 GEMMs on gfx950 (AMD Instinct MI355X) whose
 * epilogues finish the Transformer's memory-bound operators while the output tile is
 * still on chip, after the method of "CODA: Rewriting Transformer Blocks as
 * GEMM-Epilogue Programs" (arXiv 2605.19269).
 *
 * Sources cited below:
 *   [notes] the papernotes.org notes on CODA: section "方法详解" (method), key designs
 *           ("关键设计") 1 to 4 and their displayed equations;
 *   [pith]  the pith.science page on CODA: captions of Figures 4, 5 and 7 and the
 *           fragments of Appendix A.1 / Listing 2 (epilogue visitors EVTResidual,
 *           EVTColBlockReductionStore, EVTRowVecMulPostAct).
 *
 * Conventions for every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns; outputs are rounded from fp32
 *     to bf16 with round-to-nearest-even. fp32 tensors are plain IEEE floats.
 *   - Every tensor is a dense row-major array in DEVICE memory (hipMalloc'd or a torch
 *     CUDA tensor's data pointer), and every bf16 pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream. All work is
 *     enqueued on that stream, asynchronously; the call returns before it finishes.
 *   - Ownership: the caller owns and allocates every buffer, workspaces included. The
 *     library allocates no device memory, keeps no state between calls and may be
 *     called from several host threads at once (on different buffers). The one
 *     exception is coda_gemm_rmsnorm_fwd_noalloc, which keeps its row partials in a
 *     fixed device array of the library (see there).
 *   - Aliasing: an output buffer may overlap neither an input nor another output
 *     (byte ranges of the sizes the call implies); such a call returns CODA_ERR_ARG.
 *     Inputs are only read and may alias each other.
 *   - Errors: argument errors are detected before anything is enqueued and return a
 *     nonzero status (nothing is written). A failed kernel launch returns
 *     CODA_ERR_HIP. Faults during execution surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.
 *   - Shapes: M (rows / tokens) may be any value from 0 to 16777216 (2^24; M == 0 is a
 *     no-op returning CODA_OK). Depth K and every output width must be positive
 *     multiples of 8, and at most 4194304 (2^22); so a GEMM has fewer than 2^30 output
 *     tiles. Any M is handled by row predication; ragged K and widths by zero-filled
 *     tails. Larger sizes return CODA_ERR_SHAPE.
 *   - Accumulation is fp32 on the MFMA units; epilogue math is fp32; only stores round.
 *   - Results are deterministic: no atomics, fixed summation orders.
 */
#ifndef CODA_H
#define CODA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define CODA_OK 0
#define CODA_ERR_NULL 1      /* a required pointer is NULL */
#define CODA_ERR_SHAPE 2     /* a size violates the shape rules above */
#define CODA_ERR_ALIGN 3     /* a bf16 pointer is not 16-byte aligned (fp32: 8-byte) */
#define CODA_ERR_WORKSPACE 4 /* the workspace a call needs exceeds what it has */
#define CODA_ERR_HIP 5       /* a HIP launch failed */
#define CODA_ERR_ARG 6       /* another argument is invalid (mode, eps, theta, overlap) */

/* Width of one column tile of the row-partial workspace: partial t of a row covers
 * output columns [t*256, (t+1)*256) (the last tile may be ragged). */
#define CODA_PARTIAL_TILE_N 256

/* Modes of coda_rowstat_reduce. */
#define CODA_ROWSTAT_RSQRT_MEAN_EPS 0 /* out[m] = 1 / sqrt(sum_t P[m,t] / d + eps) */
#define CODA_ROWSTAT_MEAN 1           /* out[m] = sum_t P[m,t] / d                  */

/* Human-readable name of a status code (static string, never NULL). */
const char* coda_status_string(int status);

/* ABI version of this header (major * 100 + minor): 101 adds the split-depth forward
 * and the schedule probe to 100; 102 adds the split-depth backward and cross-entropy
 * entry points; 103 adds coda_split_plan. */
int coda_abi_version(void);

/* SHA-256 (64 hex digits, static string) of the sources and compile flags this library
 * was built from, as computed by the build step; "unknown" for a build that did not
 * set it. Lets a loader refuse a library that is stale against its sources. */
const char* coda_build_source_hash(void);

/* Number of row partials nb = ceil(width / CODA_PARTIAL_TILE_N) that the epilogues
 * write per row for an output of `width` columns. Returns CODA_ERR_NULL or
 * CODA_ERR_SHAPE (width < 1). */
int coda_rowstat_num_partials(int width, int* nb);

/* ---------------------------------------------------------------------------------
 * Forward GEMM-RMSNorm-GEMM, [notes] key design 1 (both equations) and [pith] Fig. 4:
 *     y = RMSNorm(x W0 + z, gamma) W1 = r ((x W0 + z) * gamma) W1,  r = 1 / rms(x W0 + z)
 * computed as three launches on `stream`:
 *   (1) GEMM1 x W0 whose epilogue adds the residual, h1 = acc + z (stored), scales by
 *       gamma into the side output h2 = h1 * gamma (stored), and writes per-tile row
 *       partials P[m, t] = sum over the tile's columns of h1^2 taken from the fp32 h1
 *       before any rounding ([pith] Listing 2: the square is of the unscaled output);
 *   (2) the auxiliary reduction r[m] = 1 / sqrt(sum_t P[m, t] / D + eps)
 *       ([pith] Fig. 4 and the formula under Fig. 5);
 *   (3) GEMM2 h2 W1 whose epilogue applies the deferred row scale,
 *       y[i, j] = r[i] * (h2 W1)[i, j] ([notes] key design 1).
 * Arguments
 *   x [M,K], w0 [K,D], z [M,D], gamma [D], w1 [D,N1]: bf16 inputs (read only).
 *   eps: >= 0 and finite, added to the mean square inside the square root.
 *   h1 [M,D], h2 [M,D]: bf16 outputs (h2 is also GEMM2's input).
 *   partials [M, nb] fp32 workspace/output, nb = coda_rowstat_num_partials(D).
 *   r [M] fp32 output.  y [M,N1] bf16 output.
 * Output buffers must not overlap inputs or each other (CODA_ERR_ARG).
 * ------------------------------------------------------------------------------- */
int coda_gemm_rmsnorm_fwd(const uint16_t* x, const uint16_t* w0, const uint16_t* z,
                          const uint16_t* gamma, const uint16_t* w1, int M, int K, int D,
                          int N1, float eps, uint16_t* h1, uint16_t* h2, float* partials,
                          float* r, uint16_t* y, void* stream);

/* coda_gemm_rmsnorm_fwd with a split-depth schedule for outputs with fewer 256 x 256
 * tiles than the current device has compute units (small batches, one GPU's share of a
 * token-sharded batch). The same steps (1)-(3), where a GEMM with too few tiles cuts
 * each tile's depth into S equal slices, runs one workgroup per slice (fp32 partial
 * tiles into `workspace`) and then one per tile that sums the S partials in slice order
 * and runs the tile's epilogue, (1) or (3) above, on the sum. A GEMM with at most half
 * as many tiles as CUs splits every tile. A larger one whose last wave of tiles (one per
 * CU) is at most half full runs its full waves as coda_gemm_rmsnorm_fwd does and splits
 * only the last wave's tiles. Any other GEMM runs as in coda_gemm_rmsnorm_fwd. Results
 * are deterministic for a given shape and device; a split tile's fp32 rounding differs
 * from coda_gemm_rmsnorm_fwd's by the order of the depth sum, within the same tolerance
 * against exact arithmetic.
 * workspace: caller-owned device memory of workspace_bytes bytes, 16-byte aligned, at
 * least coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1) (else CODA_ERR_WORKSPACE;
 * may be NULL when that is 0); read and written by the call, overlapping no other
 * argument (CODA_ERR_ARG). Calls that overlap in time must not share a workspace.
 * Three to five launches on `stream`. Other arguments, rules and errors as
 * coda_gemm_rmsnorm_fwd; a negative workspace_bytes is CODA_ERR_ARG. */
int coda_gemm_rmsnorm_fwd_ws(const uint16_t* x, const uint16_t* w0, const uint16_t* z,
                             const uint16_t* gamma, const uint16_t* w1, int M, int K, int D,
                             int N1, float eps, uint16_t* h1, uint16_t* h2, float* partials,
                             float* r, uint16_t* y, void* workspace, long long workspace_bytes,
                             void* stream);
/* Bytes of workspace coda_gemm_rmsnorm_fwd_ws needs on the current device (0 when no
 * GEMM of the shape is split): 256 KiB per slice of every split tile of the GEMM that
 * needs more.
 * Shape rules as coda_gemm_rmsnorm_fwd; CODA_ERR_HIP if the device cannot be queried. */
int coda_gemm_rmsnorm_fwd_workspace_bytes(int M, int K, int D, int N1, long long* bytes);

/* Capacity, in fp32 values, of the fixed device array that coda_gemm_rmsnorm_fwd_noalloc
 * uses as its row-partial workspace (4 MiB per GPU). */
#define CODA_NOALLOC_SCRATCH_FLOATS (1 << 20)

/* coda_gemm_rmsnorm_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same three
 * launches and bit-identical h1, h2, r and y, with the row partials kept in a fixed
 * device array inside the library instead of a caller's buffer. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); the first call on a
 * device looks up that device's copy of the array.
 * Limits and sharing: M * nb <= CODA_NOALLOC_SCRATCH_FLOATS with nb =
 * coda_rowstat_num_partials(D) (e.g. M <= 65536 at D = 4096), else CODA_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's array, and every partial is written before it
 * is read, so nothing needs clearing between calls; but calls whose work overlaps in time
 * on one GPU (different streams, or different host threads) race on the array and give
 * undefined results. Other arguments, rules and errors as coda_gemm_rmsnorm_fwd. */
int coda_gemm_rmsnorm_fwd_noalloc(const uint16_t* x, const uint16_t* w0, const uint16_t* z,
                                  const uint16_t* gamma, const uint16_t* w1, int M, int K,
                                  int D, int N1, float eps, uint16_t* h1, uint16_t* h2,
                                  float* r, uint16_t* y, void* stream);

/* Stage (1) of coda_gemm_rmsnorm_fwd alone (same arguments and outputs). */
int coda_gemm_residual_rmsnorm_partials(const uint16_t* x, const uint16_t* w0,
                                        const uint16_t* z, const uint16_t* gamma, int M,
                                        int K, int D, uint16_t* h1, uint16_t* h2,
                                        float* partials, void* stream);

/* Stage (3) of coda_gemm_rmsnorm_fwd alone: y[i, j] = r[i] * (h2 W1)[i, j].
 * h2 [M,D] bf16, w1 [D,N1] bf16, r [M] fp32 -> y [M,N1] bf16. */
int coda_gemm_rowscale(const uint16_t* h2, const uint16_t* w1, const float* r, int M, int D,
                       int N1, uint16_t* y, void* stream);

/* The auxiliary row reduction over tile partials ([pith] Fig. 4; [notes] key
 * design 1 for r, key design 3 for s). partials [M, nb] fp32 row-major; out [M] fp32.
 * Each row is summed in the fixed order t = 0 .. nb-1, then divided by d (> 0).
 * mode CODA_ROWSTAT_RSQRT_MEAN_EPS: out = 1 / sqrt(sum / d + eps) (eps >= 0);
 * mode CODA_ROWSTAT_MEAN: out = sum / d (eps ignored). nb >= 1. */
int coda_rowstat_reduce(const float* partials, int M, int nb, int d, float eps, int mode,
                        float* out, void* stream);

/* ---------------------------------------------------------------------------------
 * RoPE tables: cos_t[p_os, p] = cos(p_os * theta^(-2p/head_dim)) and sin_t likewise,
 * for p_os in [0, seq_len), p in [0, head_dim/2), computed in fp64 on the device and
 * rounded to fp32 (the tables the QKV epilogue reads; [notes] key design 2: the
 * sin/cos vectors are precomputed and broadcast). cos_t, sin_t: [seq_len, head_dim/2]
 * fp32 outputs, 8-byte aligned. head_dim even and >= 2, seq_len >= 1, theta > 0.
 * ------------------------------------------------------------------------------- */
int coda_rope_tables(float* cos_t, float* sin_t, int seq_len, int head_dim, double theta,
                     void* stream);

/* GEMM + RoPE for the fused QKV projection ([notes] key design 2; [pith] Fig. 7: each
 * adjacent feature pair is rotated in registers and yields two outputs).
 *   h = x W with x [M,K] bf16 and w [K, n_q+n_k+n_v] bf16; the output out [M, n_q+n_k+n_v]
 *   bf16 holds [Q | K | V] in contiguous column blocks. In the Q and K blocks, within
 *   each head of head_dim columns, the pair (2p, 2p+1) of row i is rotated by the angle
 *   pos * theta_p with pos = (i + pos_offset) mod seq_len:
 *       out[2p] = h[2p] cos - h[2p+1] sin,   out[2p+1] = h[2p] sin + h[2p+1] cos,
 *   where cos/sin = cos_t/sin_t[pos, p] (from coda_rope_tables). V is stored unrotated.
 * Rules: head_dim % 8 == 0; n_q, n_k, n_v >= 0 multiples of head_dim with a positive
 * sum; seq_len >= 1 (else CODA_ERR_ARG); seq_len * head_dim <= 2^29 (tables under 2^31
 * bytes, else CODA_ERR_SHAPE); pos_offset >= 0. */
int coda_gemm_rope(const uint16_t* x, const uint16_t* w, const float* cos_t,
                   const float* sin_t, int M, int K, int n_q, int n_k, int n_v, int head_dim,
                   int seq_len, int pos_offset, uint16_t* out, void* stream);

/* coda_gemm_rope with the split-depth schedule of coda_gemm_rmsnorm_fwd_ws (outputs of
 * at most half as many 256 x 256 tiles as the current device has CUs split every tile;
 * a larger output's at most half-full last wave splits its tiles): `workspace` holds at least
 * coda_split_workspace_bytes(M, n_q + n_k + n_v, K) bytes (16-byte aligned; NULL when
 * that is 0; overlapping no other argument), else CODA_ERR_WORKSPACE. Same outputs up to
 * the fp32 order of the depth sum; a negative workspace_bytes is CODA_ERR_ARG. */
int coda_gemm_rope_ws(const uint16_t* x, const uint16_t* w, const float* cos_t,
                      const float* sin_t, int M, int K, int n_q, int n_k, int n_v,
                      int head_dim, int seq_len, int pos_offset, uint16_t* out,
                      void* workspace, long long workspace_bytes, void* stream);

/* coda_gemm_rope under the persistent schedule ([notes] main experiment table, "主实验":
 * GEMM + RoPE measured at M = N = K = 4096 and 8192 with a 3N QKV width; a schedule
 * variant of the same computation): min(tiles, CUs) workgroups walk the output
 * tiles, and the last depth steps of a tile load the first two of the next, so their
 * latency hides under the epilogue and no workgroup launch separates tiles. Same
 * arguments, rules, errors and bit-identical output as coda_gemm_rope (K < 128 runs the
 * one-workgroup-per-tile kernel). CODA_ERR_HIP also if the CU count cannot be read. */
int coda_gemm_rope_persistent(const uint16_t* x, const uint16_t* w, const float* cos_t,
                              const float* sin_t, int M, int K, int n_q, int n_k, int n_v,
                              int head_dim, int seq_len, int pos_offset, uint16_t* out,
                              void* stream);

/* GEMM + SwiGLU ([notes] key design 2; [pith] Fig. 7): h = x W with x [M,K] bf16 and
 * w [K, 2F] bf16 whose columns interleave gate and up (even column 2j = G_j, odd
 * column 2j+1 = U_j); out [M,F] bf16 = silu(G) * U with silu(g) = g / (1 + exp(-g)).
 * The halving and compaction happen in the epilogue. F % 8 == 0 (and F >= 8). */
int coda_gemm_swiglu(const uint16_t* x, const uint16_t* w, int M, int K, int F,
                     uint16_t* out, void* stream);

/* coda_gemm_swiglu with the split-depth schedule (as coda_gemm_rope_ws); the GEMM's
 * output width is 2F: workspace of coda_split_workspace_bytes(M, 2 F, K) bytes. */
int coda_gemm_swiglu_ws(const uint16_t* x, const uint16_t* w, int M, int K, int F,
                        uint16_t* out, void* workspace, long long workspace_bytes,
                        void* stream);

/* Bytes of split-depth workspace one GEMM with output [M, N] (N the GEMM's full output
 * width) and depth K needs on the current device: 256 KiB per slice of every split
 * tile (every tile of an output of at most half as many tiles as CUs, or the tiles of
 * an at most half-full last wave of a larger one), 0 when it does not split. Shape
 * rules as the GEMMs; CODA_ERR_HIP if the device cannot be queried. */
int coda_split_workspace_bytes(int M, int N, int K, long long* bytes);
/* The split-depth plan of one GEMM (output [M, N], depth K) on a device of `cus` compute
 * units, computed on the host alone (no device is queried): *slices per split tile (1:
 * the one-kernel schedule for every tile), *steps of 32 depth per slice (the last may be
 * shorter), *first_split_tile (tiles before it in the tile order run the one-kernel
 * schedule) and the workspace *bytes, as the _ws entry points plan it on such a device.
 * CODA_ERR_NULL, CODA_ERR_SHAPE as the GEMMs, CODA_ERR_ARG if cus < 1. */
int coda_split_plan(int M, int N, int K, int cus, int* slices, int* steps, int* first_split_tile,
                    long long* bytes);

/* RoPE backward ([notes] key design 2; [pith] Fig. 7; the rotation is orthogonal, so its
 * gradient is the rotation by the negated angle): same arguments, layouts and rules as
 * coda_gemm_rope, with every Q and K pair of out = x W rotated by -pos * theta_p. It is
 * the epilogue of the GEMM that produces the gradient of the rotated Q and K. */
int coda_gemm_rope_bwd(const uint16_t* x, const uint16_t* w, const float* cos_t,
                       const float* sin_t, int M, int K, int n_q, int n_k, int n_v,
                       int head_dim, int seq_len, int pos_offset, uint16_t* out,
                       void* stream);
/* coda_gemm_rope_bwd with the split-depth schedule of coda_gemm_rope_ws (same workspace:
 * coda_split_workspace_bytes(M, n_q + n_k + n_v, K) bytes, same rules and errors). */
int coda_gemm_rope_bwd_ws(const uint16_t* x, const uint16_t* w, const float* cos_t,
                          const float* sin_t, int M, int K, int n_q, int n_k, int n_v,
                          int head_dim, int seq_len, int pos_offset, uint16_t* out,
                          void* workspace, long long workspace_bytes, void* stream);

/* SwiGLU backward pairwise map ([notes] key design 2, last item; [pith] Fig. 7: one
 * incoming gradient becomes the gradients of both paired inputs), in the epilogue of the
 * down projection's grad GEMM:
 *   dOut = dy W_down^T          (dy [M,Dm] bf16, w_down [F,Dm] bf16: the forward's
 *                                down-projection weight, read as W_down^T; not stored)
 *   dh[m, 2j]   = dOut U silu'(G),  dh[m, 2j+1] = dOut silu(G)
 * with G = h[m, 2j], U = h[m, 2j+1] the saved interleaved pre-activations h [M,2F] bf16
 * and silu'(g) = s (1 + g (1 - s)), s = 1/(1 + exp(-g)). dh [M,2F] bf16 output.
 * Rules: Dm % 8 == 0 (>= 8), F % 8 == 0 (>= 8); 16-byte aligned pointers. One launch;
 * M == 0 is a no-op. */
int coda_gemm_swiglu_bwd(const uint16_t* dy, const uint16_t* w_down, const uint16_t* h,
                         int M, int Dm, int F, uint16_t* dh, void* stream);
/* coda_gemm_swiglu_bwd with the split-depth schedule (as coda_gemm_rope_ws); the grad
 * GEMM's output width is F and its depth Dm: workspace of coda_split_workspace_bytes(M, F,
 * Dm) bytes. */
int coda_gemm_swiglu_bwd_ws(const uint16_t* dy, const uint16_t* w_down, const uint16_t* h,
                            int M, int Dm, int F, uint16_t* dh, void* workspace,
                            long long workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * RMSNorm-backward row statistic from the grad GEMM's epilogue ([notes] key design 3):
 *   dh2 = dy W1^T                              (dy [M,N] bf16, w1 [D,N] bf16 -> dh2 [M,D])
 *   P[m, t] = sum over the tile's columns of dh2 * h2, from the fp32 accumulator and
 *             the bf16 h2 [M,D]
 *   s[m] = (1/D) sum_t P[m, t]                 (auxiliary reduction, fixed order)
 * which equals (1/D) sum_j dy[m, j] (h2 W1)[m, j] by the identity of key design 3.
 * partials [M, nb] fp32 workspace/output (nb = coda_rowstat_num_partials(D));
 * s [M] fp32 output. Two launches on `stream`.
 * ------------------------------------------------------------------------------- */
int coda_gemm_rmsnorm_bwd_stats(const uint16_t* dy, const uint16_t* w1, const uint16_t* h2,
                                int M, int D, int N, uint16_t* dh2, float* partials,
                                float* s, void* stream);
/* coda_gemm_rmsnorm_bwd_stats with the split-depth schedule (as coda_gemm_rope_ws):
 * output width D, depth N, workspace of coda_split_workspace_bytes(M, D, N) bytes. */
int coda_gemm_rmsnorm_bwd_stats_ws(const uint16_t* dy, const uint16_t* w1, const uint16_t* h2,
                                   int M, int D, int N, uint16_t* dh2, float* partials,
                                   float* s, void* workspace, long long workspace_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------------------
 * The rest of the RMSNorm backward ([notes] key design 3 and the duality paragraph
 * before its statistic; [pith] Fig. 9). Forward (key design 1, non-deferred form):
 * r = 1/sqrt(mean(h1^2) + eps), o = r h1 * gamma (the GEMM2 input), y = o W1.
 * Backward with upstream gradient dy [M,N]:
 *   dO     = dy W1^T                      (grad GEMM, never written to HBM here)
 *   s      = (1/D) sum_cols(dO * o) = (1/D) sum_j dy[m, j] y[m, j]   (key design 3:
 *            the statistic is available before the grad GEMM, from the output side)
 *   dh1    = r gamma dO - r^2 s h1 (+ g_res, the gradient reaching h1 through the
 *            residual stream)           -> stored bf16 in the grad GEMM's epilogue
 *   dgamma = sum_rows(dO r h1)          -> fp32 column partials per 256-row tile in the
 *            epilogue, then a column reduction in the fixed order of the tiles.
 * Layouts: dy [M,N] bf16; w1 [D,N] bf16 (the forward GEMM2 weight, read as W1^T);
 * h1, g_res, dh1 [M,D] bf16; gamma [D] bf16; r, s [M] fp32; y [M,N] bf16 (the forward
 * output); dgamma_partials [T, D] fp32 with T = coda_colstat_num_partials(M) (row tile
 * t covers rows [256 t, 256 t + 256)); dgamma [D] fp32. Rules as for the other GEMMs:
 * D % 8 == 0 and N % 8 == 0 (both >= 8); bf16 pointers 16-byte aligned, fp32 pointers
 * 4-byte aligned; outputs must not overlap inputs or each other.
 * ------------------------------------------------------------------------------- */
/* T = ceil(rows / 256): row tiles of the dgamma column-partial workspace. Returns
 * CODA_ERR_NULL or CODA_ERR_SHAPE (rows < 0). */
int coda_colstat_num_partials(int rows, int* tiles);

/* s[m] = (1/d) sum_j dy[m, j] y[m, j] for dy, y [M,N] bf16 (one wave per row, lane
 * partial sums then a fixed butterfly: deterministic). d >= 1. M == 0 is a no-op. */
int coda_rowdot_stat(const uint16_t* dy, const uint16_t* y, int M, int N, int d, float* s,
                     void* stream);

/* out[n] = sum_t partials[t, n], t = 0 .. tiles-1 in order, for partials [tiles, width]
 * fp32; tiles == 0 writes zeros (partials may then be NULL). */
int coda_colsum_reduce(const float* partials, int tiles, int width, float* out, void* stream);

/* The grad GEMM dy W1^T with the RMSNorm-backward epilogue: dh1 and dgamma_partials as
 * above, from the caller's r and s (e.g. s from coda_rowdot_stat, or from the epilogue
 * of the GEMM that produced dy). g_res may be NULL (no residual-stream gradient).
 * One launch; M == 0 is a no-op. */
int coda_gemm_rmsnorm_bwd_dx(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1,
                             const uint16_t* gamma, const float* r, const float* s,
                             const uint16_t* g_res, int M, int D, int N, uint16_t* dh1,
                             float* dgamma_partials, void* stream);
/* coda_gemm_rmsnorm_bwd_dx with the split-depth schedule (as coda_gemm_rope_ws): output
 * width D, depth N, workspace of coda_split_workspace_bytes(M, D, N) bytes. The dgamma
 * partials come from the summed accumulators, so their values match the one-kernel call
 * up to the fp32 order of the depth sum. */
int coda_gemm_rmsnorm_bwd_dx_ws(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1,
                                const uint16_t* gamma, const float* r, const float* s,
                                const uint16_t* g_res, int M, int D, int N, uint16_t* dh1,
                                float* dgamma_partials, void* workspace,
                                long long workspace_bytes, void* stream);

/* All of it: s from (dy, y), the grad GEMM with its epilogue, and dgamma. Three
 * launches on `stream`. s [M], dh1, dgamma_partials and dgamma are outputs. With M == 0
 * only dgamma is written (zeros: a sum over no rows), so dgamma is always required. */
int coda_rmsnorm_bwd(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1,
                     const uint16_t* gamma, const float* r, const uint16_t* y,
                     const uint16_t* g_res, int M, int D, int N, float* s, uint16_t* dh1,
                     float* dgamma_partials, float* dgamma, void* stream);

/* ---------------------------------------------------------------------------------
 * GEMM + cross-entropy ([notes] method overview: the cross-entropy log-sum-exp is a
 * cross-tile statistic emitted as tile partials and merged by an auxiliary kernel; the
 * five epilogue primitives, (5) stateful transforms such as an online log-sum-exp):
 *   z = x W                         (x [M,K] bf16, w [K,V] bf16; z is never stored)
 *   tile_lse[m, t] = log sum over the columns of 256-column tile t of exp(z[m, .])
 *   target[m] = z[m, labels[m]]     (fp32, from the accumulator)
 *   lse[m] = log sum_t exp(tile_lse[m, t])   (auxiliary merge, order t = 0, 1, ...)
 *   loss[m] = lse[m] - target[m]
 * labels [M] int32; a label outside [0, V) marks an ignored row: loss = target = 0 there.
 * tile_lse [M, nb] fp32 workspace/output with nb = coda_rowstat_num_partials(V); target,
 * lse, loss [M] fp32 outputs. Rules: K % 8 == 0, V % 8 == 0 (both >= 8); x, w 16-byte
 * aligned, the rest 4-byte aligned. Two launches on `stream`; M == 0 is a no-op.
 * ------------------------------------------------------------------------------- */
int coda_gemm_cross_entropy(const uint16_t* x, const uint16_t* w, const int32_t* labels,
                            int M, int K, int V, float* tile_lse, float* target, float* lse,
                            float* loss, void* stream);
/* coda_gemm_cross_entropy with the split-depth schedule (as coda_gemm_rope_ws): output
 * width V, depth K, workspace of coda_split_workspace_bytes(M, V, K) bytes. */
int coda_gemm_cross_entropy_ws(const uint16_t* x, const uint16_t* w, const int32_t* labels,
                               int M, int K, int V, float* tile_lse, float* target,
                               float* lse, float* loss, void* workspace,
                               long long workspace_bytes, void* stream);
/* The auxiliary merge alone (tile_lse and target from the epilogue above). nb must equal
 * coda_rowstat_num_partials(V). */
int coda_lse_reduce(const float* tile_lse, const int32_t* labels, int M, int nb, int V,
                    float* target, float* lse, float* loss, void* stream);

/* ---------------------------------------------------------------------------------
 * Unfused baselines, for measurement and numerics comparison only (not the fused
 * path): the same MFMA main loop with a plain store, and separate HBM-bound kernels
 * for what the fused epilogues do (the standard operator-by-operator path).
 * ------------------------------------------------------------------------------- */
/* c [M,N] bf16 = a [M,K] b, with b [K,N] if b_kn != 0 else b [N,K] (c = a b^T). */
int coda_baseline_gemm(const uint16_t* a, const uint16_t* b, int M, int K, int N, int b_kn,
                       uint16_t* c, void* stream);
/* h1 = h0 + z; r = 1/sqrt(mean(h1^2) + eps); o = r h1 * gamma. h0, z, h1, o [M,D] bf16
 * (h1 rounded before the norm reads it back, as a separate operator would). */
int coda_baseline_residual_rmsnorm(const uint16_t* h0, const uint16_t* z,
                                   const uint16_t* gamma, int M, int D, float eps,
                                   uint16_t* h1, float* r, uint16_t* o, void* stream);
/* out = RoPE(h) on the Q and K blocks of h [M, n_q+n_k+n_v] (V copied). */
int coda_baseline_rope(const uint16_t* h, const float* cos_t, const float* sin_t, int M,
                       int n_q, int n_k, int n_v, int head_dim, int seq_len, int pos_offset,
                       uint16_t* out, void* stream);
/* out [M,F] = silu(h[:, 0::2]) * h[:, 1::2] for h [M,2F]. */
int coda_baseline_swiglu(const uint16_t* h, int M, int F, uint16_t* out, void* stream);
/* s[m] = (1/D) sum_k a[m,k] b[m,k] for a, b [M,D] bf16. */
int coda_baseline_rowdot(const uint16_t* a, const uint16_t* b, int M, int D, float* s,
                         void* stream);
/* dst = src, `bytes` a positive multiple of 16: a plain copy kernel of known traffic. */
int coda_baseline_copy(const void* src, void* dst, int64_t bytes, void* stream);
/* Measurement probe (no step of the method): `grid` workgroups of 512 threads; thread g
 * reads fragments 16 g .. 16 g + 15 (mod n_frag) of operands [n_frag, 8] bf16 once, then
 * each wave runs `iters` rounds of 32 v_mfma_f32_16x16x32_bf16 (the GEMM's MFMA form and
 * per-wave shape) on registers only; out [grid * 512] fp32 receives each thread's
 * accumulator sum. FLOPs = grid * 8 * iters * 32 * 16384. With operands drawn like the workloads' data it gives
 * the MFMA rate sustained under the chip's power limit (the practical ceiling beside the
 * nominal peak). Rules: n_frag, iters >= 1; 1 <= grid <= 65535; operands 16-byte aligned. */
int coda_baseline_mfma_loop(const uint16_t* operands, int n_frag, int iters, int grid,
                            float* out, void* stream);
/* Measurement probe (no step of the method): the GEMM main loop's per-step LDS operand
 * reads and MFMAs, in its order and with its priorities, on an LDS image written once
 * (seed 0: every bf16 element = bf16(fill); otherwise bits hashed from (seed, position):
 * values +-[1/4, 1/2) with random signs and mantissas, as the MFMA's rate depends on
 * the operand bits); no DMA and nothing rewritten. `grid` workgroups of
 * 512 threads run `steps` 32-deep steps each. kind 0: KN-W reads (two transposed 8-byte
 * reads per W block), one workgroup barrier per step as in the GEMM; 1: the same without
 * the barrier; 2: NK-W reads (one 16-byte read per W block) with the barrier; 3: the
 * reads of kind 0 alone, no MFMAs; 4: the MFMAs of kind 0 alone, on operands read once
 * before the loop, no barrier; 5: kind 0 with only the W reads (X operands read once
 * before the loop); 6: kind 0 with only the X reads (W operands read once before the
 * loop); 7: kind 0 plus the GEMM's DMA issue (4 loads of 1 KiB per wave and step into
 * the ring) through a descriptor of no bytes, so every load zero-fills LDS without a
 * memory access; only with fill == 0 and seed == 0 (else CODA_ERR_ARG), whose image the
 * fills leave unchanged. out [grid * 512] fp32: kinds 0-2 and 4-7 each thread's
 * accumulator sum (seed 0: = 128 * 32 * fill^2 * steps up to rounding; every workgroup
 * computes the same values); kind 3 the bit pattern of
 * the 32-bit wrapping sum of every word the thread read (48 words per step). cycles
 * [grid * 8] int64: each wave's core-clock cycles over the steps (s_memtime). Rules:
 * 0 <= kind <= 7, steps >= 1, 1 <= grid <= 65535; out 4-, cycles 8-byte aligned. */
int coda_baseline_schedule_probe(int kind, int steps, int grid, float fill, uint32_t seed,
                                 float* out, long long* cycles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H */
