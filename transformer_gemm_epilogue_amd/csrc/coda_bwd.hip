// C-ABI entry points of the backward epilogue programs (declared in coda.h): the rest of
// the RMSNorm backward (the row statistic from the output side, the grad GEMM with the
// RMSNorm-backward epilogue, the column reduction of the gamma-gradient partials) and
// the SwiGLU backward pairwise map on the down projection's grad GEMM.
#include "coda_abi.hpp"
#include "coda_bwd.hpp"
#include "coda_launch.hpp"

using namespace coda;

namespace {

// s[m] = (1/d) sum_j dy[m, j] * y[m, j]: one wave per row, 16-byte loads of both rows,
// each lane summing its chunks (columns 8 (lane + 64 i) ..) in order, then a fixed
// butterfly over the 64 lanes. A streaming kernel: 4 N bytes read per row.
constexpr int kRdWaves = 4;

__global__ __launch_bounds__(64 * kRdWaves) void rowdot_stat_kernel(const uint16_t* __restrict__ dy,
                                                                    const uint16_t* __restrict__ y, int M, int N,
                                                                    float d, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRdWaves + (threadIdx.x >> 6);
  if (m >= M) return;  // wave-uniform
  const uint16_t* a = dy + (size_t)m * N;
  const uint16_t* b = y + (size_t)m * N;
  float acc = 0.f;
#pragma unroll 4
  for (int c = lane * 8; c < N; c += 64 * 8) {  // N % 8 == 0
    const u32x4_t va = *(const u32x4_t*)(a + c);
    const u32x4_t vb = *(const u32x4_t*)(b + c);
    float t = bf16_lo(va.x) * bf16_lo(vb.x) + bf16_hi(va.x) * bf16_hi(vb.x);
    t += bf16_lo(va.y) * bf16_lo(vb.y) + bf16_hi(va.y) * bf16_hi(vb.y);
    t += bf16_lo(va.z) * bf16_lo(vb.z) + bf16_hi(va.z) * bf16_hi(vb.z);
    t += bf16_lo(va.w) * bf16_lo(vb.w) + bf16_hi(va.w) * bf16_hi(vb.w);
    acc += t;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) s[m] = acc / d;
}

// out[n] = sum_t P[t, n] in the order t = 0, 1, ..., tiles-1 (one thread per column).
// The loads go out 16 at a time and are then added in order: a few memory round trips per
// column instead of one per tile (the width, not the tile count, sets the parallelism).
__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float* __restrict__ P, int tiles, int width,
                                                            float* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= width) return;
  float acc = 0.f;
  int t = 0;
  for (; t + 16 <= tiles; t += 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = P[(size_t)(t + k) * width + n];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc += v[k];
  }
  for (; t < tiles; ++t) acc += P[(size_t)t * width + n];
  out[n] = acc;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0.f;
}

inline unsigned blocks(long long n, int per) { return (unsigned)((n + per - 1) / per); }
inline int row_tiles(int M) { return (M + kBM - 1) / kBM; }

int check_rowdot(const uint16_t* dy, const uint16_t* y, int M, int N, int d, float* s) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(N));
  if (d < 1) return CODA_ERR_SHAPE;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(dy);
  CODA_NONNULL(y);
  CODA_NONNULL(s);
  CODA_ALIGN16(dy);
  CODA_ALIGN16(y);
  if (!aligned(s, 4)) return CODA_ERR_ALIGN;
  return CODA_OK;
}

int check_dx(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1, const uint16_t* gamma, const float* r,
             const float* s, const uint16_t* g_res, int M, int D, int N, uint16_t* dh1, float* pgamma) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(D));
  CODA_TRY(check_depth_or_width(N));
  if (M == 0) return CODA_OK;
  CODA_NONNULL(dy);
  CODA_NONNULL(w1);
  CODA_NONNULL(h1);
  CODA_NONNULL(gamma);
  CODA_NONNULL(r);
  CODA_NONNULL(s);
  CODA_NONNULL(dh1);
  CODA_NONNULL(pgamma);
  CODA_ALIGN16(dy);
  CODA_ALIGN16(w1);
  CODA_ALIGN16(h1);
  CODA_ALIGN16(gamma);
  CODA_ALIGN16(dh1);
  if (g_res) CODA_ALIGN16(g_res);
  if (!aligned(r, 4) || !aligned(s, 4) || !aligned(pgamma, 4)) return CODA_ERR_ALIGN;
  return CODA_OK;
}

int launch_rowdot(const uint16_t* dy, const uint16_t* y, int M, int N, int d, float* s, hipStream_t st) {
  hipLaunchKernelGGL(rowdot_stat_kernel, dim3(blocks(M, kRdWaves)), dim3(64 * kRdWaves), 0, st, dy, y, M, N,
                     (float)d, s);
  return launch_status();
}

// sp: the split-depth plan (S == 1: the one-kernel schedule) and ws its workspace.
int launch_dx(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1, const uint16_t* gamma, const float* r,
              const float* s, const uint16_t* g_res, int M, int D, int N, uint16_t* dh1, float* pgamma,
              hipStream_t st, const SplitPlan& sp = SplitPlan{1, 0}, float* ws = nullptr) {
  // dy [M, N] times W1^T: depth = N, output width = D; W1 [D, N] is the NK layout.
  const GemmProblem p{dy, w1, M, D, N};
  const EpiRmsNormBwd::Args ea{h1, gamma, r, s, g_res, dh1, pgamma};
  return launch_gemm_split<false, EpiRmsNormBwd>(p, ea, sp, ws, st);
}

int launch_colsum(const float* P, int tiles, int width, float* out, hipStream_t st) {
  if (tiles == 0)
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks(width, 256)), dim3(256), 0, st, out, width);
  else
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3(blocks(width, 256)), dim3(256), 0, st, P, tiles, width, out);
  return launch_status();
}

int gemm_swiglu_bwd(const uint16_t* dy, const uint16_t* w_down, const uint16_t* h, int M, int Dm, int F, uint16_t* dh,
                    bool split, void* workspace, long long workspace_bytes, hipStream_t st) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(Dm));
  if (F < 8 || F % 8 != 0 || 2LL * F > kMaxDim) return CODA_ERR_SHAPE;
  if (split && workspace_bytes < 0) return CODA_ERR_ARG;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(dy);
  CODA_NONNULL(w_down);
  CODA_NONNULL(h);
  CODA_NONNULL(dh);
  CODA_ALIGN16(dy);
  CODA_ALIGN16(w_down);
  CODA_ALIGN16(h);
  CODA_ALIGN16(dh);
  CODA_TRY(check_disjoint({bf16_span(dh, M, 2LL * F)},
                          {bf16_span(dy, M, Dm), bf16_span(w_down, F, Dm), bf16_span(h, M, 2LL * F)}));
  // dy [M, Dm] times W_down^T: depth = Dm, output width = F; W_down [F, Dm] is the NK layout.
  const GemmProblem p{dy, w_down, M, F, Dm};
  const EpiSwiGLUBwd::Args ea{h, dh};
  SplitPlan sp{1, 0};
  if (split)
    CODA_TRY(split_for_call(M, F, Dm, workspace, workspace_bytes,
                            {bf16_span(dh, M, 2LL * F), bf16_span(dy, M, Dm), bf16_span(w_down, F, Dm),
                             bf16_span(h, M, 2LL * F)},
                            &sp));
  return launch_gemm_split<false, EpiSwiGLUBwd>(p, ea, sp, static_cast<float*>(workspace), st);
}

}  // namespace

extern "C" {

int coda_colstat_num_partials(int rows, int* tiles) {
  CODA_NONNULL(tiles);
  CODA_TRY(check_rows(rows));
  *tiles = row_tiles(rows);
  return CODA_OK;
}

int coda_rowdot_stat(const uint16_t* dy, const uint16_t* y, int M, int N, int d, float* s, void* stream) {
  CODA_TRY(check_rowdot(dy, y, M, N, d, s));
  if (M == 0) return CODA_OK;
  CODA_TRY(check_disjoint({f32_span(s, M)}, {bf16_span(dy, M, N), bf16_span(y, M, N)}));
  return launch_rowdot(dy, y, M, N, d, s, as_stream(stream));
}

int coda_colsum_reduce(const float* partials, int tiles, int width, float* out, void* stream) {
  if (tiles < 0 || width < 1 || width > kMaxDim) return CODA_ERR_SHAPE;
  CODA_NONNULL(out);
  if (tiles > 0) CODA_NONNULL(partials);
  if ((partials && !aligned(partials, 4)) || !aligned(out, 4)) return CODA_ERR_ALIGN;
  CODA_TRY(check_disjoint({f32_span(out, width)}, {f32_span(partials, tiles, width)}));
  return launch_colsum(partials, tiles, width, out, as_stream(stream));
}

int coda_gemm_rmsnorm_bwd_dx(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1, const uint16_t* gamma,
                             const float* r, const float* s, const uint16_t* g_res, int M, int D, int N,
                             uint16_t* dh1, float* dgamma_partials, void* stream) {
  CODA_TRY(check_dx(dy, w1, h1, gamma, r, s, g_res, M, D, N, dh1, dgamma_partials));
  if (M == 0) return CODA_OK;
  CODA_TRY(check_disjoint({bf16_span(dh1, M, D), f32_span(dgamma_partials, row_tiles(M), D)},
                          {bf16_span(dy, M, N), bf16_span(w1, D, N), bf16_span(h1, M, D), bf16_span(gamma, D),
                           f32_span(r, M), f32_span(s, M), bf16_span(g_res, M, D)}));
  return launch_dx(dy, w1, h1, gamma, r, s, g_res, M, D, N, dh1, dgamma_partials, as_stream(stream));
}

int coda_gemm_rmsnorm_bwd_dx_ws(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1, const uint16_t* gamma,
                                const float* r, const float* s, const uint16_t* g_res, int M, int D, int N,
                                uint16_t* dh1, float* dgamma_partials, void* workspace, long long workspace_bytes,
                                void* stream) {
  if (workspace_bytes < 0) return CODA_ERR_ARG;
  CODA_TRY(check_dx(dy, w1, h1, gamma, r, s, g_res, M, D, N, dh1, dgamma_partials));
  if (M == 0) return CODA_OK;
  CODA_TRY(check_disjoint({bf16_span(dh1, M, D), f32_span(dgamma_partials, row_tiles(M), D)},
                          {bf16_span(dy, M, N), bf16_span(w1, D, N), bf16_span(h1, M, D), bf16_span(gamma, D),
                           f32_span(r, M), f32_span(s, M), bf16_span(g_res, M, D)}));
  SplitPlan sp;
  CODA_TRY(split_for_call(M, D, N, workspace, workspace_bytes,
                          {bf16_span(dh1, M, D), f32_span(dgamma_partials, row_tiles(M), D), bf16_span(dy, M, N),
                           bf16_span(w1, D, N), bf16_span(h1, M, D), bf16_span(gamma, D), f32_span(r, M),
                           f32_span(s, M), bf16_span(g_res, M, D)},
                          &sp));
  return launch_dx(dy, w1, h1, gamma, r, s, g_res, M, D, N, dh1, dgamma_partials, as_stream(stream), sp,
                   static_cast<float*>(workspace));
}

int coda_rmsnorm_bwd(const uint16_t* dy, const uint16_t* w1, const uint16_t* h1, const uint16_t* gamma,
                     const float* r, const uint16_t* y, const uint16_t* g_res, int M, int D, int N, float* s,
                     uint16_t* dh1, float* dgamma_partials, float* dgamma, void* stream) {
  CODA_TRY(check_dx(dy, w1, h1, gamma, r, s, g_res, M, D, N, dh1, dgamma_partials));
  CODA_TRY(check_rowdot(dy, y, M, N, D, s));
  CODA_NONNULL(dgamma);
  if (!aligned(dgamma, 4)) return CODA_ERR_ALIGN;
  // s is written by the first launch and read by the second: an output here
  if (M > 0)
    CODA_TRY(check_disjoint({f32_span(s, M), bf16_span(dh1, M, D), f32_span(dgamma_partials, row_tiles(M), D),
                             f32_span(dgamma, D)},
                            {bf16_span(dy, M, N), bf16_span(w1, D, N), bf16_span(h1, M, D), bf16_span(gamma, D),
                             f32_span(r, M), bf16_span(y, M, N), bf16_span(g_res, M, D)}));
  const hipStream_t st = as_stream(stream);
  if (M > 0) {
    CODA_TRY(launch_rowdot(dy, y, M, N, D, s, st));
    CODA_TRY(launch_dx(dy, w1, h1, gamma, r, s, g_res, M, D, N, dh1, dgamma_partials, st));
  }
  return launch_colsum(dgamma_partials, row_tiles(M), D, dgamma, st);
}

int coda_gemm_swiglu_bwd(const uint16_t* dy, const uint16_t* w_down, const uint16_t* h, int M, int Dm, int F,
                         uint16_t* dh, void* stream) {
  return gemm_swiglu_bwd(dy, w_down, h, M, Dm, F, dh, false, nullptr, 0, as_stream(stream));
}

int coda_gemm_swiglu_bwd_ws(const uint16_t* dy, const uint16_t* w_down, const uint16_t* h, int M, int Dm, int F,
                            uint16_t* dh, void* workspace, long long workspace_bytes, void* stream) {
  return gemm_swiglu_bwd(dy, w_down, h, M, Dm, F, dh, true, workspace, workspace_bytes, as_stream(stream));
}

}  // extern "C"
