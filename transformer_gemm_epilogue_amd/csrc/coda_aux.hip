// Auxiliary kernels: the row reduction over tile partials, the RoPE table builder, the
// unfused baseline operators (kept for measurement and the numerics comparison), and two
// measurement probes (a register-only MFMA loop and the GEMM main loop's reads and MFMAs
// on a fixed LDS image).
#include <algorithm>

#include "coda_abi.hpp"
#include "coda_common.hpp"
#include "coda_gemm.hpp"

using namespace coda;

namespace {

// Auxiliary row reduction of the per-tile partials: one thread per row sums its row in
// the fixed order t = 0, 1, ..., nb-1 (deterministic, independent of the launch) and
// applies the row statistic. Loads go out four 16-byte vectors at a time per thread, so
// a wave has 4 KiB of HBM reads in flight with no LDS or barrier; this is a pure
// streaming kernel (nb * 4 bytes read and 4 written per row).
constexpr int kRsThreads = 256;

template <bool kVec4>
__global__ __launch_bounds__(kRsThreads) void rowstat_reduce_kernel(const float* __restrict__ P, int M, int nb,
                                                                    float d, float eps, int mode,
                                                                    float* __restrict__ out) {
  const int m = blockIdx.x * kRsThreads + threadIdx.x;
  if (m >= M) return;
  const float* row = P + (size_t)m * nb;
  float s = 0.f;
  if constexpr (kVec4) {
    for (int c0 = 0; c0 < nb; c0 += 16) {  // nb % 4 == 0
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c0 + 4 * q < nb) v[q] = *(const float4*)(row + c0 + 4 * q);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c0 + 4 * q < nb) s = (((s + v[q].x) + v[q].y) + v[q].z) + v[q].w;
    }
  } else {
    for (int c = 0; c < nb; ++c) s += row[c];
  }
  const float mean = s / d;
  out[m] = (mode == CODA_ROWSTAT_RSQRT_MEAN_EPS) ? 1.0f / sqrtf(mean + eps) : mean;
}

// The same reduction with contiguous loads, for nb = 4 L with L = 1, 2, 4, 8 or 16 lanes
// per row: each 16-byte load of a wave reads 1 KiB of consecutive partials, so lane i of
// load q holds floats 4c .. 4c + 3 (c = i mod L) of row 64 q / L + i / L. The running sum
// then passes from lane to lane (a DPP shift by one within each 16-lane row) in chunk
// order, so every row is still summed in the order t = 0, 1, ..., nb-1 (the same fp32
// additions as the thread-per-row form, bit for bit). Reading whole lines per load
// instead of a quarter of 32 lines measured 5.9 against 5.3 TB/s on a 1 GiB buffer.
// The partials are read once, so the loads are non-temporal (streaming), two per lane:
// 6.4 TB/s on 1 GiB, a plain read's rate, against 5.8 with four cached loads.
constexpr int kChainLoads = 2;
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
template <int L>
__global__ __launch_bounds__(kRsThreads) void rowstat_chain_kernel(const float* __restrict__ P, int M, float d,
                                                                   float eps, int mode, float* __restrict__ out) {
  constexpr int kRowsPerLoad = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row0 = ((long long)blockIdx.x * (kRsThreads / 64) + wave) * (kChainLoads * kRowsPerLoad);
  const f32x4v_t* P4 = (const f32x4v_t*)P;
  const long long n4 = (long long)M * L;
  f32x4v_t v[kChainLoads];
#pragma unroll
  for (int q = 0; q < kChainLoads; ++q) {
    const long long i = row0 * L + q * 64 + lane;
    v[q] = i < n4 ? __builtin_nontemporal_load(P4 + i) : f32x4v_t{0.f, 0.f, 0.f, 0.f};
  }
  const int c = lane % L;
#pragma unroll
  for (int q = 0; q < kChainLoads; ++q) {
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const float in =
          __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, run), 0x111, 0xF, 0xF, false));
      const float start = k == 0 ? 0.f : in;  // row_shr:1: lane i receives lane i - 1
      if (c == k) run = (((start + v[q].x) + v[q].y) + v[q].z) + v[q].w;
    }
    const long long m = row0 + q * kRowsPerLoad + lane / L;
    if (c == L - 1 && m < M) {
      const float mean = run / d;
      out[m] = (mode == CODA_ROWSTAT_RSQRT_MEAN_EPS) ? 1.0f / sqrtf(mean + eps) : mean;
    }
  }
}

// ------------------------------------------------------------------------ RoPE tables
__global__ void rope_tables_kernel(float* __restrict__ cos_t, float* __restrict__ sin_t, int seq_len, int half,
                                   int head_dim, double theta) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)seq_len * half) return;
  const int pos = (int)(i / half);
  const int p = (int)(i - (long long)pos * half);
  const double inv_freq = pow(theta, -2.0 * (double)p / (double)head_dim);
  const double a = (double)pos * inv_freq;
  cos_t[i] = (float)cos(a);
  sin_t[i] = (float)sin(a);
}

// ---------------------------------------------------------------- unfused baselines
__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// One row per 256-thread block: h1 = bf16(h0 + z); r from the stored bf16 h1 (as a
// separate RMSNorm operator reads it); o = bf16(r h1 gamma).
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(const uint16_t* __restrict__ h0,
                                                                const uint16_t* __restrict__ z,
                                                                const uint16_t* __restrict__ gamma, int D, float eps,
                                                                uint16_t* __restrict__ h1, float* __restrict__ r,
                                                                uint16_t* __restrict__ o) {
  __shared__ float red[4];
  const size_t base = (size_t)blockIdx.x * D;
  float ss = 0.f;
  for (int c = threadIdx.x * 8; c < D; c += 256 * 8) {
    const u32x4_t a = *(const u32x4_t*)(h0 + base + c);
    const u32x4_t b = *(const u32x4_t*)(z + base + c);
    u32x4_t h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = pack_bf16x2(bf16_lo(a[q]) + bf16_lo(b[q]), bf16_hi(a[q]) + bf16_hi(b[q]));
      h[q] = w;
      ss += bf16_lo(w) * bf16_lo(w) + bf16_hi(w) * bf16_hi(w);
    }
    *(u32x4_t*)(h1 + base + c) = h;
  }
  const float tot = block_sum_256(ss, red);
  const float rr = 1.0f / sqrtf(tot / (float)D + eps);
  if (threadIdx.x == 0) r[blockIdx.x] = rr;
  for (int c = threadIdx.x * 8; c < D; c += 256 * 8) {
    const u32x4_t h = *(const u32x4_t*)(h1 + base + c);
    const u32x4_t g = *(const u32x4_t*)(gamma + c);
    u32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = pack_bf16x2(rr * bf16_lo(h[q]) * bf16_lo(g[q]), rr * bf16_hi(h[q]) * bf16_hi(g[q]));
    *(u32x4_t*)(o + base + c) = v;
  }
}

__global__ __launch_bounds__(256) void rowdot_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                      int D, float* __restrict__ s) {
  __shared__ float red[4];
  const size_t base = (size_t)blockIdx.x * D;
  float acc = 0.f;
  for (int c = threadIdx.x * 8; c < D; c += 256 * 8) {
    const u32x4_t x = *(const u32x4_t*)(a + base + c);
    const u32x4_t y = *(const u32x4_t*)(b + base + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc += bf16_lo(x[q]) * bf16_lo(y[q]) + bf16_hi(x[q]) * bf16_hi(y[q]);
  }
  const float tot = block_sum_256(acc, red);
  if (threadIdx.x == 0) s[blockIdx.x] = tot / (float)D;
}

// 8 consecutive columns (4 rotation pairs) per thread.
__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* __restrict__ h, const float* __restrict__ cos_t,
                                                    const float* __restrict__ sin_t, int M, int N, int n_rot,
                                                    int head_dim, int seq_len, int pos_offset,
                                                    uint16_t* __restrict__ out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = N / 8;
  if (i >= (long long)M * per_row) return;
  const int m = (int)(i / per_row);
  const int n = (int)(i - (long long)m * per_row) * 8;
  const size_t off = (size_t)m * N + n;
  u32x4_t v = *(const u32x4_t*)(h + off);
  if (n < n_rot) {
    const int pos = (int)(((long long)m + pos_offset) % seq_len);
    const int half = head_dim >> 1;
    const int p0 = (n % head_dim) >> 1;
    const float4 c = *(const float4*)(cos_t + (size_t)pos * half + p0);
    const float4 s = *(const float4*)(sin_t + (size_t)pos * half + p0);
    const float cc[4] = {c.x, c.y, c.z, c.w};
    const float sn[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float e = bf16_lo(v[q]), o = bf16_hi(v[q]);
      v[q] = pack_bf16x2(e * cc[q] - o * sn[q], e * sn[q] + o * cc[q]);
    }
  }
  *(u32x4_t*)(out + off) = v;
}

// 8 accumulator columns (4 gate/up pairs) -> 4 outputs per thread.
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ h, int M, int F,
                                                      uint16_t* __restrict__ out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = F / 4;
  if (i >= (long long)M * per_row) return;
  const int m = (int)(i / per_row);
  const int j = (int)(i - (long long)m * per_row) * 4;
  const u32x4_t v = *(const u32x4_t*)(h + (size_t)m * 2 * F + 2 * j);
  float y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float g = bf16_lo(v[q]), u = bf16_hi(v[q]);
    y[q] = g / (1.0f + __expf(-g)) * u;
  }
  u32x2_t o;
  o.x = pack_bf16x2(y[0], y[1]);
  o.y = pack_bf16x2(y[2], y[3]);
  *(u32x2_t*)(out + (size_t)m * F + j) = o;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                    long long n16) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

inline unsigned blocks_for(long long n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

// Register-only MFMA loop, a measurement probe: each thread reads 16 operand fragments
// once, then every wave runs `iters` rounds of 32 v_mfma_f32_16x16x32_bf16 on 32
// independent accumulators (the GEMM's per-wave shape: 4 feature blocks x 8 token
// blocks, 8 waves per workgroup, two per SIMD) with no memory traffic in between; the
// token blocks 0..3 and 4..7 take different operand sets. Fed with operands drawn like
// the workloads' data, it shows the MFMA rate the chip sustains under its power limit.
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void mfma_loop_kernel(const bf16x8_t* __restrict__ ops, int n_frag, int iters, float* __restrict__ out) {
  const long long gt = (long long)blockIdx.x * 512 + threadIdx.x;
  bf16x8_t a[4], c[4], b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[(gt * 16 + i) % n_frag];
    c[i] = ops[(gt * 16 + 4 + i) % n_frag];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = ops[(gt * 16 + 8 + j) % n_frag];
  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(j < 4 ? a[i] : c[i], b[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) s += acc[i][j][v];
  out[gt] = s;
}

}  // namespace

// Shared with the GEMM entry points (no argument checks: callers have checked).
int coda_rowstat_reduce_impl(const float* partials, int M, int nb, int d, float eps, int mode, float* out,
                             hipStream_t stream) {
  const unsigned grid = blocks_for(M, kRsThreads);
  if (aligned(partials, 16) && (nb == 4 || nb == 8 || nb == 16 || nb == 32 || nb == 64)) {
    const unsigned cg = (unsigned)blocks_for(M, kRsThreads * kChainLoads / (nb / 4));  // rows per block
    switch (nb) {
      case 4: hipLaunchKernelGGL((rowstat_chain_kernel<1>), dim3(cg), dim3(kRsThreads), 0, stream, partials, M, (float)d, eps, mode, out); break;
      case 8: hipLaunchKernelGGL((rowstat_chain_kernel<2>), dim3(cg), dim3(kRsThreads), 0, stream, partials, M, (float)d, eps, mode, out); break;
      case 16: hipLaunchKernelGGL((rowstat_chain_kernel<4>), dim3(cg), dim3(kRsThreads), 0, stream, partials, M, (float)d, eps, mode, out); break;
      case 32: hipLaunchKernelGGL((rowstat_chain_kernel<8>), dim3(cg), dim3(kRsThreads), 0, stream, partials, M, (float)d, eps, mode, out); break;
      default: hipLaunchKernelGGL((rowstat_chain_kernel<16>), dim3(cg), dim3(kRsThreads), 0, stream, partials, M, (float)d, eps, mode, out); break;
    }
    return launch_status();
  }
  if (nb % 4 == 0 && aligned(partials, 16))
    hipLaunchKernelGGL((rowstat_reduce_kernel<true>), dim3(grid), dim3(kRsThreads), 0, stream, partials, M, nb,
                       (float)d, eps, mode, out);
  else
    hipLaunchKernelGGL((rowstat_reduce_kernel<false>), dim3(grid), dim3(kRsThreads), 0, stream, partials, M, nb,
                       (float)d, eps, mode, out);
  return launch_status();
}

extern "C" {

int coda_rowstat_reduce(const float* partials, int M, int nb, int d, float eps, int mode, float* out,
                        void* stream) {
  CODA_TRY(check_rows(M));
  if (nb < 1 || nb > kMaxDim || d < 1) return CODA_ERR_SHAPE;
  if (mode != CODA_ROWSTAT_RSQRT_MEAN_EPS && mode != CODA_ROWSTAT_MEAN) return CODA_ERR_ARG;
  if (mode == CODA_ROWSTAT_RSQRT_MEAN_EPS && (!(eps >= 0.0f) || !(eps < __builtin_huge_valf()))) return CODA_ERR_ARG;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(partials);
  CODA_NONNULL(out);
  if (!aligned(partials, 4) || !aligned(out, 4)) return CODA_ERR_ALIGN;
  CODA_TRY(check_disjoint({f32_span(out, M)}, {f32_span(partials, M, nb)}));
  return coda_rowstat_reduce_impl(partials, M, nb, d, eps, mode, out, as_stream(stream));
}

int coda_rope_tables(float* cos_t, float* sin_t, int seq_len, int head_dim, double theta, void* stream) {
  CODA_NONNULL(cos_t);
  CODA_NONNULL(sin_t);
  if (seq_len < 1 || head_dim < 2 || head_dim % 2 != 0 || head_dim > kMaxDim) return CODA_ERR_SHAPE;
  if (!(theta > 0.0) || !(theta < __builtin_huge_val())) return CODA_ERR_ARG;
  if (!aligned(cos_t, 8) || !aligned(sin_t, 8)) return CODA_ERR_ALIGN;
  const long long n = (long long)seq_len * (head_dim / 2);
  CODA_TRY(check_disjoint({f32_span(cos_t, n), f32_span(sin_t, n)}, {}));
  hipLaunchKernelGGL(rope_tables_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, as_stream(stream), cos_t, sin_t,
                     seq_len, head_dim / 2, head_dim, theta);
  return launch_status();
}

int coda_baseline_residual_rmsnorm(const uint16_t* h0, const uint16_t* z, const uint16_t* gamma, int M, int D,
                                   float eps, uint16_t* h1, float* r, uint16_t* o, void* stream) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(D));
  if (M == 0) return CODA_OK;
  CODA_NONNULL(h0);
  CODA_NONNULL(z);
  CODA_NONNULL(gamma);
  CODA_NONNULL(h1);
  CODA_NONNULL(r);
  CODA_NONNULL(o);
  CODA_ALIGN16(h0);
  CODA_ALIGN16(z);
  CODA_ALIGN16(gamma);
  CODA_ALIGN16(h1);
  CODA_ALIGN16(o);
  CODA_TRY(check_disjoint({bf16_span(h1, M, D), f32_span(r, M), bf16_span(o, M, D)},
                          {bf16_span(h0, M, D), bf16_span(z, M, D), bf16_span(gamma, D)}));
  hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(M), dim3(256), 0, as_stream(stream), h0, z, gamma, D, eps, h1, r,
                     o);
  return launch_status();
}

int coda_baseline_rowdot(const uint16_t* a, const uint16_t* b, int M, int D, float* s, void* stream) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(D));
  if (M == 0) return CODA_OK;
  CODA_NONNULL(a);
  CODA_NONNULL(b);
  CODA_NONNULL(s);
  CODA_ALIGN16(a);
  CODA_ALIGN16(b);
  CODA_TRY(check_disjoint({f32_span(s, M)}, {bf16_span(a, M, D), bf16_span(b, M, D)}));
  hipLaunchKernelGGL(rowdot_kernel, dim3(M), dim3(256), 0, as_stream(stream), a, b, D, s);
  return launch_status();
}

int coda_baseline_rope(const uint16_t* h, const float* cos_t, const float* sin_t, int M, int n_q, int n_k, int n_v,
                       int head_dim, int seq_len, int pos_offset, uint16_t* out, void* stream) {
  CODA_TRY(check_rows(M));
  if (head_dim < 8 || head_dim % 8 != 0) return CODA_ERR_SHAPE;
  if (n_q < 0 || n_k < 0 || n_v < 0 || n_q % head_dim || n_k % head_dim || n_v % head_dim) return CODA_ERR_SHAPE;
  const long long N = (long long)n_q + n_k + n_v;
  if (N < 8 || N > kMaxDim) return CODA_ERR_SHAPE;
  if (seq_len < 1 || pos_offset < 0) return CODA_ERR_ARG;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(h);
  CODA_NONNULL(cos_t);
  CODA_NONNULL(sin_t);
  CODA_NONNULL(out);
  CODA_ALIGN16(h);
  CODA_ALIGN16(out);
  if (!aligned(cos_t, 16) || !aligned(sin_t, 16)) return CODA_ERR_ALIGN;
  const long long tab = (long long)seq_len * (head_dim / 2);
  CODA_TRY(check_disjoint({bf16_span(out, M, N)}, {bf16_span(h, M, N), f32_span(cos_t, tab), f32_span(sin_t, tab)}));
  const long long n = (long long)M * (N / 8);
  hipLaunchKernelGGL(rope_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, as_stream(stream), h, cos_t, sin_t, M,
                     (int)N, n_q + n_k, head_dim, seq_len, pos_offset, out);
  return launch_status();
}

int coda_baseline_swiglu(const uint16_t* h, int M, int F, uint16_t* out, void* stream) {
  CODA_TRY(check_rows(M));
  if (F < 8 || F % 8 != 0 || 2LL * F > kMaxDim) return CODA_ERR_SHAPE;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(h);
  CODA_NONNULL(out);
  CODA_ALIGN16(h);
  CODA_ALIGN16(out);
  CODA_TRY(check_disjoint({bf16_span(out, M, F)}, {bf16_span(h, M, 2LL * F)}));
  const long long n = (long long)M * (F / 4);
  hipLaunchKernelGGL(swiglu_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, as_stream(stream), h, M, F, out);
  return launch_status();
}

int coda_baseline_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  CODA_NONNULL(src);
  CODA_NONNULL(dst);
  if (bytes <= 0 || bytes % 16 != 0) return CODA_ERR_SHAPE;
  CODA_ALIGN16(src);
  CODA_ALIGN16(dst);
  CODA_TRY(check_disjoint({Span{dst, (uint64_t)bytes}}, {Span{src, (uint64_t)bytes}}));
  const long long n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<long long>(blocks_for(n16, 256), 256LL * 16);
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, as_stream(stream), (const u32x4_t*)src, (u32x4_t*)dst,
                     n16);
  return launch_status();
}

int coda_baseline_mfma_loop(const uint16_t* operands, int n_frag, int iters, int grid, float* out, void* stream) {
  if (n_frag < 1 || iters < 1 || grid < 1 || grid > 65535) return CODA_ERR_SHAPE;
  CODA_NONNULL(operands);
  CODA_NONNULL(out);
  CODA_ALIGN16(operands);
  if (!aligned(out, 4)) return CODA_ERR_ALIGN;
  CODA_TRY(check_disjoint({f32_span(out, (long long)grid * 512)}, {bf16_span(operands, n_frag, 8)}));
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(512), 0, as_stream(stream), (const bf16x8_t*)operands, n_frag,
                     iters, out);
  return launch_status();
}

}  // extern "C"

namespace {

// Main-loop schedule probe, a measurement kernel (no step of the method): the GEMM main
// loop's per-step LDS operand reads and MFMAs, with its read order, priorities and
// scheduling pins, on an LDS image written once before the timed loop (seed 0: every bf16
// element equal to `fill`; otherwise element bits from a hash of (seed, position), values
// +-[1/4, 1/2) with random signs and mantissas, since the MFMA's rate depends on the
// operand bits; nothing rewrites the image, so there is no DMA and no hazard). Kinds:
//   0  KN-W reads (two transposed 8-byte reads per W block), the per-step barrier
//   1  the same without the barrier
//   2  NK-W reads (one 16-byte read per W block), the per-step barrier
//   3  the reads of kind 0 alone, no MFMAs: every 32-bit word read is added (mod 2^32)
//   4  the MFMAs of kind 0 alone, on operands read once before the loop
//   5  kind 0 with only the W reads (the X operands read once before the loop)
//   6  kind 0 with only the X reads (the W operands read once before the loop)
//   7  kind 0 plus the GEMM's DMA issue into the ring (per wave and step, two W loads
//      after the first-half MFMAs and two X loads behind the second-half ones, into the
//      slots three and four steps ahead) through a descriptor of no bytes: every load
//      zero-fills its 1 KiB of LDS without touching memory. Only for the all-zero image
//      (fill 0, seed 0), which the zero fills leave unchanged, so no step waits for them;
//      they are all waited for after the timed loop, before the workgroup ends.
// out[thread]: kinds 0-2 and 4-6 the sum of the thread's 128 accumulator values; kind 3 the
// bits of its word sum. Each wave records the core-clock cycles of its `steps` steps
// (s_memtime) in cycles[].
template <int kKind>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void schedule_probe_kernel(float fill, uint32_t seed, int steps, float* __restrict__ out,
                           long long* __restrict__ cycles) {
  constexpr bool kKN = kKind != 2;
  constexpr bool kBarrier = kKind != 1 && kKind != 4;
  constexpr bool kMfma = kKind != 3;
  constexpr bool kReads = kKind != 4;
  constexpr bool kReadX = kReads && kKind != 5;
  constexpr bool kReadW = kReads && kKind != 6;
  constexpr bool kDma = kKind == 7;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kSlotBytes];
  const uint32_t fill2 = f32_to_bf16(fill) * 0x10001u;
  for (int i = threadIdx.x; i < kStages * kSlotBytes / 4; i += kThreads) {
    uint32_t h = (uint32_t)i * 0x9E3779B1u ^ seed * 0x85EBCA77u;  // multiplicative hash and mix
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    h *= 0x297A2D39u;
    h ^= h >> 15;
    ((uint32_t*)smem)[i] = seed ? (h & 0x807F807Fu) | 0x3E803E80u : fill2;
  }
  __syncthreads();
  const LdsRing lds = make_ring(smem, 0, 0, threadIdx.x);
  const GemmProblem p{nullptr, nullptr, kBM, kBN, kBK, 0};  // only the LDS offsets are used
  Mainloop<kKN> ml;
  ml.init(p, threadIdx.x);
  AccTile acc;
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t rsum = 0u;
  constexpr int kH = kMJ / 2;
  constexpr int kMfmaH = kNI * kH;
  bf16x8_t a[kNI], b[kMJ];
#pragma unroll
  for (int i = 0; i < kNI; ++i) a[i] = ml.read_w(lds.slot[0], i);
#pragma unroll
  for (int j = 0; j < (kReadX ? kH : kMJ); ++j) b[j] = ml.read_x(lds.slot[0], j);
  auto use = [&](int i, int j) {
    if constexpr (kMfma)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  auto fold = [&](const bf16x8_t& v) {
    if constexpr (!kMfma) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, v);
      rsum += (w.x + w.y) + (w.z + w.w);
    }
  };
  const i32x4_t none = rsrc_words(out, 0u);  // no bytes: every load zero-fills
  const uint32_t wave_off = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (kXJ * 1024u);
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  auto step = [&](const int S) {
#pragma unroll
    for (int j = kH; j < kMJ; ++j) {
      if constexpr (kReadX) b[j] = ml.read_x(lds.slot[S], j);
      fold(b[j]);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
      for (int j = 0; j < kH; ++j) use(i, j);
    __builtin_amdgcn_sched_group_barrier(0x100, kH, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaH, 0);
    if constexpr (kDma) {
      const uint32_t w3 = lds_addr(lds.slot[(S + 3) % kStages]) + (uint32_t)kTileBytes + wave_off;
      dma16(none, w3, 0u);
      dma16(none, w3 + 1024u, 0u);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kBarrier) __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const char* next = lds.slot[(S + 1) % kStages];
#pragma unroll
    for (int r = 0; r < kMfmaH; ++r) {
      const int i = r / kH, j = kH + r % kH;
      use(i, j);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (kDma && (r == kMfmaH - 8 || r == kMfmaH - 4)) {
        const int q = r == kMfmaH - 8 ? 3 : 4;
        dma16(none, lds_addr(lds.slot[(S + q) % kStages]) + wave_off, 0u);
      }
      if (kReadX && r < kH) {
        b[r] = ml.read_x(next, r);
        fold(b[r]);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      if (kReadW && r % kH == kH - 1) {
        a[i] = ml.read_w(next, i);
        fold(a[i]);
        __builtin_amdgcn_sched_group_barrier(0x100, kKN ? 2 : 1, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s + kStages <= steps; s += kStages) {
    step(0);
    step(1);
    step(2);
    step(3);
    step(4);
  }
  if (s < steps) step(0);
  if (s + 1 < steps) step(1);
  if (s + 2 < steps) step(2);
  if (s + 3 < steps) step(3);
  const long long t1 = __builtin_amdgcn_s_memtime();
  if constexpr (kDma) {
    wait_vmcnt<0>();  // every zero fill has landed before the workgroup's LDS is given back
    __syncthreads();
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j) sum += (acc[i][j][0] + acc[i][j][1]) + (acc[i][j][2] + acc[i][j][3]);
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = kMfma ? sum : __uint_as_float(rsum);
  if ((threadIdx.x & 63) == 0) cycles[(size_t)blockIdx.x * kWaves + (threadIdx.x >> 6)] = t1 - t0;
}

}  // namespace

extern "C" {

int coda_baseline_schedule_probe(int kind, int steps, int grid, float fill, uint32_t seed, float* out,
                                 long long* cycles, void* stream) {
  if (kind < 0 || kind > 7 || steps < 1 || grid < 1 || grid > 65535) return CODA_ERR_SHAPE;
  if (kind == 7 && (fill != 0.0f || seed != 0u)) return CODA_ERR_ARG;  // the zero image only
  CODA_NONNULL(out);
  CODA_NONNULL(cycles);
  if (!aligned(out, 4) || !aligned(cycles, 8)) return CODA_ERR_ALIGN;
  CODA_TRY(check_disjoint({f32_span(out, (long long)grid * kThreads), Span{cycles, 8ull * grid * kWaves}}, {}));
  const hipStream_t st = as_stream(stream);
  switch (kind) {
    case 0: hipLaunchKernelGGL(schedule_probe_kernel<0>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    case 1: hipLaunchKernelGGL(schedule_probe_kernel<1>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    case 2: hipLaunchKernelGGL(schedule_probe_kernel<2>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    case 3: hipLaunchKernelGGL(schedule_probe_kernel<3>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    case 5: hipLaunchKernelGGL(schedule_probe_kernel<5>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    case 6: hipLaunchKernelGGL(schedule_probe_kernel<6>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    case 7: hipLaunchKernelGGL(schedule_probe_kernel<7>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
    default: hipLaunchKernelGGL(schedule_probe_kernel<4>, dim3(grid), dim3(kThreads), 0, st, fill, seed, steps, out, cycles); break;
  }
  return launch_status();
}

}  // extern "C"
