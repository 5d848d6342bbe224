// C-ABI entry points of GEMM + cross-entropy (declared in coda.h): the GEMM whose
// epilogue emits per-tile log-sum-exp partials and the label logit, and the auxiliary
// merge into lse and the loss.
#include "coda_abi.hpp"
#include "coda_ce.hpp"
#include "coda_launch.hpp"

using namespace coda;

namespace {

// One thread per row: lse = M + log sum_t exp(lse_t - M) with M = max_t lse_t, the sum
// in the order t = 0, 1, ..., nb-1; loss = lse - target for a label in [0, V), else 0
// (and target is set to 0 for such an ignored row).
constexpr int kLseThreads = 256;

__global__ __launch_bounds__(kLseThreads) void lse_reduce_kernel(const float* __restrict__ P, const int32_t* labels,
                                                                 int M, int nb, int V, float* __restrict__ target,
                                                                 float* __restrict__ lse, float* __restrict__ loss) {
  const int m = blockIdx.x * kLseThreads + threadIdx.x;
  if (m >= M) return;
  const float* row = P + (size_t)m * nb;
  float mx = row[0];
  for (int t = 1; t < nb; ++t) mx = fmaxf(mx, row[t]);
  float s = 0.f;
  for (int t = 0; t < nb; ++t) s += expf(row[t] - mx);
  const float l = mx + logf(s);
  const int lab = labels[m];
  const bool valid = lab >= 0 && lab < V;
  lse[m] = l;
  if (valid) {
    loss[m] = l - target[m];
  } else {
    loss[m] = 0.f;
    target[m] = 0.f;
  }
}

// The same merge with 16 lanes per row (one DPP row; 4 rows per wave): lane c holds the R
// partials t = c R .. c R + R - 1. The row maximum is a 16-lane reduction (exact in any
// order); the sum of exp(t - max) passes from lane to lane in chunk order (a DPP shift by
// one within the row), so every row is still summed in the order t = 0, 1, ..., nb - 1: the
// same fp32 operations as one thread per row, bit for bit, with M / 4 waves in flight
// instead of M / 64 (at 8192 rows x 128 tiles: 35 -> a few microseconds).
constexpr int kLseMaxR = 32;  // nb <= 16 * 32 = 512 (vocabularies up to 131072)

template <int R>
__global__ __launch_bounds__(kLseThreads) void lse_chain_kernel(const float* __restrict__ P, const int32_t* labels,
                                                                int M, int nb, int V, float* __restrict__ target,
                                                                float* __restrict__ lse, float* __restrict__ loss) {
  const int lane = threadIdx.x & 63, c = lane & 15;
  const long long m = ((long long)blockIdx.x * (kLseThreads / 64) + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool ok = m < M;  // lanes of rows past M still take part in the lane exchanges
  const float ninf = -__builtin_huge_valf();
  float v[R];
  float mx = ninf;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int t = c * R + k;
    v[k] = (ok && t < nb) ? P[m * nb + t] : ninf;
    mx = fmaxf(mx, v[k]);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float e[R];  // every lane's exponentials at once; only the in-order adds run lane by lane
#pragma unroll
  for (int j = 0; j < R; ++j) e[j] = expf(v[j] - mx);
  float run = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float in =
        __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, run), 0x111, 0xF, 0xF, false));
    if (c == k) {
      run = k == 0 ? 0.f : in;  // row_shr:1: lane c receives lane c - 1
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (c * R + j < nb) run += e[j];
    }
  }
  if (c == 15 && ok) {
    const float l = mx + logf(run);
    const int lab = labels[m];
    lse[m] = l;
    if (lab >= 0 && lab < V) {
      loss[m] = l - target[m];
    } else {
      loss[m] = 0.f;
      target[m] = 0.f;
    }
  }
}

int check_ce_outputs(const int32_t* labels, float* target, float* lse, float* loss) {
  CODA_NONNULL(labels);
  CODA_NONNULL(target);
  CODA_NONNULL(lse);
  CODA_NONNULL(loss);
  if (!aligned(labels, 4) || !aligned(target, 4) || !aligned(lse, 4) || !aligned(loss, 4)) return CODA_ERR_ALIGN;
  return CODA_OK;
}

int launch_lse(const float* P, const int32_t* labels, int M, int nb, int V, float* target, float* lse, float* loss,
               hipStream_t st) {
  if (nb > 16 * kLseMaxR) {
    hipLaunchKernelGGL(lse_reduce_kernel, dim3((M + kLseThreads - 1) / kLseThreads), dim3(kLseThreads), 0, st, P,
                       labels, M, nb, V, target, lse, loss);
    return launch_status();
  }
  const dim3 grid((unsigned)((M + 4 * (kLseThreads / 64) - 1) / (4 * (kLseThreads / 64))));
  const int R = (nb + 15) / 16;
  if (R <= 1)
    hipLaunchKernelGGL(lse_chain_kernel<1>, grid, dim3(kLseThreads), 0, st, P, labels, M, nb, V, target, lse, loss);
  else if (R <= 2)
    hipLaunchKernelGGL(lse_chain_kernel<2>, grid, dim3(kLseThreads), 0, st, P, labels, M, nb, V, target, lse, loss);
  else if (R <= 4)
    hipLaunchKernelGGL(lse_chain_kernel<4>, grid, dim3(kLseThreads), 0, st, P, labels, M, nb, V, target, lse, loss);
  else if (R <= 8)
    hipLaunchKernelGGL(lse_chain_kernel<8>, grid, dim3(kLseThreads), 0, st, P, labels, M, nb, V, target, lse, loss);
  else if (R <= 16)
    hipLaunchKernelGGL(lse_chain_kernel<16>, grid, dim3(kLseThreads), 0, st, P, labels, M, nb, V, target, lse, loss);
  else
    hipLaunchKernelGGL(lse_chain_kernel<32>, grid, dim3(kLseThreads), 0, st, P, labels, M, nb, V, target, lse, loss);
  return launch_status();
}

int gemm_ce(const uint16_t* x, const uint16_t* w, const int32_t* labels, int M, int K, int V, float* tile_lse,
            float* target, float* lse, float* loss, bool split, void* workspace, long long workspace_bytes,
            hipStream_t st) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  CODA_TRY(check_depth_or_width(V));
  if (split && workspace_bytes < 0) return CODA_ERR_ARG;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(x);
  CODA_NONNULL(w);
  CODA_NONNULL(tile_lse);
  CODA_ALIGN16(x);
  CODA_ALIGN16(w);
  if (!aligned(tile_lse, 4)) return CODA_ERR_ALIGN;
  const int nb = (V + kBN - 1) / kBN;
  CODA_TRY(check_ce_outputs(labels, target, lse, loss));
  CODA_TRY(check_disjoint({f32_span(tile_lse, M, nb), f32_span(target, M), f32_span(lse, M), f32_span(loss, M)},
                          {bf16_span(x, M, K), bf16_span(w, K, V), Span{labels, (uint64_t)M * 4u}}));
  const GemmProblem p{x, w, M, V, K};
  const EpiCrossEntropy::Args ea{labels, tile_lse, target, nb};
  SplitPlan sp{1, 0};
  if (split)
    CODA_TRY(split_for_call(M, V, K, workspace, workspace_bytes,
                            {f32_span(tile_lse, M, nb), f32_span(target, M), f32_span(lse, M), f32_span(loss, M),
                             bf16_span(x, M, K), bf16_span(w, K, V), Span{labels, (uint64_t)M * 4u}},
                            &sp));
  CODA_TRY((launch_gemm_split<true, EpiCrossEntropy>(p, ea, sp, static_cast<float*>(workspace), st)));
  return launch_lse(tile_lse, labels, M, nb, V, target, lse, loss, st);
}

}  // namespace

extern "C" {

int coda_lse_reduce(const float* tile_lse, const int32_t* labels, int M, int nb, int V, float* target, float* lse,
                    float* loss, void* stream) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(V));
  if (nb != (V + kBN - 1) / kBN) return CODA_ERR_SHAPE;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(tile_lse);
  if (!aligned(tile_lse, 4)) return CODA_ERR_ALIGN;
  CODA_TRY(check_ce_outputs(labels, target, lse, loss));
  // target is read and rewritten (zero on ignored rows): an output
  CODA_TRY(check_disjoint({f32_span(target, M), f32_span(lse, M), f32_span(loss, M)},
                          {f32_span(tile_lse, M, nb), Span{labels, (uint64_t)M * 4u}}));
  return launch_lse(tile_lse, labels, M, nb, V, target, lse, loss, as_stream(stream));
}

int coda_gemm_cross_entropy(const uint16_t* x, const uint16_t* w, const int32_t* labels, int M, int K, int V,
                            float* tile_lse, float* target, float* lse, float* loss, void* stream) {
  return gemm_ce(x, w, labels, M, K, V, tile_lse, target, lse, loss, false, nullptr, 0, as_stream(stream));
}

int coda_gemm_cross_entropy_ws(const uint16_t* x, const uint16_t* w, const int32_t* labels, int M, int K, int V,
                               float* tile_lse, float* target, float* lse, float* loss, void* workspace,
                               long long workspace_bytes, void* stream) {
  return gemm_ce(x, w, labels, M, K, V, tile_lse, target, lse, loss, true, workspace, workspace_bytes,
                 as_stream(stream));
}

}  // extern "C"
