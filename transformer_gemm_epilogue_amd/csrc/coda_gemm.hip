// C-ABI entry points of the fused GEMM-epilogue programs (declared in coda.h).
#include <mutex>

#include "coda_abi.hpp"
#include "coda_gemm.hpp"
#include "coda_launch.hpp"

using namespace coda;

int coda_rowstat_reduce_impl(const float* partials, int M, int nb, int d, float eps, int mode,
                             float* out, hipStream_t stream);

namespace {

// Persistent schedule: min(tiles, CUs of the current device) workgroups walk the tiles
// (one workgroup fills a CU's LDS); below the minimum depth the per-tile kernel runs
// instead. Both give bit-identical results.
template <bool kWKN, class Epi>
int launch_gemm_persistent(const GemmProblem& p, const typename Epi::Args& ea, hipStream_t stream) {
  if ((p.K + kBK - 1) / kBK < kPersistMinSteps) return launch_gemm<kWKN, Epi>(p, ea, stream);
  int cus = 0;
  CODA_TRY(device_cus(&cus));
  const int tiles = gemm_grid(p.M, p.N);
  const int grid = tiles < cus ? tiles : cus;
  hipLaunchKernelGGL((gemm_persistent_kernel<kWKN, Epi>), dim3(grid), dim3(kThreads), 0, stream, p, ea);
  return launch_status();
}

// Shape rules first; an empty batch (M == 0) needs no buffers at all, so pointers are
// checked only when there is work to do.
int check_gemm1(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma, int M,
                int K, int D, uint16_t* h1, uint16_t* h2, float* partials) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  CODA_TRY(check_depth_or_width(D));
  if (M == 0) return CODA_OK;
  CODA_NONNULL(x);
  CODA_NONNULL(w0);
  CODA_NONNULL(z);
  CODA_NONNULL(gamma);
  CODA_NONNULL(h1);
  CODA_NONNULL(h2);
  CODA_NONNULL(partials);
  CODA_ALIGN16(x);
  CODA_ALIGN16(w0);
  CODA_ALIGN16(z);
  CODA_ALIGN16(gamma);
  CODA_ALIGN16(h1);
  CODA_ALIGN16(h2);
  if (!aligned(partials, 4)) return CODA_ERR_ALIGN;
  return CODA_OK;
}

int disjoint_gemm1(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma, int M, int K,
                   int D, uint16_t* h1, uint16_t* h2, float* partials) {
  const int nb = (D + kBN - 1) / kBN;
  return check_disjoint({bf16_span(h1, M, D), bf16_span(h2, M, D), f32_span(partials, M, nb)},
                        {bf16_span(x, M, K), bf16_span(w0, K, D), bf16_span(z, M, D), bf16_span(gamma, D)});
}

int check_gemm2(const uint16_t* h2, const uint16_t* w1, const float* r, int M, int D, int N1, uint16_t* y) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(D));
  CODA_TRY(check_depth_or_width(N1));
  if (M == 0) return CODA_OK;
  CODA_NONNULL(h2);
  CODA_NONNULL(w1);
  CODA_NONNULL(r);
  CODA_NONNULL(y);
  CODA_ALIGN16(h2);
  CODA_ALIGN16(w1);
  CODA_ALIGN16(y);
  if (!aligned(r, 4)) return CODA_ERR_ALIGN;
  return CODA_OK;
}

// The three stages' buffers together: h2 and r are outputs that later stages read back;
// x, w0, z, gamma and w1 are inputs.
int disjoint_fwd(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma,
                 const uint16_t* w1, int M, int K, int D, int N1, uint16_t* h1, uint16_t* h2, float* partials,
                 float* r, uint16_t* y) {
  return check_disjoint({bf16_span(h1, M, D), bf16_span(h2, M, D), f32_span(partials, M, (D + kBN - 1) / kBN),
                         f32_span(r, M), bf16_span(y, M, N1)},
                        {bf16_span(x, M, K), bf16_span(w0, K, D), bf16_span(z, M, D), bf16_span(gamma, D),
                         bf16_span(w1, D, N1)});
}

int run_gemm1(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma, int M, int K,
              int D, uint16_t* h1, uint16_t* h2, float* partials, hipStream_t s) {
  const GemmProblem p{x, w0, M, D, K};
  const EpiResidualRmsPartials::Args ea{z, gamma, h1, h2, partials, (D + kBN - 1) / kBN};
  return launch_gemm<true, EpiResidualRmsPartials>(p, ea, s);
}

int run_gemm2(const uint16_t* h2, const uint16_t* w1, const float* r, int M, int D, int N1, uint16_t* y,
              hipStream_t s) {
  const GemmProblem p{h2, w1, M, N1, D};
  const EpiRowScale::Args ea{r, y};
  return launch_gemm<true, EpiRowScale>(p, ea, s);
}

}  // namespace

extern "C" {

const char* coda_status_string(int status) {
  switch (status) {
    case CODA_OK: return "CODA_OK";
    case CODA_ERR_NULL: return "CODA_ERR_NULL: a required pointer is NULL";
    case CODA_ERR_SHAPE: return "CODA_ERR_SHAPE: a size violates the shape rules";
    case CODA_ERR_ALIGN: return "CODA_ERR_ALIGN: a pointer is misaligned";
    case CODA_ERR_WORKSPACE: return "CODA_ERR_WORKSPACE: workspace too small";
    case CODA_ERR_HIP: return "CODA_ERR_HIP: a HIP launch failed";
    case CODA_ERR_ARG: return "CODA_ERR_ARG: invalid argument";
    default: return "unknown status";
  }
}

int coda_abi_version(void) { return 103; }

#ifndef CODA_SOURCE_HASH
#define CODA_SOURCE_HASH "unknown"
#endif
const char* coda_build_source_hash(void) { return CODA_SOURCE_HASH; }

int coda_rowstat_num_partials(int width, int* nb) {
  CODA_NONNULL(nb);
  if (width < 1) return CODA_ERR_SHAPE;
  *nb = (int)(((long long)width + CODA_PARTIAL_TILE_N - 1) / CODA_PARTIAL_TILE_N);
  return CODA_OK;
}

int coda_gemm_residual_rmsnorm_partials(const uint16_t* x, const uint16_t* w0, const uint16_t* z,
                                        const uint16_t* gamma, int M, int K, int D, uint16_t* h1,
                                        uint16_t* h2, float* partials, void* stream) {
  CODA_TRY(check_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials));
  if (M == 0) return CODA_OK;
  CODA_TRY(disjoint_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials));
  return run_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials, as_stream(stream));
}

int coda_gemm_rowscale(const uint16_t* h2, const uint16_t* w1, const float* r, int M, int D, int N1,
                       uint16_t* y, void* stream) {
  CODA_TRY(check_gemm2(h2, w1, r, M, D, N1, y));
  if (M == 0) return CODA_OK;
  CODA_TRY(check_disjoint({bf16_span(y, M, N1)}, {bf16_span(h2, M, D), bf16_span(w1, D, N1), f32_span(r, M)}));
  return run_gemm2(h2, w1, r, M, D, N1, y, as_stream(stream));
}

int coda_gemm_rmsnorm_fwd(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma,
                          const uint16_t* w1, int M, int K, int D, int N1, float eps, uint16_t* h1,
                          uint16_t* h2, float* partials, float* r, uint16_t* y, void* stream) {
  if (!(eps >= 0.0f) || !(eps < __builtin_huge_valf())) return CODA_ERR_ARG;
  CODA_TRY(check_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials));
  CODA_TRY(check_gemm2(h2, w1, r, M, D, N1, y));
  if (M == 0) return CODA_OK;
  CODA_TRY(disjoint_fwd(x, w0, z, gamma, w1, M, K, D, N1, h1, h2, partials, r, y));
  const hipStream_t s = as_stream(stream);
  CODA_TRY(run_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials, s));
  CODA_TRY(coda_rowstat_reduce_impl(partials, M, (D + kBN - 1) / kBN, D, eps, CODA_ROWSTAT_RSQRT_MEAN_EPS, r, s));
  return run_gemm2(h2, w1, r, M, D, N1, y, s);
}

// ----------------------------------------------------- forward with the split-depth schedule
int coda_gemm_rmsnorm_fwd_workspace_bytes(int M, int K, int D, int N1, long long* bytes) {
  CODA_NONNULL(bytes);
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  CODA_TRY(check_depth_or_width(D));
  CODA_TRY(check_depth_or_width(N1));
  *bytes = 0;
  if (M == 0) return CODA_OK;
  int cus = 0;
  CODA_TRY(device_cus(&cus));
  const long long f1 = split_workspace_floats(M, D, split_plan(M, D, K, cus));
  const long long f2 = split_workspace_floats(M, N1, split_plan(M, N1, D, cus));
  *bytes = 4 * std::max(f1, f2);
  return CODA_OK;
}

int coda_gemm_rmsnorm_fwd_ws(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma,
                             const uint16_t* w1, int M, int K, int D, int N1, float eps, uint16_t* h1,
                             uint16_t* h2, float* partials, float* r, uint16_t* y, void* workspace,
                             long long workspace_bytes, void* stream) {
  if (!(eps >= 0.0f) || !(eps < __builtin_huge_valf())) return CODA_ERR_ARG;
  if (workspace_bytes < 0) return CODA_ERR_ARG;
  CODA_TRY(check_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials));
  CODA_TRY(check_gemm2(h2, w1, r, M, D, N1, y));
  if (M == 0) return CODA_OK;
  CODA_TRY(disjoint_fwd(x, w0, z, gamma, w1, M, K, D, N1, h1, h2, partials, r, y));
  int cus = 0;
  CODA_TRY(device_cus(&cus));
  const SplitPlan sp1 = split_plan(M, D, K, cus), sp2 = split_plan(M, N1, D, cus);
  const long long need = 4 * std::max(split_workspace_floats(M, D, sp1), split_workspace_floats(M, N1, sp2));
  if (need > 0) {
    CODA_NONNULL(workspace);
    CODA_ALIGN16(workspace);
    if (workspace_bytes < need) return CODA_ERR_WORKSPACE;
    CODA_TRY(check_disjoint({Span{workspace, (uint64_t)need}},
                            {bf16_span(x, M, K), bf16_span(w0, K, D), bf16_span(z, M, D), bf16_span(gamma, D),
                             bf16_span(w1, D, N1), bf16_span(h1, M, D), bf16_span(h2, M, D),
                             f32_span(partials, M, (D + kBN - 1) / kBN), f32_span(r, M), bf16_span(y, M, N1)}));
  }
  float* ws = static_cast<float*>(workspace);
  const hipStream_t s = as_stream(stream);
  const int nb = (D + kBN - 1) / kBN;
  CODA_TRY((launch_gemm_split<true, EpiResidualRmsPartials>(GemmProblem{x, w0, M, D, K},
                                                            EpiResidualRmsPartials::Args{z, gamma, h1, h2, partials, nb},
                                                            sp1, ws, s)));
  CODA_TRY(coda_rowstat_reduce_impl(partials, M, nb, D, eps, CODA_ROWSTAT_RSQRT_MEAN_EPS, r, s));
  return launch_gemm_split<true, EpiRowScale>(GemmProblem{h2, w1, M, N1, D}, EpiRowScale::Args{r, y}, sp2, ws, s);
}

// ----------------------------------------------------------- forward without allocation
// The row-partial workspace of the forward rewrite in a fixed device array, for callers
// that cannot allocate device memory. Each GPU the library runs on holds its own copy of
// the array (at its own address) until the process ends. In host code `scratch` names a
// host-side stand-in, never the device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) float scratch[CODA_NOALLOC_SCRATCH_FLOATS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CODA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CODA_ERR_HIP;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return CODA_OK;
}
}  // namespace

int coda_gemm_rmsnorm_fwd_noalloc(const uint16_t* x, const uint16_t* w0, const uint16_t* z, const uint16_t* gamma,
                                  const uint16_t* w1, int M, int K, int D, int N1, float eps, uint16_t* h1,
                                  uint16_t* h2, float* r, uint16_t* y, void* stream) {
  if (!(eps >= 0.0f) || !(eps < __builtin_huge_valf())) return CODA_ERR_ARG;
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  CODA_TRY(check_depth_or_width(D));
  CODA_TRY(check_depth_or_width(N1));
  const int nb = (D + kBN - 1) / kBN;
  if ((long long)M * nb > CODA_NOALLOC_SCRATCH_FLOATS) return CODA_ERR_WORKSPACE;
  if (M == 0) return CODA_OK;
  float* partials = nullptr;
  CODA_TRY(scratch_on_current_device(&partials));
  CODA_TRY(check_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials));
  CODA_TRY(check_gemm2(h2, w1, r, M, D, N1, y));
  CODA_TRY(disjoint_fwd(x, w0, z, gamma, w1, M, K, D, N1, h1, h2, partials, r, y));
  // every partial the reduction reads is written by GEMM1 first: nothing to clear
  const hipStream_t s = as_stream(stream);
  CODA_TRY(run_gemm1(x, w0, z, gamma, M, K, D, h1, h2, partials, s));
  CODA_TRY(coda_rowstat_reduce_impl(partials, M, nb, D, eps, CODA_ROWSTAT_RSQRT_MEAN_EPS, r, s));
  return run_gemm2(h2, w1, r, M, D, N1, y, s);
}

namespace {
enum class Schedule { kPerTile, kPersistent, kSplit };

int gemm_rope(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int M, int K, int n_q,
              int n_k, int n_v, int head_dim, int seq_len, int pos_offset, uint16_t* out, int inverse,
              Schedule schedule, hipStream_t stream, void* workspace = nullptr, long long workspace_bytes = 0) {
  if (schedule == Schedule::kSplit && workspace_bytes < 0) return CODA_ERR_ARG;
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  if (head_dim < 8 || head_dim % 8 != 0 || head_dim > kMaxDim) return CODA_ERR_SHAPE;
  if (n_q < 0 || n_k < 0 || n_v < 0 || n_q % head_dim || n_k % head_dim || n_v % head_dim) return CODA_ERR_SHAPE;
  const long long N = (long long)n_q + n_k + n_v;
  if (N < 8 || N > kMaxDim) return CODA_ERR_SHAPE;
  if (seq_len < 1 || pos_offset < 0) return CODA_ERR_ARG;
  if ((long long)seq_len * head_dim > (1LL << 29)) return CODA_ERR_SHAPE;  // each table stays < 2^31 bytes
  if (M == 0) return CODA_OK;
  CODA_NONNULL(x);
  CODA_NONNULL(w);
  CODA_NONNULL(cos_t);
  CODA_NONNULL(sin_t);
  CODA_NONNULL(out);
  CODA_ALIGN16(x);
  CODA_ALIGN16(w);
  CODA_ALIGN16(out);
  if (!aligned(cos_t, 8) || !aligned(sin_t, 8)) return CODA_ERR_ALIGN;
  const long long tab = (long long)seq_len * (head_dim / 2);
  CODA_TRY(check_disjoint({bf16_span(out, M, N)},
                          {bf16_span(x, M, K), bf16_span(w, K, N), f32_span(cos_t, tab), f32_span(sin_t, tab)}));
  const GemmProblem p{x, w, M, (int)N, K};
  const EpiRope::Args ea{cos_t, sin_t, out, n_q + n_k, head_dim, seq_len, pos_offset, inverse};
  if (schedule == Schedule::kPersistent) return launch_gemm_persistent<true, EpiRope>(p, ea, stream);
  if (schedule == Schedule::kSplit) {
    SplitPlan sp;
    CODA_TRY(split_for_call(M, (int)N, K, workspace, workspace_bytes,
                            {bf16_span(out, M, N), bf16_span(x, M, K), bf16_span(w, K, N), f32_span(cos_t, tab),
                             f32_span(sin_t, tab)},
                            &sp));
    return launch_gemm_split<true, EpiRope>(p, ea, sp, static_cast<float*>(workspace), stream);
  }
  return launch_gemm<true, EpiRope>(p, ea, stream);
}
int gemm_swiglu(const uint16_t* x, const uint16_t* w, int M, int K, int F, uint16_t* out, bool split, void* workspace,
                long long workspace_bytes, hipStream_t stream) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  if (F < 8 || F % 8 != 0 || 2LL * F > kMaxDim) return CODA_ERR_SHAPE;
  if (split && workspace_bytes < 0) return CODA_ERR_ARG;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(x);
  CODA_NONNULL(w);
  CODA_NONNULL(out);
  CODA_ALIGN16(x);
  CODA_ALIGN16(w);
  CODA_ALIGN16(out);
  CODA_TRY(check_disjoint({bf16_span(out, M, F)}, {bf16_span(x, M, K), bf16_span(w, K, 2LL * F)}));
  const GemmProblem p{x, w, M, 2 * F, K};
  const EpiSwiGLU::Args ea{out, F};
  if (!split) return launch_gemm<true, EpiSwiGLU>(p, ea, stream);
  SplitPlan sp;
  CODA_TRY(split_for_call(M, 2 * F, K, workspace, workspace_bytes,
                          {bf16_span(out, M, F), bf16_span(x, M, K), bf16_span(w, K, 2LL * F)}, &sp));
  return launch_gemm_split<true, EpiSwiGLU>(p, ea, sp, static_cast<float*>(workspace), stream);
}
int gemm_bwd_stats(const uint16_t* dy, const uint16_t* w1, const uint16_t* h2, int M, int D, int N, uint16_t* dh2,
                   float* partials, float* s, bool split, void* workspace, long long workspace_bytes,
                   hipStream_t st) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(D));
  CODA_TRY(check_depth_or_width(N));
  if (split && workspace_bytes < 0) return CODA_ERR_ARG;
  if (M == 0) return CODA_OK;
  CODA_NONNULL(dy);
  CODA_NONNULL(w1);
  CODA_NONNULL(h2);
  CODA_NONNULL(dh2);
  CODA_NONNULL(partials);
  CODA_NONNULL(s);
  CODA_ALIGN16(dy);
  CODA_ALIGN16(w1);
  CODA_ALIGN16(h2);
  CODA_ALIGN16(dh2);
  if (!aligned(partials, 4) || !aligned(s, 4)) return CODA_ERR_ALIGN;
  const int nb = (D + kBN - 1) / kBN;
  CODA_TRY(check_disjoint({bf16_span(dh2, M, D), f32_span(partials, M, nb), f32_span(s, M)},
                          {bf16_span(dy, M, N), bf16_span(w1, D, N), bf16_span(h2, M, D)}));
  // dy [M, N] times W1^T: depth = N, output width = D, W1 [D, N] is the NK layout.
  const GemmProblem p{dy, w1, M, D, N};
  const EpiDotRowPartials::Args ea{h2, dh2, partials, nb};
  if (split) {
    SplitPlan sp;
    CODA_TRY(split_for_call(M, D, N, workspace, workspace_bytes,
                            {bf16_span(dh2, M, D), f32_span(partials, M, nb), f32_span(s, M), bf16_span(dy, M, N),
                             bf16_span(w1, D, N), bf16_span(h2, M, D)},
                            &sp));
    CODA_TRY((launch_gemm_split<false, EpiDotRowPartials>(p, ea, sp, static_cast<float*>(workspace), st)));
  } else {
    CODA_TRY((launch_gemm<false, EpiDotRowPartials>(p, ea, st)));
  }
  return coda_rowstat_reduce_impl(partials, M, nb, D, 0.0f, CODA_ROWSTAT_MEAN, s, st);
}

}  // namespace

int coda_gemm_rope(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int M, int K,
                   int n_q, int n_k, int n_v, int head_dim, int seq_len, int pos_offset, uint16_t* out,
                   void* stream) {
  return gemm_rope(x, w, cos_t, sin_t, M, K, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out, 0,
                   Schedule::kPerTile, as_stream(stream));
}

int coda_gemm_rope_ws(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int M, int K,
                      int n_q, int n_k, int n_v, int head_dim, int seq_len, int pos_offset, uint16_t* out,
                      void* workspace, long long workspace_bytes, void* stream) {
  return gemm_rope(x, w, cos_t, sin_t, M, K, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out, 0, Schedule::kSplit,
                   as_stream(stream), workspace, workspace_bytes);
}

int coda_gemm_rope_persistent(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int M,
                              int K, int n_q, int n_k, int n_v, int head_dim, int seq_len, int pos_offset,
                              uint16_t* out, void* stream) {
  return gemm_rope(x, w, cos_t, sin_t, M, K, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out, 0,
                   Schedule::kPersistent, as_stream(stream));
}

int coda_gemm_rope_bwd(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int M, int K,
                       int n_q, int n_k, int n_v, int head_dim, int seq_len, int pos_offset, uint16_t* out,
                       void* stream) {
  return gemm_rope(x, w, cos_t, sin_t, M, K, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out, 1,
                   Schedule::kPerTile, as_stream(stream));
}

int coda_gemm_rope_bwd_ws(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int M, int K,
                          int n_q, int n_k, int n_v, int head_dim, int seq_len, int pos_offset, uint16_t* out,
                          void* workspace, long long workspace_bytes, void* stream) {
  return gemm_rope(x, w, cos_t, sin_t, M, K, n_q, n_k, n_v, head_dim, seq_len, pos_offset, out, 1, Schedule::kSplit,
                   as_stream(stream), workspace, workspace_bytes);
}

int coda_gemm_swiglu(const uint16_t* x, const uint16_t* w, int M, int K, int F, uint16_t* out, void* stream) {
  return gemm_swiglu(x, w, M, K, F, out, false, nullptr, 0, as_stream(stream));
}

int coda_gemm_swiglu_ws(const uint16_t* x, const uint16_t* w, int M, int K, int F, uint16_t* out, void* workspace,
                        long long workspace_bytes, void* stream) {
  return gemm_swiglu(x, w, M, K, F, out, true, workspace, workspace_bytes, as_stream(stream));
}

int coda_split_plan(int M, int N, int K, int cus, int* slices, int* steps, int* first_split_tile,
                    long long* bytes) {
  CODA_NONNULL(slices);
  CODA_NONNULL(steps);
  CODA_NONNULL(first_split_tile);
  CODA_NONNULL(bytes);
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(N));
  CODA_TRY(check_depth_or_width(K));
  if (cus < 1) return CODA_ERR_ARG;
  const SplitPlan sp = M == 0 ? SplitPlan{1, (K + kBK - 1) / kBK, 0} : split_plan(M, N, K, cus);
  *slices = sp.S;
  *steps = sp.steps;
  *first_split_tile = sp.tile0;
  *bytes = M == 0 ? 0 : 4 * split_workspace_floats(M, N, sp);
  return CODA_OK;
}

int coda_split_workspace_bytes(int M, int N, int K, long long* bytes) {
  CODA_NONNULL(bytes);
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(N));
  CODA_TRY(check_depth_or_width(K));
  *bytes = 0;
  if (M == 0) return CODA_OK;
  int cus = 0;
  CODA_TRY(device_cus(&cus));
  *bytes = 4 * split_workspace_floats(M, N, split_plan(M, N, K, cus));
  return CODA_OK;
}

int coda_gemm_rmsnorm_bwd_stats(const uint16_t* dy, const uint16_t* w1, const uint16_t* h2, int M, int D, int N,
                                uint16_t* dh2, float* partials, float* s, void* stream) {
  return gemm_bwd_stats(dy, w1, h2, M, D, N, dh2, partials, s, false, nullptr, 0, as_stream(stream));
}

int coda_gemm_rmsnorm_bwd_stats_ws(const uint16_t* dy, const uint16_t* w1, const uint16_t* h2, int M, int D, int N,
                                   uint16_t* dh2, float* partials, float* s, void* workspace,
                                   long long workspace_bytes, void* stream) {
  return gemm_bwd_stats(dy, w1, h2, M, D, N, dh2, partials, s, true, workspace, workspace_bytes, as_stream(stream));
}

int coda_baseline_gemm(const uint16_t* a, const uint16_t* b, int M, int K, int N, int b_kn, uint16_t* c,
                       void* stream) {
  CODA_TRY(check_rows(M));
  CODA_TRY(check_depth_or_width(K));
  CODA_TRY(check_depth_or_width(N));
  if (M == 0) return CODA_OK;
  CODA_NONNULL(a);
  CODA_NONNULL(b);
  CODA_NONNULL(c);
  CODA_ALIGN16(a);
  CODA_ALIGN16(b);
  CODA_ALIGN16(c);
  CODA_TRY(check_disjoint({bf16_span(c, M, N)}, {bf16_span(a, M, K), bf16_span(b, K, N)}));
  const GemmProblem p{a, b, M, N, K};
  const EpiStore::Args ea{c};
  if (b_kn) return launch_gemm<true, EpiStore>(p, ea, as_stream(stream));
  return launch_gemm<false, EpiStore>(p, ea, as_stream(stream));
}

}  // extern "C"
