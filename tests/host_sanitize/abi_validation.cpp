// Host-only driver for the C ABI's argument validation, built with the address and
// undefined-behaviour sanitizers (host code only, no device code object) and run on a
// machine without a GPU. Every entry point is called with NULL, misaligned, overlapping
// and extreme size arguments (every int argument swept over values around the shape
// limits and the int range); each call must return a status in range, and the calls
// that are invalid must be refused with the expected status. Calls whose arguments pass
// validation reach the HIP runtime, which, with no device present, must refuse them with
// CODA_ERR_HIP. Any sanitizer report aborts the run. Fake device pointers are never
// dereferenced by host code.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <climits>
#include <vector>

#include "coda.h"

static int failures = 0;
static long calls = 0;

#define EXPECT(cond, ...)                   \
  do {                                      \
    if (!(cond)) {                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);         \
      fprintf(stderr, "\n");                \
      ++failures;                           \
    }                                       \
  } while (0)

// distinct, 256-byte aligned fake device addresses, 2^36 bytes apart
static void* fake(int i) { return (void*)(uintptr_t)((1ull << 40) + (uint64_t)i * (1ull << 36)); }
template <class T>
static T* F(int i) { return (T*)fake(i); }

static const int kSweep[] = {INT_MIN, INT_MIN + 1, -8, -1, 0, 1, 7, 8, 9, 16, 255, 256, 257, 4096, (1 << 22) - 8,
                             1 << 22, (1 << 22) + 8, 1 << 24, (1 << 24) + 1, 1 << 29, INT_MAX - 7, INT_MAX};

static void status_ok(int st, const char* what) {
  ++calls;
  EXPECT(st >= CODA_OK && st <= CODA_ERR_ARG, "%s returned %d", what, st);
  // with no device, a call that passes validation and has work must fail in HIP
}

// Sweep one int argument (index k of n) over kSweep with the others at `base`.
template <class Fn>
static void sweep(const char* what, std::vector<int> base, Fn fn) {
  for (size_t k = 0; k < base.size(); ++k) {
    for (int v : kSweep) {
      std::vector<int> a = base;
      a[k] = v;
      status_ok(fn(a), what);
    }
  }
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    printf("SKIPPED: a GPU is visible; this driver is for hosts without one\n");
    return 0;
  }
  const uint16_t* b = F<const uint16_t>(0);
  // ---------------------------------------------------------------- forward rewrite
  auto fwd = [&](const std::vector<int>& a, float eps = 1e-5f) {
    return coda_gemm_rmsnorm_fwd(F<uint16_t>(1), F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), F<uint16_t>(5), a[0],
                                 a[1], a[2], a[3], eps, F<uint16_t>(6), F<uint16_t>(7), F<float>(8), F<float>(9),
                                 F<uint16_t>(10), nullptr);
  };
  sweep("coda_gemm_rmsnorm_fwd", {256, 256, 256, 256}, [&](const std::vector<int>& a) { return fwd(a); });
  EXPECT(fwd({256, 256, 256, 256}, -1.f) == CODA_ERR_ARG, "negative eps");
  EXPECT(fwd({256, 256, 256, 256}, __builtin_nanf("")) == CODA_ERR_ARG, "nan eps");
  EXPECT(fwd({256, 256, 256, 256}) == CODA_ERR_HIP, "valid arguments without a device");
  EXPECT(coda_gemm_rmsnorm_fwd(F<uint16_t>(1), F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), F<uint16_t>(5), 256, 256,
                               256, 256, 1e-5f, F<uint16_t>(6), F<uint16_t>(6), F<float>(8), F<float>(9),
                               F<uint16_t>(10), nullptr) == CODA_ERR_ARG,
         "h1 == h2");
  auto noalloc = [&](const std::vector<int>& a) {
    return coda_gemm_rmsnorm_fwd_noalloc(F<uint16_t>(1), F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4),
                                         F<uint16_t>(5), a[0], a[1], a[2], a[3], 1e-5f, F<uint16_t>(6),
                                         F<uint16_t>(7), F<float>(9), F<uint16_t>(10), nullptr);
  };
  sweep("coda_gemm_rmsnorm_fwd_noalloc", {256, 256, 256, 256}, noalloc);
  EXPECT(noalloc({CODA_NOALLOC_SCRATCH_FLOATS + 1, 256, 256, 256}) == CODA_ERR_WORKSPACE, "noalloc capacity");
  EXPECT(noalloc({256, 256, 256, 256}) == CODA_ERR_HIP, "noalloc without a device");
  sweep("coda_gemm_residual_rmsnorm_partials", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_residual_rmsnorm_partials(b, F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), a[0], a[1], a[2],
                                               F<uint16_t>(6), F<uint16_t>(7), F<float>(8), nullptr);
  });
  sweep("coda_gemm_rowscale", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_rowscale(b, F<uint16_t>(2), F<float>(3), a[0], a[1], a[2], F<uint16_t>(4), nullptr);
  });
  for (int mode : {-1, 0, 1, 2, INT_MAX})
    sweep("coda_rowstat_reduce", {256, 16, 4096}, [&](const std::vector<int>& a) {
      return coda_rowstat_reduce(F<float>(1), a[0], a[1], a[2], 1e-5f, mode, F<float>(2), nullptr);
    });
  int nb = 0;
  for (int v : kSweep) status_ok(coda_rowstat_num_partials(v, &nb), "coda_rowstat_num_partials");
  for (int v : kSweep) status_ok(coda_colstat_num_partials(v, &nb), "coda_colstat_num_partials");
  EXPECT(coda_rowstat_num_partials(8, nullptr) == CODA_ERR_NULL, "nb NULL");
  // ---------------------------------------------------------------- RoPE, SwiGLU
  sweep("coda_rope_tables", {64, 128}, [&](const std::vector<int>& a) {
    return coda_rope_tables(F<float>(1), F<float>(2), a[0], a[1], 1e4, nullptr);
  });
  for (auto fn : {coda_gemm_rope, coda_gemm_rope_persistent, coda_gemm_rope_bwd})
    sweep("coda_gemm_rope*", {256, 256, 128, 128, 128, 128, 256, 0}, [&](const std::vector<int>& a) {
      return fn(b, F<uint16_t>(2), F<float>(3), F<float>(4), a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7],
                F<uint16_t>(5), nullptr);
    });
  sweep("coda_gemm_swiglu", {256, 256, 128}, [&](const std::vector<int>& a) {
    return coda_gemm_swiglu(b, F<uint16_t>(2), a[0], a[1], a[2], F<uint16_t>(3), nullptr);
  });
  sweep("coda_gemm_swiglu_bwd", {256, 256, 128}, [&](const std::vector<int>& a) {
    return coda_gemm_swiglu_bwd(b, F<uint16_t>(2), F<uint16_t>(3), a[0], a[1], a[2], F<uint16_t>(4), nullptr);
  });
  // ---------------------------------------------------------------- backward
  sweep("coda_gemm_rmsnorm_bwd_stats", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_rmsnorm_bwd_stats(b, F<uint16_t>(2), F<uint16_t>(3), a[0], a[1], a[2], F<uint16_t>(4),
                                       F<float>(5), F<float>(6), nullptr);
  });
  sweep("coda_rowdot_stat", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_rowdot_stat(b, F<uint16_t>(2), a[0], a[1], a[2], F<float>(3), nullptr);
  });
  sweep("coda_colsum_reduce", {2, 256}, [&](const std::vector<int>& a) {
    return coda_colsum_reduce(F<float>(1), a[0], a[1], F<float>(2), nullptr);
  });
  sweep("coda_gemm_rmsnorm_bwd_dx", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_rmsnorm_bwd_dx(b, F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), F<float>(5), F<float>(6),
                                    F<uint16_t>(7), a[0], a[1], a[2], F<uint16_t>(8), F<float>(9), nullptr);
  });
  sweep("coda_rmsnorm_bwd", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_rmsnorm_bwd(b, F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), F<float>(5), F<uint16_t>(6),
                            F<uint16_t>(7), a[0], a[1], a[2], F<float>(8), F<uint16_t>(9), F<float>(10), F<float>(11),
                            nullptr);
  });
  // ---------------------------------------------------------------- cross-entropy
  sweep("coda_gemm_cross_entropy", {256, 256, 512}, [&](const std::vector<int>& a) {
    return coda_gemm_cross_entropy(b, F<uint16_t>(2), F<int32_t>(3), a[0], a[1], a[2], F<float>(4), F<float>(5),
                                   F<float>(6), F<float>(7), nullptr);
  });
  sweep("coda_lse_reduce", {256, 2, 512}, [&](const std::vector<int>& a) {
    return coda_lse_reduce(F<float>(1), F<int32_t>(2), a[0], a[1], a[2], F<float>(3), F<float>(4), F<float>(5),
                           nullptr);
  });
  // ---------------------------------------------------------------- baselines
  for (int kn : {0, 1})
    sweep("coda_baseline_gemm", {256, 256, 256}, [&](const std::vector<int>& a) {
      return coda_baseline_gemm(b, F<uint16_t>(2), a[0], a[1], a[2], kn, F<uint16_t>(3), nullptr);
    });
  sweep("coda_baseline_residual_rmsnorm", {256, 256}, [&](const std::vector<int>& a) {
    return coda_baseline_residual_rmsnorm(b, F<uint16_t>(2), F<uint16_t>(3), a[0], a[1], 1e-5f, F<uint16_t>(4),
                                          F<float>(5), F<uint16_t>(6), nullptr);
  });
  sweep("coda_baseline_rope", {256, 128, 128, 128, 128, 256, 0}, [&](const std::vector<int>& a) {
    return coda_baseline_rope(b, F<float>(2), F<float>(3), a[0], a[1], a[2], a[3], a[4], a[5], a[6],
                              F<uint16_t>(4), nullptr);
  });
  sweep("coda_baseline_swiglu", {256, 128}, [&](const std::vector<int>& a) {
    return coda_baseline_swiglu(b, a[0], a[1], F<uint16_t>(2), nullptr);
  });
  sweep("coda_baseline_rowdot", {256, 256}, [&](const std::vector<int>& a) {
    return coda_baseline_rowdot(b, F<uint16_t>(2), a[0], a[1], F<float>(3), nullptr);
  });
  for (int64_t bytes : {(int64_t)INT64_MIN, (int64_t)-16, (int64_t)0, (int64_t)15, (int64_t)16, (int64_t)1 << 40,
                        (int64_t)INT64_MAX})
    status_ok(coda_baseline_copy(fake(1), fake(2), bytes, nullptr), "coda_baseline_copy");
  sweep("coda_baseline_mfma_loop", {8, 4, 16}, [&](const std::vector<int>& a) {
    return coda_baseline_mfma_loop(b, a[0], a[1], a[2], F<float>(2), nullptr);
  });
  sweep("coda_baseline_schedule_probe", {0, 5, 1}, [&](const std::vector<int>& a) {
    return coda_baseline_schedule_probe(a[0], a[1], a[2], 0.125f, 7u, F<float>(1), F<long long>(2), nullptr);
  });
  // ------------------------------------------------------- split-depth forward
  sweep("coda_gemm_rmsnorm_fwd_ws", {256, 256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_rmsnorm_fwd_ws(b, F<uint16_t>(1), F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), a[0], a[1],
                                    a[2], a[3], 1e-5f, F<uint16_t>(5), F<uint16_t>(6), F<float>(7), F<float>(8),
                                    F<uint16_t>(9), fake(10), 1ll << 32, nullptr);
  });
  for (long long ws : {LLONG_MIN, -1ll, 0ll, 1ll << 40, LLONG_MAX})
    status_ok(coda_gemm_rmsnorm_fwd_ws(b, F<uint16_t>(1), F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), 256, 256,
                                       256, 256, 1e-5f, F<uint16_t>(5), F<uint16_t>(6), F<float>(7), F<float>(8),
                                       F<uint16_t>(9), fake(10), ws, nullptr),
              "coda_gemm_rmsnorm_fwd_ws workspace_bytes");
  EXPECT(coda_gemm_rmsnorm_fwd_ws(b, F<uint16_t>(1), F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), 256, 256, 256,
                                  256, 1e-5f, F<uint16_t>(5), F<uint16_t>(6), F<float>(7), F<float>(8),
                                  F<uint16_t>(9), fake(10), -1, nullptr) == CODA_ERR_ARG,
         "negative workspace_bytes");
  sweep("coda_gemm_rope_ws", {256, 256, 128, 128, 128, 128, 256, 0}, [&](const std::vector<int>& a) {
    return coda_gemm_rope_ws(b, F<uint16_t>(2), F<float>(3), F<float>(4), a[0], a[1], a[2], a[3], a[4], a[5], a[6],
                             a[7], F<uint16_t>(5), fake(6), 1ll << 32, nullptr);
  });
  sweep("coda_gemm_swiglu_ws", {256, 256, 128}, [&](const std::vector<int>& a) {
    return coda_gemm_swiglu_ws(b, F<uint16_t>(2), a[0], a[1], a[2], F<uint16_t>(3), fake(4), 1ll << 32, nullptr);
  });
  // ------------------------------------------ split-depth backward, cross-entropy
  sweep("coda_gemm_rope_bwd_ws", {256, 256, 128, 128, 128, 128, 256, 0}, [&](const std::vector<int>& a) {
    return coda_gemm_rope_bwd_ws(b, F<uint16_t>(2), F<float>(3), F<float>(4), a[0], a[1], a[2], a[3], a[4], a[5],
                                 a[6], a[7], F<uint16_t>(5), fake(6), 1ll << 32, nullptr);
  });
  sweep("coda_gemm_swiglu_bwd_ws", {256, 256, 128}, [&](const std::vector<int>& a) {
    return coda_gemm_swiglu_bwd_ws(b, F<uint16_t>(2), F<uint16_t>(3), a[0], a[1], a[2], F<uint16_t>(4), fake(5),
                                   1ll << 32, nullptr);
  });
  sweep("coda_gemm_rmsnorm_bwd_stats_ws", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_rmsnorm_bwd_stats_ws(b, F<uint16_t>(2), F<uint16_t>(3), a[0], a[1], a[2], F<uint16_t>(4),
                                          F<float>(5), F<float>(6), fake(7), 1ll << 32, nullptr);
  });
  sweep("coda_gemm_rmsnorm_bwd_dx_ws", {256, 256, 256}, [&](const std::vector<int>& a) {
    return coda_gemm_rmsnorm_bwd_dx_ws(b, F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), F<float>(5), F<float>(6),
                                       F<uint16_t>(7), a[0], a[1], a[2], F<uint16_t>(8), F<float>(9), fake(10),
                                       1ll << 32, nullptr);
  });
  sweep("coda_gemm_cross_entropy_ws", {256, 256, 512}, [&](const std::vector<int>& a) {
    return coda_gemm_cross_entropy_ws(b, F<uint16_t>(2), F<int32_t>(3), a[0], a[1], a[2], F<float>(4), F<float>(5),
                                      F<float>(6), F<float>(7), fake(8), 1ll << 32, nullptr);
  });
  for (long long ws : {LLONG_MIN, -1ll, 0ll, 1ll << 40, LLONG_MAX}) {
    status_ok(coda_gemm_swiglu_bwd_ws(b, F<uint16_t>(2), F<uint16_t>(3), 256, 256, 128, F<uint16_t>(4), fake(5), ws,
                                      nullptr),
              "coda_gemm_swiglu_bwd_ws workspace_bytes");
    status_ok(coda_gemm_cross_entropy_ws(b, F<uint16_t>(2), F<int32_t>(3), 256, 256, 512, F<float>(4), F<float>(5),
                                         F<float>(6), F<float>(7), fake(8), ws, nullptr),
              "coda_gemm_cross_entropy_ws workspace_bytes");
  }
  EXPECT(coda_gemm_rmsnorm_bwd_dx_ws(b, F<uint16_t>(2), F<uint16_t>(3), F<uint16_t>(4), F<float>(5), F<float>(6),
                                     F<uint16_t>(7), 256, 256, 256, F<uint16_t>(8), F<float>(9), fake(10), -1,
                                     nullptr) == CODA_ERR_ARG,
         "negative workspace_bytes (dx)");
  {
    long long bytes = 0;
    sweep("coda_split_workspace_bytes", {256, 256, 256}, [&](const std::vector<int>& a) {
      return coda_split_workspace_bytes(a[0], a[1], a[2], &bytes);
    });
  }
  {
    int sl = 0, st = 0, t0 = 0;
    long long bytes = 0;
    sweep("coda_split_plan", {256, 256, 256, 256}, [&](const std::vector<int>& a) {
      return coda_split_plan(a[0], a[1], a[2], a[3], &sl, &st, &t0, &bytes);
    });
    EXPECT(coda_split_plan(1 << 24, 1 << 22, 1 << 22, INT_MAX, &sl, &st, &t0, &bytes) == CODA_OK && sl == 1,
           "largest grid, most CUs");
    EXPECT(coda_split_plan(8, 8, 8, 256, nullptr, &st, &t0, &bytes) == CODA_ERR_NULL, "slices NULL");
    EXPECT(coda_split_plan(8, 8, 8, 0, &sl, &st, &t0, &bytes) == CODA_ERR_ARG, "no CUs");
  }
  {
    long long bytes = 0;
    sweep("coda_gemm_rmsnorm_fwd_workspace_bytes", {256, 256, 256, 256}, [&](const std::vector<int>& a) {
      return coda_gemm_rmsnorm_fwd_workspace_bytes(a[0], a[1], a[2], a[3], &bytes);
    });
    EXPECT(coda_gemm_rmsnorm_fwd_workspace_bytes(8, 8, 8, 8, nullptr) == CODA_ERR_NULL, "bytes NULL");
  }
  for (int st = -1; st <= 7; ++st) EXPECT(coda_status_string(st) != nullptr, "status string %d", st);
  printf("%ld calls, %d failures\n", calls, failures);
  return failures ? 1 : 0;
}
