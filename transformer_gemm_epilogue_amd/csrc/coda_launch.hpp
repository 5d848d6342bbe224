// Host-side launch of the GEMM kernels shared by the entry points of every source file:
// the one-kernel schedule (one workgroup per output tile), and the split-depth schedule
// of coda_splitk.hpp with the checks of its caller-owned workspace.
#pragma once

#include <initializer_list>

#include "coda_abi.hpp"
#include "coda_gemm.hpp"
#include "coda_splitk.hpp"

namespace coda {

// The one-kernel schedule over tiles [0, tiles) of the tile order (all of them by default).
template <bool kWKN, class Epi>
int launch_gemm(const GemmProblem& p, const typename Epi::Args& ea, hipStream_t stream, int tiles = -1) {
  const int grid = tiles < 0 ? gemm_grid(p.M, p.N) : tiles;
  if constexpr (kWKN) {
    if (kn_one_descriptor_fits(p.K, p.N)) {
      hipLaunchKernelGGL((gemm_epilogue_kernel<true, Epi, true>), dim3(grid), dim3(kThreads), 0, stream, p, ea);
      return launch_status();
    }
  }
  hipLaunchKernelGGL((gemm_epilogue_kernel<kWKN, Epi>), dim3(grid), dim3(kThreads), 0, stream, p, ea);
  return launch_status();
}

// Compute units of the current device.
inline int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || *cus < 1)
    return CODA_ERR_HIP;
  return CODA_OK;
}

// Split-depth schedule (coda_splitk.hpp) when the plan has more than one slice: the
// one-kernel schedule over the tiles before sp.tile0 (if any), then the split tiles'
// slices, then their epilogues on the summed partials; otherwise the one-kernel schedule.
// ws holds split_workspace_floats(M, N, sp) floats.
template <bool kWKN, class Epi>
int launch_gemm_split(const GemmProblem& p, const typename Epi::Args& ea, const SplitPlan& sp, float* ws,
                      hipStream_t stream) {
  if (sp.S <= 1) return launch_gemm<kWKN, Epi>(p, ea, stream);
  if (sp.tile0 > 0) CODA_TRY((launch_gemm<kWKN, Epi>(p, ea, stream, sp.tile0)));
  const int Tq = gemm_grid(p.M, p.N) - sp.tile0;
  const dim3 units((unsigned)(((Tq + 7) / 8) * 8 * sp.S));
  f32x4_t* w4 = reinterpret_cast<f32x4_t*>(ws);
  if (kWKN && kn_one_descriptor_fits(p.K, p.N))
    hipLaunchKernelGGL((gemm_split_kernel<kWKN, kWKN>), units, dim3(kThreads), 0, stream, p, sp.S, sp.steps, sp.tile0,
                       w4);
  else
    hipLaunchKernelGGL((gemm_split_kernel<kWKN, false>), units, dim3(kThreads), 0, stream, p, sp.S, sp.steps,
                       sp.tile0, w4);
  CODA_TRY(launch_status());
  hipLaunchKernelGGL((split_epilogue_kernel<Epi>), dim3(Tq), dim3(kThreads), 0, stream, p, ea, sp.S, sp.tile0,
                     (const f32x4_t*)w4);
  return launch_status();
}

// The split plan of one GEMM on the current device and its workspace checks: enough bytes,
// 16-byte aligned, overlapping none of the call's other buffers (`others`).
inline int split_for_call(int M, int N, int K, void* workspace, long long workspace_bytes,
                          std::initializer_list<Span> others, SplitPlan* sp) {
  if (workspace_bytes < 0) return CODA_ERR_ARG;
  int cus = 0;
  CODA_TRY(device_cus(&cus));
  *sp = split_plan(M, N, K, cus);
  const long long need = 4 * split_workspace_floats(M, N, *sp);
  if (need == 0) return CODA_OK;
  CODA_NONNULL(workspace);
  CODA_ALIGN16(workspace);
  if (workspace_bytes < need) return CODA_ERR_WORKSPACE;
  return check_disjoint({Span{workspace, (uint64_t)need}}, others);
}

}  // namespace coda
