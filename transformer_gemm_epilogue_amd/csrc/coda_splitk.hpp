// Split-depth schedule for outputs with fewer 256 x 256 tiles than the GPU has CUs (a
// small batch, or one GPU's share of token-sharded rows): with one workgroup per tile
// most CUs would idle. Each tile's depth steps are cut into S slices of equal, even
// length; a workgroup runs the same main loop over one slice and stores its fp32
// accumulator tile to a workspace; a second kernel then sums a tile's S partial tiles in
// the fixed order s = 0, 1, ..., S-1 and runs the tile's epilogue program on the sum, as
// the one-kernel schedule runs it on its accumulator. The result is deterministic (it
// depends only on the shape and S), though its fp32 rounding differs from the one-kernel
// schedule's, whose depth order is rotated per tile.
#pragma once

#include <algorithm>

#include "coda_gemm.hpp"

namespace coda {

constexpr int kSplitMinSteps = 16;  // depth steps per slice at least (the ring's fill costs ~3)
constexpr int kSplitMax = 8;        // slices per tile at most
// Slices of a partial last wave split beside the full waves of the one-kernel schedule
// (which run anyway) are at least this deep: splitting saves (S - 1) / S of the partial
// wave's depth walk and costs the partial tiles' traffic and a second launch.
constexpr int kRemainderMinSteps = 32;
constexpr long long kSplitTileFloats = (long long)kNI * kMJ * kThreads * 4;  // one fp32 tile: 256 KiB

struct SplitPlan {
  int S;          // slices per split tile (1: the one-kernel schedule for every tile)
  int steps;      // depth steps per slice (the last one may be shorter)
  int tile0 = 0;  // tiles [0, tile0) run the one-kernel schedule, [tile0, T) are split
};

// The split of T' tiles of KT depth steps: as many slices as fit one workgroup per CU
// (T' S <= CUs: a second, partial wave of workgroups would cost a whole slice's time for
// a few of them), at most kSplitMax and with at least min_steps steps each; slices are an
// even number of steps (paired X loads share 128-byte lines), and S is recomputed so
// that none is empty.
__host__ inline SplitPlan split_slices(int Tp, int KT, int cus, int min_steps, int tile0) {
  int S = std::min(cus / Tp, std::min(kSplitMax, KT / min_steps));
  if (S <= 1) return SplitPlan{1, KT, 0};
  int steps = (KT + S - 1) / S;
  steps += steps & 1;
  S = (KT + steps - 1) / steps;
  if (S <= 1) return SplitPlan{1, KT, 0};
  return SplitPlan{S, steps, tile0};
}

// Outputs with at most half as many tiles as CUs split every tile. Larger ones whose last
// wave of workgroups is at most half full run their full waves in the one-kernel schedule
// and split the tiles of the partial wave (the last in the tile order), which would
// otherwise leave at least half of the CUs idle for a whole tile.
__host__ inline SplitPlan split_plan(int M, int N, int K, int cus) {
  const int T = gemm_grid(M, N), KT = (K + kBK - 1) / kBK;
  if (T <= cus / 2) return split_slices(T, KT, cus, kSplitMinSteps, 0);  // 2T <= cus, without overflow
  const int r = T % cus;
  if (r > 0 && r <= cus / 2) return split_slices(r, KT, cus, kRemainderMinSteps, T - r);
  return SplitPlan{1, KT, 0};
}

// fp32 workspace of a plan, in floats: S partial tiles per split tile.
__host__ inline long long split_workspace_floats(int M, int N, const SplitPlan& sp) {
  return sp.S > 1 ? (long long)(gemm_grid(M, N) - sp.tile0) * sp.S * kSplitTileFloats : 0;
}

// Workgroup u -> (tile t, slice s). Workgroups go round-robin to the 8 XCDs, so the S
// slices of a tile are placed on the same XCD (u mod 8 = t mod 8), where their partial
// tiles meet in one L2; ceil(T / 8) * 8 * S workgroups, those past the last tile idle.
__device__ __forceinline__ void split_unit(int u, int S, int& t, int& s) {
  const int g = u / (8 * S), r = u - g * 8 * S;
  s = r / 8;
  t = g * 8 + (r - s * 8);
}

// Partial tile layout: [split tile][slice][accumulator block i * kMJ + j][thread] of
// f32x4, so that every store and load instruction of a wave covers 1 KiB of consecutive
// bytes. Split tile q is output tile tile0 + q.
template <bool kWKN, bool kWOneDesc>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_split_kernel(GemmProblem p, int S, int slice_steps, int tile0, f32x4_t* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kSlotBytes];
  int q, s;
  split_unit(blockIdx.x, S, q, s);
  if (q >= gemm_grid(p.M, p.N) - tile0) return;  // workgroup-uniform
  const int t = tile0 + q;
  const LdsRing lds = make_ring(smem, 0, 0, threadIdx.x);
  int m0, n0;
  tile_coords(p.M, p.N, p.K, p.group_m, t, m0, n0);
  Mainloop<kWKN, kWOneDesc> ml;
  ml.init(p, threadIdx.x);
  TileSrc src = ml.src(t, m0, n0);
  src.kstart = s * slice_steps;  // no per-XCD rotation: the slice starts the walk
  const int steps = min(slice_steps, ml.KT - src.kstart);
  AccTile acc;
  mainloop_prologue(ml, src, lds);
  mainloop_body<false>(ml, src, src, false, lds, acc, steps);
  f32x4_t* out = ws + ((size_t)q * S + s) * (size_t)(kNI * kMJ * kThreads) + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j) out[(size_t)(i * kMJ + j) * kThreads] = acc[i][j];
}

// One workgroup per split tile (output tile tile0 + blockIdx.x): the sum of its S partial
// tiles, in slice order, then the tile's epilogue program, exactly as the one-kernel
// schedule calls it.
template <class Epi>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void split_epilogue_kernel(GemmProblem p, typename Epi::Args ea, int S, int tile0, const f32x4_t* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kSlotBytes];
  const int q = blockIdx.x, t = tile0 + q;
  int m0, n0;
  tile_coords(p.M, p.N, p.K, p.group_m, t, m0, n0);
  const LdsRing lds = make_ring(smem, 0, 0, threadIdx.x);
  const f32x4_t* in = ws + (size_t)q * S * (size_t)(kNI * kMJ * kThreads) + threadIdx.x;
  AccTile acc;
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j) acc[i][j] = in[(size_t)(i * kMJ + j) * kThreads];
  for (int s = 1; s < S; ++s) {
    in += (size_t)(kNI * kMJ * kThreads);
    // two feature blocks (16 loads, 64 registers) in flight at a time: the whole next
    // partial tile (128 values) would not fit beside the accumulators in the register
    // budget, and fewer loads in flight leave the sum bound by their latency
    constexpr int kB = 2;
#pragma unroll
    for (int i0 = 0; i0 < kNI; i0 += kB) {
      f32x4_t v[kB][kMJ];
#pragma unroll
      for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int j = 0; j < kMJ; ++j) v[b][j] = in[(size_t)((i0 + b) * kMJ + j) * kThreads];
#pragma unroll
      for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int j = 0; j < kMJ; ++j) acc[i0 + b][j] += v[b][j];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  Epi::apply(acc, ea, p, m0, n0, lds);
}

}  // namespace coda
