// Epilogue of GEMM + cross-entropy: the logits z = x W never leave the chip. Each tile
// reduces its 256 columns per row to one log-sum-exp partial (the stateful online
// log-sum-exp of [notes] method overview and the five primitives), and the lane that
// holds a row's label column records that logit; an auxiliary kernel merges the tile
// partials, lse = log sum_t exp(lse_t), and forms loss = lse - z[label].
#pragma once

#include "coda_gemm.hpp"

namespace coda {

// Maximum over the 16 lanes of a DPP row (same exchange pattern as sum16).
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

struct EpiCrossEntropy {
  struct Args {
    const int32_t* labels;  // [M]; outside [0, V) marks an ignored row
    float* tile_lse;        // [M, nb] log-sum-exp of each 256-column tile
    float* target;          // [M] z[m, label[m]] (written by the tile that holds it)
    int nb;
  };
  struct Op {
    const EpiLane& L;
    const Args& a;
    int M, N, n;
    bool nok;
    WaveRowsF32 lab;  // labels, read as 32-bit words
    static constexpr bool kRowStat = true;
    static constexpr bool kColStat = false;
    typedef float2 Stat;  // (max over the wave's 64 columns, sum of exp(z - max) over them)
    typedef float Pre;    // the row's label bits
    __device__ __forceinline__ Pre fetch(int r) const { return lab.load(r); }
    __device__ __forceinline__ Stat row(int r, const f32x4_t& v, const Pre& lbits) const {
      const float ninf = -__builtin_huge_valf();
      const float z0 = nok ? v.x : ninf, z1 = nok ? v.y : ninf, z2 = nok ? v.z : ninf, z3 = nok ? v.w : ninf;
      const float mx = max16(fmaxf(fmaxf(z0, z1), fmaxf(z2, z3)));
      const float sh = mx == ninf ? 0.f : mx;  // a wave with no valid column contributes 0
      const float se = sum16((__expf(z0 - sh) + __expf(z1 - sh)) + (__expf(z2 - sh) + __expf(z3 - sh)));
      const int m = L.token(r);
      const int label = __builtin_bit_cast(int, lbits);
      if (nok && m < M && label >= n && label < n + 4) {
        const int e = label - n;
        a.target[m] = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
      }
      return make_float2(mx, se);
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    Op op{L, a, p.M, p.N, n, n < p.N, WaveRowsF32((const float*)a.labels, L, p.M)};
    epilogue_rows(acc, lds, L, op);
    __syncthreads();
    // merge the four feature-waves of each row in the order wn = 0, 1, 2, 3
    const int t = lds.tid;
    if (t < kBM) {
      const int wm = t >> 7, r = t & 127;
      const float2* st = (const float2*)lds.red + wm * kWavesN * 128 + r;
      float mx = st[0].x;
#pragma unroll
      for (int w = 1; w < kWavesN; ++w) mx = fmaxf(mx, st[w * 128].x);
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWavesN; ++w) {
        const float2 q = st[w * 128];
        s += q.y == 0.f ? 0.f : q.y * expf(q.x - mx);
      }
      const int m = m0 + t;
      if (m < p.M) a.tile_lse[(size_t)m * a.nb + n0 / kBN] = mx + logf(s);
    }
  }
};
static_assert(kWaves * 128 * 8 <= kSlotBytes, "per-wave row states fit in the last slot");

}  // namespace coda
