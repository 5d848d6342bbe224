// Epilogue of GEMM + cross-entropy: the logits z = x W never leave the chip. Each tile
// reduces its 256 columns per row to one log-sum-exp partial (the stateful online
// log-sum-exp of [notes] method overview and the five primitives), and the lane that
// holds a row's label column records that logit; an auxiliary kernel merges the tile
// partials, lse = log sum_t exp(lse_t), and forms loss = lse - z[label].
#pragma once

#include "coda_gemm.hpp"

namespace coda {

// The epilogue works in the accumulator layout itself, with no row-major relayout: it has
// no per-element side input and writes no tile, and a lane already holds 16 of a row's 64
// wave-features (acc[i][j][v] is feature 16 i + 4 (lane >> 4) + v of token
// 16 j + (lane & 15)); the lanes 16, 32 and 48 away hold the other 48. So each row's
// maximum and sum of exponentials reduce within the lane, then across those four lanes.
struct EpiCrossEntropy {
  struct Args {
    const int32_t* labels;  // [M]; outside [0, V) marks an ignored row
    float* tile_lse;        // [M, nb] log-sum-exp of each 256-column tile
    float* target;          // [M] z[m, label[m]] (written by the tile that holds it)
    int nb;
  };
  // Per 16-token block j: the row's maximum and sum of exp(z - max) over this wave's 64
  // columns (kFull: all of them inside the width, no column masks), recorded per
  // (wave, row); the lane holding the label's column writes the target logit. The
  // exponential is exp2 of one fused multiply-add; the label search runs only for the
  // blocks where some lane of the wave can hold a label column (64 of V columns).
  template <bool kFull>
  __device__ __forceinline__ static void rows(AccTile& acc, const Args& a, const GemmProblem& p, const EpiLane& L,
                                              int nbase, const int (&label)[kMJ], float2* red) {
    const float ninf = -__builtin_huge_valf();
    const float l2e = 1.4426950408889634f;
    const int r16 = L.lane & 15;
    // columns 16 i .. 16 i + 3 of this lane are inside the width (N % 8 == 0)
    bool ok[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) ok[i] = kFull || nbase + 16 * i < p.N;
#pragma unroll
    for (int j = 0; j < kMJ; ++j) {
      float mx = ninf;
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = ok[i] ? fmaxf(mx, acc[i][j][v]) : mx;
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float shl = (mx == ninf ? 0.f : mx) * l2e;  // a wave with no valid column contributes 0
      float se = 0.f;
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) se += ok[i] ? __builtin_amdgcn_exp2f(fmaf(acc[i][j][v], l2e, -shl)) : 0.f;
      se += __shfl_xor(se, 16);
      se += __shfl_xor(se, 32);
      const int m = L.token(16 * j + r16);
      const int rel = label[j] - nbase;  // this lane's column offset of the label
      const bool maybe = (unsigned)rel < (unsigned)(4 * 16) && (rel & 12) == 0;
      if (__builtin_amdgcn_ballot_w64(maybe) != 0) {  // wave-uniform
        float tv = 0.f;
        bool hit = false;
#pragma unroll
        for (int i = 0; i < kNI; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const bool here = ok[i] && rel == 16 * i + v;
            tv = here ? acc[i][j][v] : tv;
            hit = hit || here;
          }
        if (hit && m < p.M) a.target[m] = tv;
      }
      if (L.lane < 16) red[16 * j + r16] = make_float2(mx, se);
    }
  }
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int r16 = L.lane & 15;
    const int nbase = n0 + L.wn * kWaveN + 4 * (L.lane >> 4);  // feature of acc[0][j][0]
    const WaveRowsF32 lab((const float*)a.labels, L, p.M);
    int label[kMJ];
#pragma unroll
    for (int j = 0; j < kMJ; ++j) label[j] = __builtin_bit_cast(int, lab.load(16 * j + r16));
    float2* red = (float2*)lds.red + (L.wm * kWavesN + L.wn) * 128;
    if (n0 + kBN <= p.N)  // wave-uniform: the whole tile lies inside the width
      rows<true>(acc, a, p, L, nbase, label, red);
    else
      rows<false>(acc, a, p, L, nbase, label, red);
    __syncthreads();
    // merge the four feature-waves of each row in the order wn = 0, 1, 2, 3
    const int t = lds.tid;
    if (t < kBM) {
      const int wm = t >> 7, r = t & 127;
      const float2* st = (const float2*)lds.red + wm * kWavesN * 128 + r;
      float mxa = st[0].x;
#pragma unroll
      for (int w = 1; w < kWavesN; ++w) mxa = fmaxf(mxa, st[w * 128].x);
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWavesN; ++w) {
        const float2 q = st[w * 128];
        s += q.y == 0.f ? 0.f : q.y * expf(q.x - mxa);
      }
      const int m = m0 + t;
      if (m < p.M) a.tile_lse[(size_t)m * a.nb + n0 / kBN] = mxa + logf(s);
    }
  }
};
static_assert(kWaves * 128 * 8 <= kSlotBytes, "per-wave row states fit in the last slot");

}  // namespace coda
