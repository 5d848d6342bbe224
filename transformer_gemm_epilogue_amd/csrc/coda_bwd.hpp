// Epilogue of the RMSNorm-backward grad GEMM: the rest of the RMSNorm backward runs on
// the accumulator dO = dY W1^T while its tile is on chip ([notes] key design 3 and the
// duality paragraph before its statistic; [pith] Fig. 9).
//
// With the forward o = r h1 gamma (r = 1/rms(h1), the GEMM2 input) and the row
// statistic s = (1/d) sum_cols(dO * o), which key design 3 also obtains from the output
// side before this GEMM, the input gradient of RMSNorm is
//   dh1 = r gamma dO - r^2 s h1   (+ g_res, the gradient reaching h1 through the
//                                   residual stream),
// stored in place of dO, and the gamma gradient dgamma = sum_rows(dO r h1) leaves the
// tile as one fp32 column partial per (256-row tile, feature): the cross-row sibling of
// the forward's row partials, finished by a column reduction.
#pragma once

#include "coda_gemm.hpp"

namespace coda {

struct EpiRmsNormBwd {
  struct Args {
    const uint16_t* h1;     // [M, N] (N = this GEMM's output width, the hidden size D)
    const uint16_t* gamma;  // [N]
    const float* r;         // [M]
    const float* s;         // [M]
    const uint16_t* g_res;  // [M, N] or null
    uint16_t* dh1;          // [M, N]
    float* pgamma;          // [ceil(M / 256), N]
  };
  struct Op {
    const EpiLane& L;
    const Args& a;
    const float2* tab;  // LDS: (r, r^2 s) per row of the tile
    int M, N, n;
    bool nok;
    float g0, g1, g2, g3;
    WaveRowsBf16 hv, gv;  // h1 and g_res (a null g_res reads as zero)
    static constexpr bool kRowStat = false;
    static constexpr bool kColStat = true;  // column sums of dO r h1 (dgamma partials)
    struct Pre {
      u32x2_t h, g;
    };
    __device__ __forceinline__ Pre fetch(int r) const {
      Pre t;
      t.h = hv.load4(r);
      t.g = gv.load4(r);
      return t;
    }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre& t, f32x4_t& col) const {
      const int m = L.token(r);
      const float2 rb = tab[L.wm * 128 + r];
      const float h0 = bf16_lo(t.h.x), h1 = bf16_hi(t.h.x), h2 = bf16_lo(t.h.y), h3 = bf16_hi(t.h.y);
      const float d0 = (rb.x * g0 * v.x - rb.y * h0) + bf16_lo(t.g.x);
      const float d1 = (rb.x * g1 * v.y - rb.y * h1) + bf16_hi(t.g.x);
      const float d2 = (rb.x * g2 * v.z - rb.y * h2) + bf16_lo(t.g.y);
      const float d3 = (rb.x * g3 * v.w - rb.y * h3) + bf16_hi(t.g.y);
      // Rows past M and features past N contribute nothing (their h1 reads as zero); all
      // of the row's work stays under the one branch, which keeps the compiler from
      // carrying every row's products to the end of the walk.
      if (nok && m < M) {
        store_bf16x4(a.dh1, (size_t)m * N + n, d0, d1, d2, d3);
        col.x += v.x * (rb.x * h0);
        col.y += v.y * (rb.x * h1);
        col.z += v.z * (rb.x * h2);
        col.w += v.w * (rb.x * h3);
      }
      return 0.f;
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int M = p.M, N = p.N;
    float2* tab = (float2*)(lds.red + kRedFloats);   // 2 KiB after the row-partial area
    float* colred = lds.red + kRedFloats + 2 * kBM;  // [2][256] column sums of the two token-waves
    const int t = lds.tid;
    if (t < kBM) {
      const int m = m0 + t;
      const float rr = m < M ? a.r[m] : 0.f;
      const float ss = m < M ? a.s[m] : 0.f;
      tab[t] = make_float2(rr, rr * rr * ss);
    }
    __syncthreads();
    const int n = L.col4();
    const bool nok = n < N;
    const u32x2_t gg = load_bf16x4(a.gamma, (size_t)n, nok);
    Op op{L, a, tab, M, N, n, nok, bf16_lo(gg.x), bf16_hi(gg.x), bf16_lo(gg.y), bf16_hi(gg.y),
          WaveRowsBf16(a.h1, L, M, N, n, nok), WaveRowsBf16(a.g_res, L, M, N, n, nok)};
    const f32x4_t cs = epilogue_rows(acc, lds, L, op);
    // Lanes l, l^16, l^32, l^48 hold the same 4 features over different rows.
    float c[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] += __shfl_xor(c[e], 16);
      c[e] += __shfl_xor(c[e], 32);
    }
    if (L.lane < 16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) colred[L.wm * kBN + L.wn * kWaveN + 4 * L.lane + e] = c[e];
    }
    __syncthreads();
    if (t < kBN && n0 + t < N) a.pgamma[(size_t)(m0 / kBM) * N + n0 + t] = colred[t] + colred[kBN + t];
  }
};
static_assert(kRedFloats * 4 + kBM * 8 + 2 * kBN * 4 <= kSlotBytes, "row tables fit in the last slot");

// ------------------------------------------------------------------------------------
// SwiGLU backward ([notes] key design 2, last item; [pith] Fig. 7): the grad GEMM of the
// down projection gives dOut = dY W_down^T, one gradient per SwiGLU output; the epilogue
// maps each into the gradients of its (gate, up) pair from the saved interleaved
// pre-activations h = [G_0, U_0, G_1, U_1, ...]:
//   dG = dOut U silu'(G),  dU = dOut silu(G),  silu'(g) = s (1 + g (1 - s)), s = 1/(1+e^-g)
// and stores them interleaved like h. A lane's 4 outputs j .. j+3 use and produce the 8
// interleaved columns 2j .. 2j+7: one 16-byte load of h and one 16-byte store of dh.
struct EpiSwiGLUBwd {
  struct Args {
    const uint16_t* h;  // [M, 2F] saved pre-activations (F = this GEMM's output width)
    uint16_t* dh;       // [M, 2F]
  };
  __device__ __forceinline__ static uint32_t pair_grad(float d, uint32_t gu) {
    const float g = bf16_lo(gu), u = bf16_hi(gu);
    const float sg = sigmoid_f32(g);
    return pack_bf16x2(d * u * (sg * (1.0f + g * (1.0f - sg))), d * (g * sg));
  }
  struct Op {
    WaveRowsBf16 hv;       // [M, 2F] saved (G, U) pairs of this lane's 4 columns
    WaveRowsOutBf16 dho;   // [M, 2F] their gradients, same positions
    static constexpr bool kRowStat = false;
    static constexpr bool kColStat = false;
    typedef u32x4_t Pre;
    __device__ __forceinline__ Pre fetch(int r) const { return hv.load8(r); }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre& t) const {
      u32x4_t o;
      o.x = pair_grad(v.x, t.x);
      o.y = pair_grad(v.y, t.y);
      o.z = pair_grad(v.z, t.z);
      o.w = pair_grad(v.w, t.w);
      dho.store8_at(dho.row_off(r), o);
      return 0.f;
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    const bool nok = n < p.N;
    Op op{WaveRowsBf16(a.h, L, p.M, 2 * p.N, 2 * n, nok), WaveRowsOutBf16(a.dh, L, p.M, 2 * p.N, 2 * n, nok)};
    epilogue_rows(acc, lds, L, op);
  }
};

}  // namespace coda
