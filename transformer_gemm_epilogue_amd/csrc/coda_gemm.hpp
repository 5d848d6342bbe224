// One bf16 MFMA GEMM main loop for gfx950 and the epilogue programs that run on its
// accumulator tile before anything is written to HBM.
//
// Product: C[m, n] = sum_k X[m, k] * W(k, n), X = tokens x depth (row-major, depth
// contiguous), W either [K, N] row-major ("KN", features contiguous: the forward
// projections) or [N, K] row-major ("NK", depth contiguous: the grad GEMM dY W1^T).
//
// Workgroup tile: 256 tokens x 256 features x 64 depth per step, 256 threads = 4 waves
// in a 2 x 2 arrangement, each wave owning 128 tokens x 128 features = 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (16 fp32 accumulators per lane per block).
//
// Transposed MFMA formulation. The MFMA "A" operand (rows of the MFMA output) is the
// W slice, so MFMA rows are FEATURES; the "B" operand is the X slice, so MFMA columns
// are TOKENS. With the 32x32 output layout (lane l, register v holds row
// 8*(v/4) + 4*(l/32) + v%4, column l%32), every lane holds, for one token, runs of 4
// consecutive features: the (even, odd) feature pairs of RoPE and SwiGLU sit in one
// lane's registers, and a row statistic is an in-lane sum plus one exchange between
// the two 32-lane halves.
//
// LDS: two stages of [X tile 256x64 | W tile 256x64] bf16 (depth contiguous, 128 B per
// row, 16-byte chunks XOR-swizzled per row), 128 KiB. X and NK-W tiles are copied
// chunk for chunk; a KN-W tile is transposed in registers (8x8 bf16 blocks with
// v_perm_b32) on its way to LDS so both operands are depth-contiguous for the MFMA.
// Global loads use raw buffer descriptors: rows past M, depth past K and columns past
// N read as zero, so ragged edges need no special path.
#pragma once

#include "coda_common.hpp"

namespace coda {

constexpr int kBM = 256;       // tokens per workgroup tile
constexpr int kBN = 256;       // features per workgroup tile (== CODA_PARTIAL_TILE_N)
constexpr int kBK = 64;        // depth per main-loop step
constexpr int kThreads = 256;  // 4 waves
constexpr int kTileBytes = kBM * kBK * 2;    // one operand tile: 32 KiB
constexpr int kStageBytes = 2 * kTileBytes;  // X tile + W tile
constexpr int kStgPitch = 132;               // epilogue staging row pitch, bf16 elements
constexpr int kStgWaveBytes = 128 * kStgPitch * 2;
constexpr int kRedOff = 4 * kStgWaveBytes;   // row-partial exchange area
constexpr int kLdsBytes = kRedOff + 4 * 128 * 4;
static_assert(kLdsBytes >= 2 * kStageBytes, "LDS must hold both main-loop stages");
static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");

struct GemmProblem {
  const uint16_t* x;  // [M, K]
  const uint16_t* w;  // [K, N] (KN) or [N, K] (NK)
  int M, N, K;
};

// Row swizzle of the 16-byte chunks of a 128-byte LDS row. Consecutive rows (MFMA
// operand reads) and rows 8 apart (transposed W writes) land on distinct banks.
__device__ __forceinline__ uint32_t swz(int row) {
  return (uint32_t)(((row >> 1) & 7) ^ ((row & 1) << 2) ^ ((row >> 3) & 7));
}
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return ((uint32_t)row << 7) | (((uint32_t)chunk ^ swz(row)) << 4);
}

// Workgroup -> output tile. Workgroups are dispatched round-robin over the 8 XCDs, so
// block b runs on XCD b % 8; giving each XCD a contiguous run of tiles, walked in
// groups of 8 token-tiles, keeps the X and W panels a wave of tiles shares in that
// XCD's L2.
__device__ __forceinline__ void tile_coords(int M, int N, int& m0, int& n0) {
  const int mt = (M + kBM - 1) / kBM;
  const int nt = (N + kBN - 1) / kBN;
  const int T = mt * nt;
  const int b = blockIdx.x;
  const int t = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  constexpr int GM = 8;
  const int group = t / (GM * nt);
  const int first_m = group * GM;
  const int gm = min(mt - first_m, GM);
  const int rem = t - group * GM * nt;
  m0 = (first_m + rem % gm) * kBM;
  n0 = (rem / gm) * kBN;
}

template <bool kWKN>
__device__ __forceinline__ void gemm_mainloop(const GemmProblem& p, int m0, int n0,
                                              char* __restrict__ smem, f32x16_t (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, N = p.N, K = p.K;

  // X tile loads: thread -> rows (tid >> 3) + 32 i, 16-byte chunk (tid & 7).
  const int lr = tid >> 3, lc = tid & 7;
  const int x_rows = min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(p.x + (size_t)m0 * K, (uint32_t)x_rows * (uint32_t)K * 2u);
  const uint32_t rstride = (uint32_t)K * 2u;
  const uint32_t x_off0 = (uint32_t)lr * rstride + (uint32_t)lc * 16u;

  // NK-W tile loads: same pattern as X over feature rows.
  const __amdgpu_buffer_rsrc_t wrs_nk =
      kWKN ? make_rsrc(p.w, 0u)
           : make_rsrc(p.w + (size_t)n0 * K, (uint32_t)min(kBN, N - n0) * (uint32_t)K * 2u);
  // KN-W tile loads: thread -> depth rows 8*(tid>>5) + i, features 8*(tid&31) .. +7.
  const int kb = tid >> 5, nb8 = tid & 31;
  const bool kn_col_ok = n0 + 8 * nb8 < N;
  const uint32_t kn_off0 = ((uint32_t)(8 * kb) * (uint32_t)N + (uint32_t)(8 * nb8)) * 2u;
  const uint32_t kn_rstride = (uint32_t)N * 2u;

  u32x4_t xr[8], wr[8];

  auto load = [&](int k0) {
    const uint32_t koff = (uint32_t)k0 * 2u;
    const bool kx_ok = k0 + lc * 8 < K;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xr[i] = buffer_load_16(xrs, kx_ok ? x_off0 + (uint32_t)i * 32u * rstride + koff : kOutOfRange);
    if constexpr (kWKN) {
      const int krows = min(kBK, K - k0);
      const __amdgpu_buffer_rsrc_t wrs =
          make_rsrc(p.w + (size_t)k0 * N + n0, ((uint32_t)krows * (uint32_t)N - (uint32_t)n0) * 2u);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wr[i] = buffer_load_16(wrs, kn_col_ok ? kn_off0 + (uint32_t)i * kn_rstride : kOutOfRange);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wr[i] = buffer_load_16(wrs_nk, kx_ok ? x_off0 + (uint32_t)i * 32u * rstride + koff : kOutOfRange);
    }
  };

  auto store = [&](char* stage) {
    char* xs = stage;
    char* ws = stage + kTileBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)(xs + tile_off(lr + 32 * i, lc)) = xr[i];
    if constexpr (kWKN) {
      // 8x8 bf16 transpose: wr[i] holds depth 8kb+i for features 8nb8..8nb8+7; write
      // feature row 8nb8+j, chunk kb = depth 8kb..8kb+7 in order.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t o;
        o.x = __builtin_amdgcn_perm(wr[1][d], wr[0][d], sel);
        o.y = __builtin_amdgcn_perm(wr[3][d], wr[2][d], sel);
        o.z = __builtin_amdgcn_perm(wr[5][d], wr[4][d], sel);
        o.w = __builtin_amdgcn_perm(wr[7][d], wr[6][d], sel);
        *(u32x4_t*)(ws + tile_off(8 * nb8 + j, kb)) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) *(u32x4_t*)(ws + tile_off(lr + 32 * i, lc)) = wr[i];
    }
  };

  const int r32 = lane & 31, hsel = lane >> 5;
  auto compute = [&](const char* stage) {
    const char* xs = stage;
    const char* ws = stage + kTileBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *(const bf16x8_t*)(ws + tile_off(wn * 128 + i * 32 + r32, 2 * ks + hsel));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        b[i] = *(const bf16x8_t*)(xs + tile_off(wm * 128 + i * 32 + r32, 2 * ks + hsel));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = (K + kBK - 1) / kBK;
  load(0);
  store(smem);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) load((kt + 1) * kBK);
    compute(smem + (kt & 1) * kStageBytes);
    if (more) store(smem + ((kt + 1) & 1) * kStageBytes);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// Epilogue helpers. Accumulator block acc[i][j] of a lane covers features
//   n = n0 + wn*128 + 32 i + 8 g + 4 (lane >> 5) + e,  (register v = 4 g + e)
// for the token m = m0 + wm*128 + 32 j + (lane & 31).
struct EpiLane {
  int lane, wave, wm, wn, m0, n0;
  __device__ __forceinline__ EpiLane(int m0_, int n0_)
      : lane(threadIdx.x & 63), wave(threadIdx.x >> 6), wm((threadIdx.x >> 6) >> 1),
        wn((threadIdx.x >> 6) & 1), m0(m0_), n0(n0_) {}
  __device__ __forceinline__ int row(int j) const { return m0 + wm * 128 + 32 * j + (lane & 31); }
  __device__ __forceinline__ int col(int i, int g) const {
    return n0 + wn * 128 + 32 * i + 8 * g + 4 * (lane >> 5);
  }
  // wave-local staging coordinates
  __device__ __forceinline__ int srow(int j) const { return 32 * j + (lane & 31); }
  __device__ __forceinline__ int scol(int i, int g) const { return 32 * i + 8 * g + 4 * (lane >> 5); }
};

__device__ __forceinline__ char* stage_base(char* smem, int wave) { return smem + wave * kStgWaveBytes; }

__device__ __forceinline__ void stage_put8(char* stg, int r, int c, uint32_t lo, uint32_t hi) {
  u32x2_t v;
  v.x = lo;
  v.y = hi;
  *(u32x2_t*)(stg + (r * kStgPitch + c) * 2) = v;
}
__device__ __forceinline__ void stage_put4(char* stg, int r, int c, uint32_t w) {
  *(uint32_t*)(stg + (r * kStgPitch + c) * 2) = w;
}

// Write a wave's staged [128 rows x ncols] bf16 block (ncols = 128 or 64) to
// out[row0 + r, col0 + c] (row pitch ldo elements) with 16-byte row-contiguous stores.
template <int kCols>
__device__ __forceinline__ void stage_flush(const char* stg, uint16_t* __restrict__ out, size_t ldo,
                                            int M, int ncols_total, int row0, int col0, int lane) {
  constexpr int kLanesPerRow = kCols / 8;
  constexpr int kRowsPerIter = 64 / kLanesPerRow;
  const int cseg = (lane % kLanesPerRow) * 8;
  const int n = col0 + cseg;
#pragma unroll 4
  for (int it = 0; it < 128 / kRowsPerIter; ++it) {
    const int r = it * kRowsPerIter + lane / kLanesPerRow;
    const int m = row0 + r;
    const u32x2_t lo = *(const u32x2_t*)(stg + (r * kStgPitch + cseg) * 2);
    const u32x2_t hi = *(const u32x2_t*)(stg + (r * kStgPitch + cseg + 4) * 2);
    if (m < M && n < ncols_total) {
      u32x4_t v;
      v.x = lo.x;
      v.y = lo.y;
      v.z = hi.x;
      v.w = hi.y;
      *(u32x4_t*)(out + (size_t)m * ldo + n) = v;
    }
  }
}

// Combine per-lane row partials into one fp32 value per (token, 256-column tile) and
// store it at partials[m * nb + tile]. Order is fixed: in-lane sum, the two 32-lane
// halves, then wave wn = 0 plus wave wn = 1.
__device__ __forceinline__ void store_row_partials(float (&part)[4], char* smem, const EpiLane& L,
                                                   float* __restrict__ partials, int nb, int M) {
#pragma unroll
  for (int j = 0; j < 4; ++j) part[j] += __shfl_xor(part[j], 32);
  float* red = (float*)(smem + kRedOff);
  if (L.lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(L.wm * 2 + L.wn) * 128 + 32 * j + L.lane] = part[j];
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int wm = t >> 7, r = t & 127;
  const int m = L.m0 + t;
  if (m < M) partials[(size_t)m * nb + L.n0 / kBN] = red[(wm * 2) * 128 + r] + red[(wm * 2 + 1) * 128 + r];
}

__device__ __forceinline__ u32x2_t load_bf16x4(const uint16_t* __restrict__ base, size_t idx, bool ok) {
  u32x2_t v;
  v.x = 0u;
  v.y = 0u;
  if (ok) v = *(const u32x2_t*)(base + idx);
  return v;
}

// ---------------------------------------------------------------- plain store (baseline)
struct EpiStore {
  struct Args {
    uint16_t* out;
  };
  __device__ __forceinline__ static void apply(f32x16_t (&acc)[4][4], const Args& a, const GemmProblem& p,
                                               int m0, int n0, char* smem) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(smem, L.wave);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                     pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
    __syncthreads();
    stage_flush<128>(stg, a.out, (size_t)p.N, p.M, p.N, m0 + L.wm * 128, n0 + L.wn * 128, L.lane);
  }
};

// ------------------------------------- GEMM1: residual + gamma side output + partials
// h1 = acc + z (stored), h2 = h1 * gamma (stored), P[m, tile] = sum h1^2 over the tile.
struct EpiResidualRmsPartials {
  struct Args {
    const uint16_t* z;
    const uint16_t* gamma;
    uint16_t* h1;
    uint16_t* h2;
    float* partials;
    int nb;
  };
  __device__ __forceinline__ static void apply(f32x16_t (&acc)[4][4], const Args& a, const GemmProblem& p,
                                               int m0, int n0, char* smem) {
    const EpiLane L(m0, n0);
    const int M = p.M, N = p.N;
    char* stg = stage_base(smem, L.wave);
    float part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      part[j] = 0.f;
      const int m = L.row(j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = L.col(i, g);
          const u32x2_t zz = load_bf16x4(a.z, (size_t)m * N + n, m < M && n < N);
          const float h0 = acc[i][j][4 * g + 0] + bf16_lo(zz.x);
          const float h1 = acc[i][j][4 * g + 1] + bf16_hi(zz.x);
          const float h2 = acc[i][j][4 * g + 2] + bf16_lo(zz.y);
          const float h3 = acc[i][j][4 * g + 3] + bf16_hi(zz.y);
          acc[i][j][4 * g + 0] = h0;
          acc[i][j][4 * g + 1] = h1;
          acc[i][j][4 * g + 2] = h2;
          acc[i][j][4 * g + 3] = h3;
          part[j] += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
        }
    }
    __syncthreads();
    stage_flush<128>(stg, a.h1, (size_t)N, M, N, m0 + L.wm * 128, n0 + L.wn * 128, L.lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = L.col(i, g);
        const u32x2_t gg = load_bf16x4(a.gamma, (size_t)n, n < N);
        const float g0 = bf16_lo(gg.x), g1 = bf16_hi(gg.x), g2 = bf16_lo(gg.y), g3 = bf16_hi(gg.y);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(acc[i][j][4 * g] * g0, acc[i][j][4 * g + 1] * g1),
                     pack_bf16x2(acc[i][j][4 * g + 2] * g2, acc[i][j][4 * g + 3] * g3));
      }
    __syncthreads();
    stage_flush<128>(stg, a.h2, (size_t)N, M, N, m0 + L.wm * 128, n0 + L.wn * 128, L.lane);
    store_row_partials(part, smem, L, a.partials, a.nb, M);
  }
};

// ------------------------------------------------ GEMM2: deferred row scale y = r[m] acc
struct EpiRowScale {
  struct Args {
    const float* r;
    uint16_t* y;
  };
  __device__ __forceinline__ static void apply(f32x16_t (&acc)[4][4], const Args& a, const GemmProblem& p,
                                               int m0, int n0, char* smem) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(smem, L.wave);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = L.row(j);
      const float rr = m < p.M ? a.r[m] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(rr * acc[i][j][4 * g], rr * acc[i][j][4 * g + 1]),
                     pack_bf16x2(rr * acc[i][j][4 * g + 2], rr * acc[i][j][4 * g + 3]));
    }
    __syncthreads();
    stage_flush<128>(stg, a.y, (size_t)p.N, p.M, p.N, m0 + L.wm * 128, n0 + L.wn * 128, L.lane);
  }
};

// ------------------------------------------------------- QKV projection + RoPE on Q, K
struct EpiRope {
  struct Args {
    const float* cos_t;
    const float* sin_t;
    uint16_t* out;
    int n_rot;  // n_q + n_k: columns [0, n_rot) are rotated
    int head_dim;
    int seq_len;
    int pos_offset;
  };
  __device__ __forceinline__ static void apply(f32x16_t (&acc)[4][4], const Args& a, const GemmProblem& p,
                                               int m0, int n0, char* smem) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(smem, L.wave);
    const int half = a.head_dim >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = L.row(j);
      const int pos = m < p.M ? (int)(((long long)m + a.pos_offset) % a.seq_len) : 0;
      const float* crow = a.cos_t + (size_t)pos * half;
      const float* srow = a.sin_t + (size_t)pos * half;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = L.col(i, g);
          float e0 = acc[i][j][4 * g + 0], o0 = acc[i][j][4 * g + 1];
          float e1 = acc[i][j][4 * g + 2], o1 = acc[i][j][4 * g + 3];
          if (n < a.n_rot) {
            const int pp = (n % a.head_dim) >> 1;
            const float2 c = *(const float2*)(crow + pp);
            const float2 s = *(const float2*)(srow + pp);
            const float re0 = e0 * c.x - o0 * s.x, ro0 = e0 * s.x + o0 * c.x;
            const float re1 = e1 * c.y - o1 * s.y, ro1 = e1 * s.y + o1 * c.y;
            e0 = re0;
            o0 = ro0;
            e1 = re1;
            o1 = ro1;
          }
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(e0, o0), pack_bf16x2(e1, o1));
        }
    }
    __syncthreads();
    stage_flush<128>(stg, a.out, (size_t)p.N, p.M, p.N, m0 + L.wm * 128, n0 + L.wn * 128, L.lane);
  }
};

// ---------------------------------------------- SwiGLU: out[m, j] = silu(G_j) * U_j
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

struct EpiSwiGLU {
  struct Args {
    uint16_t* out;
    int F;  // output width (= N / 2)
  };
  __device__ __forceinline__ static void apply(f32x16_t (&acc)[4][4], const Args& a, const GemmProblem& p,
                                               int m0, int n0, char* smem) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(smem, L.wave);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float y0 = silu_f32(acc[i][j][4 * g + 0]) * acc[i][j][4 * g + 1];
          const float y1 = silu_f32(acc[i][j][4 * g + 2]) * acc[i][j][4 * g + 3];
          stage_put4(stg, L.srow(j), L.scol(i, g) >> 1, pack_bf16x2(y0, y1));
        }
    __syncthreads();
    stage_flush<64>(stg, a.out, (size_t)a.F, p.M, a.F, m0 + L.wm * 128, (n0 >> 1) + L.wn * 64, L.lane);
  }
};

// ------------------------- grad GEMM: dh2 = acc (stored) + partials of dh2 * h2 per row
struct EpiDotRowPartials {
  struct Args {
    const uint16_t* h2;
    uint16_t* dh2;
    float* partials;
    int nb;
  };
  __device__ __forceinline__ static void apply(f32x16_t (&acc)[4][4], const Args& a, const GemmProblem& p,
                                               int m0, int n0, char* smem) {
    const EpiLane L(m0, n0);
    const int M = p.M, N = p.N;
    char* stg = stage_base(smem, L.wave);
    float part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      part[j] = 0.f;
      const int m = L.row(j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = L.col(i, g);
          const u32x2_t hh = load_bf16x4(a.h2, (size_t)m * N + n, m < M && n < N);
          const float d0 = acc[i][j][4 * g + 0], d1 = acc[i][j][4 * g + 1];
          const float d2 = acc[i][j][4 * g + 2], d3 = acc[i][j][4 * g + 3];
          part[j] += d0 * bf16_lo(hh.x) + d1 * bf16_hi(hh.x) + d2 * bf16_lo(hh.y) + d3 * bf16_hi(hh.y);
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(d0, d1), pack_bf16x2(d2, d3));
        }
    }
    __syncthreads();
    stage_flush<128>(stg, a.dh2, (size_t)N, M, N, m0 + L.wm * 128, n0 + L.wn * 128, L.lane);
    store_row_partials(part, smem, L, a.partials, a.nb, M);
  }
};

template <bool kWKN, class Epi>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_epilogue_kernel(GemmProblem p, typename Epi::Args ea) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  int m0, n0;
  tile_coords(p.M, p.N, m0, n0);
  f32x16_t acc[4][4];
  gemm_mainloop<kWKN>(p, m0, n0, smem, acc);
  Epi::apply(acc, ea, p, m0, n0, smem);
}

inline int gemm_grid(int M, int N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

}  // namespace coda
