// One bf16 MFMA GEMM main loop for gfx950 and the epilogue programs that run on its
// accumulator tile before anything is written to HBM.
//
// Product: C[m, n] = sum_k X[m, k] * W(k, n), X = tokens x depth (row-major, depth
// contiguous), W either [K, N] row-major ("KN", features contiguous: the forward
// projections) or [N, K] row-major ("NK", depth contiguous: the grad GEMM dY W1^T).
//
// Workgroup tile: 256 tokens x 256 features, 512 threads = 8 waves, two per SIMD, in a
// 2 (tokens) x 4 (features) arrangement; each wave owns 128 tokens x 64 features = 2 x 4
// blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane). While one wave of
// a SIMD waits on a barrier or an LDS read, the other keeps the MFMA pipe busy.
//
// Transposed MFMA formulation. The MFMA "A" operand (rows of the MFMA output) is the
// W slice, so MFMA rows are FEATURES; the "B" operand is the X slice, so MFMA columns
// are TOKENS. With the 32x32 output layout (lane l, register v holds row
// 8*(v/4) + 4*(l/32) + v%4, column l%32), every lane holds, for one token, runs of 4
// consecutive features: the (even, odd) feature pairs of RoPE and SwiGLU sit in one
// lane's registers, and a row statistic is an in-lane sum plus one exchange between
// the two 32-lane halves.
//
// Data movement. Both operand tiles go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no register staging), through a ring of 4 LDS stages of
// 32 depth each, so three depth-steps are in flight while one is consumed. X and NK-W
// tiles are stored depth-contiguous ([row][32] bf16, 64 B per row); a KN-W tile keeps
// its natural [32][256] layout and is transposed on the way out of LDS by
// ds_read_b64_tr_b16 into the depth-contiguous MFMA operand. All tiles XOR-swizzle
// their 16-byte chunks per row so that both the DMA writes and the operand reads are
// free of bank conflicts. Raw buffer descriptors make rows past M, depth past K and
// columns past N read as zero, so ragged edges need no special path.
//
// Schedule of one depth-step S (two k16 sub-steps), per wave:
//   read the sub-step-1 operands of S | 8 MFMAs of sub-step 0 of S |
//   wait for this thread's loads of S+1, barrier (S+1 complete for every wave, S-1 no
//   longer read by anyone) | 8 MFMAs of sub-step 1 of S, interleaved one for one with
//   the reads of sub-step 0 of S+1 and the DMA loads of S+3 into the slot of S-1.
// The order is pinned with scheduling barriers; the code is straight-line (the DMA of
// steps past the end only zero-fills a free slot) so the compiler's LDS wait counts
// never make an MFMA wait for reads issued after its operands.
#pragma once

#include "coda_common.hpp"

namespace coda {

constexpr int kBM = 256;        // tokens per workgroup tile
constexpr int kBN = 256;        // features per workgroup tile (== CODA_PARTIAL_TILE_N)
constexpr int kBK = 32;         // depth per LDS stage
constexpr int kStages = 4;      // LDS ring depth
constexpr int kWaves = 8;       // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesN = 4;      // waves along features
constexpr int kNI = 2;          // 32-feature MFMA blocks per wave
constexpr int kMJ = 4;          // 32-token MFMA blocks per wave
constexpr int kWaveN = 32 * kNI;  // features per wave (64)
constexpr int kXJ = 16 / kWaves;  // 1 KiB DMA instructions per wave per operand per step
constexpr int kLoadsPerStep = 2 * kXJ;  // 16-byte DMA loads per thread per step
constexpr int kTileBytes = kBM * kBK * 2;  // one operand tile per stage: 16 KiB
constexpr int kStgPitch = kWaveN + 4;      // epilogue staging row pitch, bf16 elements
constexpr int kStgWaveBytes = 128 * kStgPitch * 2;
constexpr int kSlotBytes = 2 * kStgWaveBytes > 2 * kTileBytes ? 2 * kStgWaveBytes : 2 * kTileBytes;
constexpr int kRedFloats = 2 * kWavesN * 128;
static_assert(kStages * kSlotBytes + 4 * kRedFloats <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
static_assert(kWaves == 2 * kWavesN && kWavesN * kWaveN == kBN, "wave layout covers the tile");

struct GemmProblem {
  const uint16_t* x;  // [M, K]
  const uint16_t* w;  // [K, N] (KN) or [N, K] (NK)
  int M, N, K;
};

// LDS of one workgroup: four stage slots (each also holds two waves' epilogue staging
// blocks) and the row-partial exchange area.
struct LdsRing {
  char* slot[kStages];
  float* red;
};

// Swizzle of the four 16-byte chunks of a depth-contiguous 64-byte row (X and NK-W
// tiles): operand reads hit 8 consecutive rows (32 banks) or 16 (64 banks) at one
// logical chunk; rows of equal parity (resp. equal residue mod 4) differ in bank line.
__device__ __forceinline__ uint32_t swz_k(int row) { return (uint32_t)(((row >> 1) ^ (row >> 3)) & 3); }
__device__ __forceinline__ uint32_t krow_off(int row, int chunk) {
  return ((uint32_t)row << 6) | (((uint32_t)chunk ^ swz_k(row)) << 4);
}
// Swizzle of the 32 chunks of a 512-byte KN-W row: a transposed read touches 4
// consecutive depth rows x 2 (or 4) chunks; rows r = 0..3 (mod 4) XOR with 0, 6, 10,
// 12, which spreads those 8 (16) chunks over distinct banks.
__device__ __forceinline__ uint32_t swz_n(int row) { return (0xCA60u >> (4 * (row & 3))) & 0xFu; }
__device__ __forceinline__ uint32_t nrow_off(int row, int chunk) {
  return ((uint32_t)row << 9) | (((uint32_t)chunk ^ swz_n(row)) << 4);
}

// Workgroup -> output tile: groups of 2 token-tiles walked feature-tile by feature-tile.
// Consecutive workgroups go round-robin to the 8 XCDs, so each XCD receives tiles of one
// token-tile parity and every fourth feature-tile: 8 X panels and 4 W panels shared by
// its 32 concurrent tiles, which the XCD's L2 serves. (Measured on MI355X against other
// groupings and an explicit XCD-contiguous remap; this order was the fastest.)
constexpr int kGroupM = 2;
__device__ __forceinline__ void tile_coords(int M, int N, int& m0, int& n0) {
  const int mt = (M + kBM - 1) / kBM;
  const int nt = (N + kBN - 1) / kBN;
  const int t = blockIdx.x;
  const int group = t / (kGroupM * nt);
  const int first_m = group * kGroupM;
  const int gm = min(mt - first_m, kGroupM);
  const int rem = t - group * kGroupM * nt;
  m0 = (first_m + rem % gm) * kBM;
  n0 = (rem / gm) * kBN;
}

// Depth step a workgroup starts at: the K loop of each block is rotated by an eighth of
// K per XCD (blockIdx % 8), so the XCDs stream different depth ranges of the shared
// panels at any moment instead of all hitting the same addresses. The tile's sum covers
// the same products; only the (fixed, deterministic) accumulation order changes.
__device__ __forceinline__ int k_rotation(int KT) { return (int)((blockIdx.x % 8) * (KT / 8)); }

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor as four words (for the inline-asm LDS DMA below).
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4_t r;
  r.x = (int)(uint32_t)a;
  r.y = (int)(uint32_t)(a >> 32);  // stride 0, no swizzle
  r.z = (int)bytes;
  r.w = (int)kBufferWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// One 16-byte-per-lane DMA from HBM into LDS: lane i's 16 bytes land at
// lds_base + 16 i. Issued from inline asm so that the compiler neither reorders LDS
// accesses across it nor inserts its own conservative vmcnt waits; completion is
// tracked explicitly with wait_vmcnt before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(const i32x4_t& rsrc_in, uint32_t lds_base, uint32_t voff) {
  i32x4_t rsrc;  // the descriptor must live in SGPRs
  rsrc.x = __builtin_amdgcn_readfirstlane(rsrc_in.x);
  rsrc.y = __builtin_amdgcn_readfirstlane(rsrc_in.y);
  rsrc.z = __builtin_amdgcn_readfirstlane(rsrc_in.z);
  rsrc.w = __builtin_amdgcn_readfirstlane(rsrc_in.w);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory");
}

// s_waitcnt vmcnt(N): wait until at most N vector-memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

typedef __attribute__((address_space(3))) const bf16x8_t* lds_b128_ptr;
typedef __attribute__((address_space(3))) i16x4_t* lds_tr_ptr;

template <bool kWKN>
struct Mainloop {
  i32x4_t xrs, wrs_nk;    // descriptors of the tile's X rows and (NK) W rows
  uint32_t wave_u;        // wave index, wave-uniform
  uint32_t x_off[kXJ];    // byte offsets of this lane's X chunks (depth 0 of the tile)
  uint32_t x_kchunk[kXJ]; // logical depth chunk (0..3) of each X load
  uint32_t w_off[kXJ];    // KN: offset within the stage's depth rows; NK: like x_off
  uint32_t w_kchunk[kXJ];
  bool w_col_ok[kXJ];
  const uint16_t* wbase;
  int M, N, K, m0, n0;
  int KT, kstart;           // depth steps and the rotated first step
  uint32_t xr_off[2];       // operand read offsets within a slot, per k16 sub-step
  uint32_t wr_off[2][kNI][2];

  __device__ __forceinline__ void init(const GemmProblem& p, int m0_, int n0_) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    wave_u = (uint32_t)wave;
    M = p.M;
    N = p.N;
    K = p.K;
    KT = (K + kBK - 1) / kBK;
    kstart = k_rotation(KT);
    m0 = m0_;
    n0 = n0_;
    wbase = p.w;
    const uint32_t kb = (uint32_t)K * 2u;
    xrs = rsrc_words(p.x + (size_t)m0 * K, (uint32_t)min(kBM, M - m0) * kb);
    wrs_nk = kWKN ? rsrc_words(p.w, 0u) : rsrc_words(p.w + (size_t)n0 * K, (uint32_t)min(kBN, N - n0) * kb);
#pragma unroll
    for (int j = 0; j < kXJ; ++j) {
      // X (and NK-W): instruction j of wave w fills rows (kXJ w + j)*16 .. +15 of the tile
      const int row = (wave * kXJ + j) * 16 + (lane >> 2);
      const uint32_t c = (uint32_t)(lane & 3) ^ swz_k(row);
      x_kchunk[j] = c;
      x_off[j] = (uint32_t)row * kb + c * 16u;
      if constexpr (kWKN) {
        // KN-W: instruction j of wave w fills depth rows (kXJ w + j)*2 .. +1
        const int wrow = (wave * kXJ + j) * 2 + (lane >> 5);
        const uint32_t wc = (uint32_t)(lane & 31) ^ swz_n(wrow);
        w_col_ok[j] = n0 + 8 * (int)wc < N;
        w_off[j] = ((uint32_t)wrow * (uint32_t)N + 8u * wc) * 2u;
        w_kchunk[j] = (uint32_t)wrow;
      } else {
        w_off[j] = x_off[j];
        w_kchunk[j] = c;
        w_col_ok[j] = true;
      }
    }
    const int r32 = lane & 31, hs = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      xr_off[ks] = krow_off(wm * 128 + r32, 2 * ks + hs);
      if constexpr (kWKN) {
        // transposed read: in each 16-lane group, lane 4e+q points at depth row e of the
        // group's 4 rows, features 4q..4q+3; lane i receives feature i of all 4 rows
        const int g = lane >> 4, s = lane & 15, e = s >> 2, q = s & 3;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          const int nb = wn * kWaveN + i * 32 + (g & 1) * 16 + 4 * q;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = ks * 16 + (g >> 1) * 8 + 4 * h + e;
            wr_off[ks][i][h] = kTileBytes + nrow_off(row, nb >> 3) + (uint32_t)((nb >> 2) & 1) * 8u;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          wr_off[ks][i][0] = kTileBytes + krow_off(wn * kWaveN + i * 32 + r32, 2 * ks + hs);
          wr_off[ks][i][1] = 0;
        }
      }
    }
  }

  // DMA load number j (0 .. kLoadsPerStep-1) of the kt-th depth step (rotated) into
  // `slot`. Steps past the end (kt >= KT) issue out-of-range loads that only zero-fill
  // a slot nobody reads.
  __device__ __forceinline__ void issue_one(char* slot, int kt, int j) const {
    const int ksr = kt + kstart;
    const int k0 = (kt >= KT) ? K : (ksr >= KT ? ksr - KT : ksr) * kBK;
    if (j < kXJ) {
      const uint32_t xs = lds_addr(slot) + wave_u * (kXJ * 1024u);
      const bool ok = k0 + 8 * (int)x_kchunk[j] < K;
      dma16(xrs, xs + j * 1024u, ok ? x_off[j] + (uint32_t)k0 * 2u : kOutOfRange);
    } else {
      const int jj = j - kXJ;
      const uint32_t ws = lds_addr(slot) + (uint32_t)kTileBytes + wave_u * (kXJ * 1024u);
      if constexpr (kWKN) {
        const int krows = max(0, min(kBK, K - k0));
        const i32x4_t wrs = rsrc_words(wbase + (size_t)min(k0, K - 1) * N + n0,
                                       krows ? ((uint32_t)krows * (uint32_t)N - (uint32_t)n0) * 2u : 0u);
        dma16(wrs, ws + jj * 1024u, w_col_ok[jj] ? w_off[jj] : kOutOfRange);
      } else {
        const bool ok = k0 + 8 * (int)w_kchunk[jj] < K;
        dma16(wrs_nk, ws + jj * 1024u, ok ? w_off[jj] + (uint32_t)k0 * 2u : kOutOfRange);
      }
    }
  }

  __device__ __forceinline__ void issue(char* slot, int kt) const {
#pragma unroll
    for (int j = 0; j < kLoadsPerStep; ++j) issue_one(slot, kt, j);
  }

  __device__ __forceinline__ void read(const char* slot, int ks, bf16x8_t (&a)[kNI], bf16x8_t (&b)[kMJ]) const {
    // Opaque, wave-uniform slot base: keeps the compiler from hoisting one address
    // register per (slot, read) out of the loop.
    uint32_t base = lds_addr(slot);
    asm volatile("" : "+s"(base));
    const uint32_t xb = base + xr_off[ks];
#pragma unroll
    for (int j = 0; j < kMJ; ++j) b[j] = *(lds_b128_ptr)(uintptr_t)(xb + j * 32 * 64);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      if constexpr (kWKN) {
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_ptr)(uintptr_t)(base + wr_off[ks][i][0]));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_ptr)(uintptr_t)(base + wr_off[ks][i][1]));
        a[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        a[i] = *(lds_b128_ptr)(uintptr_t)(base + wr_off[ks][i][0]);
      }
    }
  }
};

template <bool kWKN>
__device__ __forceinline__ void gemm_mainloop(const GemmProblem& p, int m0, int n0, const LdsRing& lds,
                                              f32x16_t (&acc)[kNI][kMJ]) {
  Mainloop<kWKN> ml;
  ml.init(p, m0, n0);
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = ml.KT;
  constexpr int kReads = kMJ + (kWKN ? 2 * kNI : kNI);  // LDS read instructions per k16 sub-step
  constexpr int kMfma = kNI * kMJ;                      // MFMAs per k16 sub-step
  constexpr int L = kLoadsPerStep;

  // prologue: steps 0, 1, 2 in flight; wait for step 0
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) ml.issue(lds.slot[s], s);
  wait_vmcnt<2 * L>();
  __builtin_amdgcn_s_barrier();

  bf16x8_t a0[kNI], b0[kMJ], a1[kNI], b1[kMJ];
  ml.read(lds.slot[0], 0, a0, b0);

  auto step = [&](const int S, const int kt) {
    ml.read(lds.slot[S], 1, a1, b1);
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
      for (int j = 0; j < kMJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // sub-step-1 reads first
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);   // then the sub-step-0 MFMAs
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<L>();  // this thread's loads of step kt+1 have landed (kt+2 may fly)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t na[kNI], nb[kMJ];
    ml.read(lds.slot[(S + 1) % kStages], 0, na, nb);
#pragma unroll
    for (int r = 0; r < kMfma; ++r) {
      const int i = r / kMJ, j = r % kMJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
      if (r < L) ml.issue_one(lds.slot[(S + 3) % kStages], kt + 3, r);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (r < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
#pragma unroll
    for (int i = 0; i < kNI; ++i) a0[i] = na[i];
#pragma unroll
    for (int j = 0; j < kMJ; ++j) b0[j] = nb[j];
  };

  int kt = 0;
  for (; kt + kStages <= KT; kt += kStages) {
    step(0, kt);
    step(1, kt + 1);
    step(2, kt + 2);
    step(3, kt + 3);
  }
  if (kt < KT) step(0, kt);
  if (kt + 1 < KT) step(1, kt + 1);
  if (kt + 2 < KT) step(2, kt + 2);
  wait_vmcnt<0>();  // trailing zero-fill loads land before the epilogue reuses LDS
  __syncthreads();  // all operand reads are done before the slots hold staging data
}

// ------------------------------------------------------------------------------------
// Epilogue helpers. Accumulator block acc[i][j] of a lane covers features
//   n = n0 + wn*64 + 32 i + 8 g + 4 (lane >> 5) + e,  (register v = 4 g + e)
// for the token m = m0 + wm*128 + 32 j + (lane & 31).
struct EpiLane {
  int lane, wave, wm, wn, m0, n0;
  __device__ __forceinline__ EpiLane(int m0_, int n0_)
      : lane(threadIdx.x & 63), wave(threadIdx.x >> 6), wm((threadIdx.x >> 6) / kWavesN),
        wn((threadIdx.x >> 6) % kWavesN), m0(m0_), n0(n0_) {}
  __device__ __forceinline__ int row(int j) const { return m0 + wm * 128 + 32 * j + (lane & 31); }
  __device__ __forceinline__ int col(int i, int g) const {
    return n0 + wn * kWaveN + 32 * i + 8 * g + 4 * (lane >> 5);
  }
  // wave-local staging coordinates
  __device__ __forceinline__ int srow(int j) const { return 32 * j + (lane & 31); }
  __device__ __forceinline__ int scol(int i, int g) const { return 32 * i + 8 * g + 4 * (lane >> 5); }
};

// Each wave stages its [128 x 64] block in half of one LDS slot.
__device__ __forceinline__ char* stage_base(const LdsRing& lds, int wave) {
  char* s = (wave >> 1) == 0 ? lds.slot[0] : (wave >> 1) == 1 ? lds.slot[1] : (wave >> 1) == 2 ? lds.slot[2] : lds.slot[3];
  return s + (wave & 1) * kStgWaveBytes;
}

__device__ __forceinline__ void stage_put8(char* stg, int r, int c, uint32_t lo, uint32_t hi) {
  u32x2_t v;
  v.x = lo;
  v.y = hi;
  *(u32x2_t*)(stg + (r * kStgPitch + c) * 2) = v;
}
__device__ __forceinline__ void stage_put4(char* stg, int r, int c, uint32_t w) {
  *(uint32_t*)(stg + (r * kStgPitch + c) * 2) = w;
}

// Write a wave's staged [128 rows x kCols] bf16 block to out[row0 + r, col0 + c] (row
// pitch ldo elements) with 16-byte row-contiguous stores.
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
// halves, then the four feature-waves wn = 0, 1, 2, 3 in turn.
__device__ __forceinline__ void store_row_partials(float (&part)[kMJ], const LdsRing& lds, const EpiLane& L,
                                                   float* __restrict__ partials, int nb, int M) {
#pragma unroll
  for (int j = 0; j < kMJ; ++j) part[j] += __shfl_xor(part[j], 32);
  float* red = lds.red;
  if (L.lane < 32) {
#pragma unroll
    for (int j = 0; j < kMJ; ++j) red[(L.wm * kWavesN + L.wn) * 128 + 32 * j + L.lane] = part[j];
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < kBM) {
    const int wm = t >> 7, r = t & 127;
    const int m = L.m0 + t;
    float s = red[(wm * kWavesN + 0) * 128 + r];
#pragma unroll
    for (int w = 1; w < kWavesN; ++w) s += red[(wm * kWavesN + w) * 128 + r];
    if (m < M) partials[(size_t)m * nb + L.n0 / kBN] = s;
  }
}

__device__ __forceinline__ u32x2_t load_bf16x4(const uint16_t* __restrict__ base, size_t idx, bool ok) {
  u32x2_t v;
  v.x = 0u;
  v.y = 0u;
  if (ok) v = *(const u32x2_t*)(base + idx);
  return v;
}

typedef f32x16_t AccTile[kNI][kMJ];

// ---------------------------------------------------------------- plain store (baseline)
struct EpiStore {
  struct Args {
    uint16_t* out;
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(lds, L.wave);
#pragma unroll
    for (int j = 0; j < kMJ; ++j)
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                     pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
    __syncthreads();
    stage_flush<kWaveN>(stg, a.out, (size_t)p.N, p.M, p.N, m0 + L.wm * 128, n0 + L.wn * kWaveN, L.lane);
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
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0);
    const int M = p.M, N = p.N;
    char* stg = stage_base(lds, L.wave);
    float part[kMJ];
#pragma unroll
    for (int j = 0; j < kMJ; ++j) {
      part[j] = 0.f;
      const int m = L.row(j);
#pragma unroll
      for (int i = 0; i < kNI; ++i)
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
    stage_flush<kWaveN>(stg, a.h1, (size_t)N, M, N, m0 + L.wm * 128, n0 + L.wn * kWaveN, L.lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = L.col(i, g);
        const u32x2_t gg = load_bf16x4(a.gamma, (size_t)n, n < N);
        const float g0 = bf16_lo(gg.x), g1 = bf16_hi(gg.x), g2 = bf16_lo(gg.y), g3 = bf16_hi(gg.y);
#pragma unroll
        for (int j = 0; j < kMJ; ++j)
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(acc[i][j][4 * g] * g0, acc[i][j][4 * g + 1] * g1),
                     pack_bf16x2(acc[i][j][4 * g + 2] * g2, acc[i][j][4 * g + 3] * g3));
      }
    __syncthreads();
    stage_flush<kWaveN>(stg, a.h2, (size_t)N, M, N, m0 + L.wm * 128, n0 + L.wn * kWaveN, L.lane);
    store_row_partials(part, lds, L, a.partials, a.nb, M);
  }
};

// ------------------------------------------------ GEMM2: deferred row scale y = r[m] acc
struct EpiRowScale {
  struct Args {
    const float* r;
    uint16_t* y;
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(lds, L.wave);
#pragma unroll
    for (int j = 0; j < kMJ; ++j) {
      const int m = L.row(j);
      const float rr = m < p.M ? a.r[m] : 0.f;
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          stage_put8(stg, L.srow(j), L.scol(i, g), pack_bf16x2(rr * acc[i][j][4 * g], rr * acc[i][j][4 * g + 1]),
                     pack_bf16x2(rr * acc[i][j][4 * g + 2], rr * acc[i][j][4 * g + 3]));
    }
    __syncthreads();
    stage_flush<kWaveN>(stg, a.y, (size_t)p.N, p.M, p.N, m0 + L.wm * 128, n0 + L.wn * kWaveN, L.lane);
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
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(lds, L.wave);
    const int half = a.head_dim >> 1;
#pragma unroll
    for (int j = 0; j < kMJ; ++j) {
      const int m = L.row(j);
      const int pos = m < p.M ? (int)(((long long)m + a.pos_offset) % a.seq_len) : 0;
      const float* crow = a.cos_t + (size_t)pos * half;
      const float* srow = a.sin_t + (size_t)pos * half;
#pragma unroll
      for (int i = 0; i < kNI; ++i)
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
    stage_flush<kWaveN>(stg, a.out, (size_t)p.N, p.M, p.N, m0 + L.wm * 128, n0 + L.wn * kWaveN, L.lane);
  }
};

// ---------------------------------------------- SwiGLU: out[m, j] = silu(G_j) * U_j
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

struct EpiSwiGLU {
  struct Args {
    uint16_t* out;
    int F;  // output width (= N / 2)
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0);
    char* stg = stage_base(lds, L.wave);
#pragma unroll
    for (int j = 0; j < kMJ; ++j)
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float y0 = silu_f32(acc[i][j][4 * g + 0]) * acc[i][j][4 * g + 1];
          const float y1 = silu_f32(acc[i][j][4 * g + 2]) * acc[i][j][4 * g + 3];
          stage_put4(stg, L.srow(j), L.scol(i, g) >> 1, pack_bf16x2(y0, y1));
        }
    __syncthreads();
    stage_flush<kWaveN / 2>(stg, a.out, (size_t)a.F, p.M, a.F, m0 + L.wm * 128, (n0 >> 1) + L.wn * (kWaveN / 2),
                            L.lane);
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
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0);
    const int M = p.M, N = p.N;
    char* stg = stage_base(lds, L.wave);
    float part[kMJ];
#pragma unroll
    for (int j = 0; j < kMJ; ++j) {
      part[j] = 0.f;
      const int m = L.row(j);
#pragma unroll
      for (int i = 0; i < kNI; ++i)
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
    stage_flush<kWaveN>(stg, a.dh2, (size_t)N, M, N, m0 + L.wm * 128, n0 + L.wn * kWaveN, L.lane);
    store_row_partials(part, lds, L, a.partials, a.nb, M);
  }
};

template <bool kWKN, class Epi>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_epilogue_kernel(GemmProblem p, typename Epi::Args ea) {
  __shared__ __attribute__((aligned(1024))) char slot0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot3[kSlotBytes];
  __shared__ __attribute__((aligned(16))) float red[kRedFloats];
  const LdsRing lds{{slot0, slot1, slot2, slot3}, red};
  int m0, n0;
  tile_coords(p.M, p.N, m0, n0);
  AccTile acc;
  gemm_mainloop<kWKN>(p, m0, n0, lds, acc);
  Epi::apply(acc, ea, p, m0, n0, lds);
}

inline int gemm_grid(int M, int N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

}  // namespace coda
