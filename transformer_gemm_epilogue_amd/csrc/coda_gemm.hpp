// One bf16 MFMA GEMM main loop for gfx950 and the epilogue programs that run on its
// accumulator tile before anything is written to HBM.
//
// Product: C[m, n] = sum_k X[m, k] * W(k, n), X = tokens x depth (row-major, depth
// contiguous), W either [K, N] row-major ("KN", features contiguous: the forward
// projections) or [N, K] row-major ("NK", depth contiguous: the grad GEMM dY W1^T).
//
// Workgroup tile: 256 tokens x 256 features, 512 threads = 8 waves, two per SIMD, in a
// 2 (tokens) x 4 (features) arrangement; each wave owns 128 tokens x 64 features = 4 x 8
// blocks of v_mfma_f32_16x16x32_bf16 (128 fp32 accumulators per lane). While one wave of
// a SIMD waits on a barrier or an LDS read, the other keeps the MFMA pipe busy. The
// 16x16x32 form reads and writes a quarter of the accumulator bytes per flop of the
// 32x32x16 one; on gfx950, whose clock is set by power on this loop, that buys a higher
// clock (measured on MI355X, gaussian operands: +7% in a register-only loop, +4-8% for
// this main loop together with the paired X loads below).
//
// Transposed MFMA formulation. The MFMA "A" operand (rows of the MFMA output) is the
// W slice, so MFMA rows are FEATURES; the "B" operand is the X slice, so MFMA columns
// are TOKENS. An operand lane l holds row l % 16 of its block at depth 8 (l / 16) .. +7;
// in the 16x16 output layout lane l, register v holds row 4 (l / 16) + v, column l % 16,
// so every lane holds, for one token, runs of 4 consecutive features. The epilogue keeps
// that property when it re-lays each wave's block out row-major (16 lanes per token, 4
// consecutive features per lane): the (even, odd) feature pairs of RoPE and SwiGLU stay
// in one lane's registers.
//
// Data movement. Both operand tiles go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no register staging), through a ring of 5 LDS stages of
// 32 depth each (160 KiB), so loads for up to four depth-steps are in flight while one
// is consumed. X and NK-W
// tiles are stored depth-contiguous ([row][32] bf16, 64 B per row); a KN-W tile keeps
// its natural [32][256] layout and is transposed on the way out of LDS by
// ds_read_b64_tr_b16 into the depth-contiguous MFMA operand. All tiles XOR-swizzle
// their 16-byte chunks per row so that both the DMA writes and the operand reads are
// free of bank conflicts. Raw buffer descriptors make rows past M, depth past K and
// columns past N read as zero, so ragged edges need no special path.
//
// Schedule of one depth-step S (32 MFMAs per wave: 4 feature blocks x 8 token blocks),
// per wave:
//   read X blocks 4..7 of S | the 16 MFMAs on token blocks 0..3 of S, and the W half of
//   the DMA of S+3 into the slot of S-2 | wait for this thread's loads of S+1, barrier
//   (S+1 complete for every wave, S-1 no longer read by anyone) | the 16 MFMAs on token
//   blocks 4..7 of S, interleaved one for one with the reads of W and X blocks 0..3 of
//   S+1, and, on odd steps, the X halves of the DMA of S+3 and S+4 (slots of S-2, S-1)
//   behind every other one of the last eight of those MFMAs.
// X loads go in pairs because a 32-deep X row is 64 bytes, half of a 128-byte vector-L1
// line: issued back to back, the loads of steps 2p and 2p+1 share each line, where
// loads a step apart fetched every line from L2 twice (measured on MI355X: L1 -> L2
// requests 87.8 M -> 58.8 M per 8192 x 4096 x 14336 product, and less power).
// A slot is written only after the barrier that follows its last reader's consumption,
// and the load issue is spread over the steps: on gfx950 the operand delivery is
// bounded by how many DMA loads are in flight (texture data path busy, waiting on L1),
// and the fifth stage raises that bound from 8 to 12 loads per wave.
// The order is pinned with scheduling barriers; the code is straight-line (the DMA of
// steps past the end only zero-fills a free slot) so the compiler's LDS wait counts
// never make an MFMA wait for reads issued after its operands.
#pragma once

#include <type_traits>

#include "coda_common.hpp"

namespace coda {

constexpr int kBM = 256;        // tokens per workgroup tile
constexpr int kBN = 256;        // features per workgroup tile (== CODA_PARTIAL_TILE_N)
constexpr int kBK = 32;         // depth per LDS stage
constexpr int kStages = 5;      // LDS ring depth
constexpr int kWaves = 8;       // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesN = 4;      // waves along features
constexpr int kNI = 4;          // 16-feature MFMA blocks per wave
constexpr int kMJ = 8;          // 16-token MFMA blocks per wave
constexpr int kWaveN = 16 * kNI;  // features per wave (64)
constexpr int kXJ = 16 / kWaves;  // 1 KiB DMA instructions per wave per operand per step
constexpr int kLoadsPerStep = 2 * kXJ;  // 16-byte DMA loads per thread per step
constexpr int kTileBytes = kBM * kBK * 2;  // one operand tile per stage: 16 KiB
constexpr int kSlotBytes = 2 * kTileBytes;  // one stage: X tile + W tile
constexpr int kStgRows = 32;                // tokens a wave re-lays out at a time
constexpr int kStgWaveBytes = kStgRows * kWaveN * 4;  // fp32: 8 KiB per wave
constexpr int kRedFloats = 2 * kWavesN * 128;
static_assert(4 * kStgWaveBytes == kSlotBytes, "four waves' staging areas fill one slot");
static_assert(4 * kRedFloats <= kSlotBytes, "the row exchange fits in one slot");
static_assert(kStages * kSlotBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
static_assert(kWaves == 2 * kWavesN && kWavesN * kWaveN == kBN, "wave layout covers the tile");

struct GemmProblem {
  const uint16_t* x;  // [M, K]
  const uint16_t* w;  // [K, N] (KN) or [N, K] (NK)
  int M, N, K;
  int group_m = 0;    // token-tiles per raster group; 0: chosen from the shape (raster_group_m)
};

// LDS of one workgroup: five stage slots (in the main loop's order), and the epilogue's
// areas in three of them: staging of waves 0-3 (stg[0]) and 4-7 (stg[1]), and the
// row-statistic exchange (red). tid is the thread index the epilogue works from.
struct LdsRing {
  char* slot[kStages];
  float* red;
  char* stg[2];
  int tid;
};

// Swizzle of the four 16-byte chunks of a depth-contiguous 64-byte row (X and NK-W
// tiles). gfx950 serves a 64-lane ds_read_b128 in four groups of 16 lanes over 64
// banks; measured with the LDS bank-conflict counter, a group is one 32-lane half split
// by lane bit 4 XOR lane bit 2 (give or take lanes bits 0, 1, 3). The operand read has
// lane l on row l % 16, chunk l / 16, so XOR-ing the chunk with 2 on rows whose bit 3 is
// set spreads every such group over all 64 banks, whichever of those lane bits join in
// (row bit 2 must stay out: it follows lane bit 2). The DMA writes whole 64-byte rows
// per 4 lanes, which any per-row permutation of the chunks keeps conflict-free.
__device__ __forceinline__ uint32_t swz_k(int row) { return (uint32_t)(((row >> 3) & 1) << 1); }
__device__ __forceinline__ uint32_t krow_off(int row, int chunk) {
  return ((uint32_t)row << 6) | (((uint32_t)chunk ^ swz_k(row)) << 4);
}
// Swizzle of the 32 chunks of a 512-byte KN-W row: each 16-lane group of a transposed
// read touches 4 consecutive depth rows x 2 chunks, and the two groups served together
// (32 lanes, 256 bytes) read the same chunks 8 rows apart. Rows r = 0..3 (mod 4) XOR
// with 0, 6, 10, 12, which spreads a group's 8 chunks over distinct banks, and rows with
// bit 3 set XOR with 2 more, which moves the partner group onto the other 8.
__device__ __forceinline__ uint32_t swz_n(int row) {
  return ((0xCA60u >> (4 * (row & 3))) & 0xFu) ^ ((uint32_t)((row >> 3) & 1) << 1);
}
__device__ __forceinline__ uint32_t nrow_off(int row, int chunk) {
  return ((uint32_t)row << 9) | (((uint32_t)chunk ^ swz_n(row)) << 4);
}

// Workgroup -> output tile: groups of G token-tiles walked feature-tile by feature-tile
// (token tile fastest within a group). Consecutive workgroups go round-robin to the 8
// XCDs. With G = 2 each XCD receives tiles of one token-tile parity and every fourth
// feature-tile (8 X panels and 4 W panels shared by its 32 concurrent tiles, which its
// L2 serves), and the 256 concurrent tiles cover 16 token-tiles x all features when the
// width is 16 tiles: the best order measured on MI355X for weights that fit the 256 MiB
// Infinity Cache (also against an explicit XCD-contiguous remap). A weight larger than
// that would then be streamed from HBM again by every wave of 256 tiles; with G = 32
// each wave instead covers up to 8192 tokens x 8 feature-tiles (an XCD: 4 X and 8 W
// panels), the token rows stay cache-resident across waves and the weight is streamed
// once (measured: GEMM + RoPE 8192 x 24576 x 8192 +11%, 8192 x 32768 x 8192 +16%,
// 4096 x 32768 x 4096 +8%; no gain below the cache size).
__host__ __device__ inline int raster_group_m(int M, int N, int K) {
  const long long w_bytes = 2LL * N * K;
  const long long x_group_bytes = 2LL * (M < 32 * kBM ? M : 32 * kBM) * K;
  return (w_bytes > (192LL << 20) && x_group_bytes <= (160LL << 20)) ? 32 : 2;
}
__device__ __forceinline__ void tile_coords(int M, int N, int K, int group_m, int t, int& m0, int& n0) {
  const int mt = (M + kBM - 1) / kBM;
  const int nt = (N + kBN - 1) / kBN;
  const int G = group_m > 0 ? group_m : raster_group_m(M, N, K);
  const int group = t / (G * nt);
  const int first_m = group * G;
  const int gm = min(mt - first_m, G);
  const int rem = t - group * G * nt;
  m0 = (first_m + rem % gm) * kBM;
  n0 = (rem / gm) * kBN;
}

// Depth step tile t starts at: the K loop is rotated by an eighth of K per XCD (t % 8,
// the XCD that workgroup t, or a persistent workgroup t mod 8k, runs on), so the XCDs
// stream different depth ranges of the shared panels at any moment instead of all
// hitting the same addresses. The tile's sum covers the same products; only the
// (fixed, deterministic) accumulation order changes, and it depends on t alone. The
// rotation is an even number of steps, so that paired X loads (steps 2p, 2p+1) still
// share 128-byte lines.
__device__ __forceinline__ int k_rotation(int t, int KT) { return (t % 8) * ((KT / 8) & ~1); }

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

// DMA sources of one output tile: descriptors of its X rows and of W (NK: the tile's W
// rows; KN, one-descriptor form: the tile's W columns over the whole depth; unused by the
// per-step KN form), which of this lane's KN-W chunks lie inside the width, and the
// tile's rotated first depth step.
struct TileSrc {
  i32x4_t xrs, wrs;
  int n0, kstart;
  bool w_col_ok[kXJ];
};

typedef f32x4_t AccTile[kNI][kMJ];

// KN-W loads come in two forms. With kWOneDesc, one descriptor per tile covers W's
// columns n0.. over the whole depth and a load's depth offset goes into its per-lane
// offset; rows past K lie outside the descriptor's range and read as zeros. That needs
// every such offset below 2^31, (K + kBK) N < 2^30 elements. Otherwise each depth step
// builds a descriptor of its own 32 rows (a 64-bit base computed per step: about 15 more
// scalar instructions per step; the one-descriptor form measured 1.5-2.3% faster on the
// 8192-class shapes, bit-identical).
__host__ __device__ constexpr bool kn_one_descriptor_fits(int K, int N) {
  return ((long long)K + kBK) * (long long)N < (1ll << 30);
}

template <bool kWKN, bool kWOneDesc = false>
struct Mainloop {
  static constexpr bool kKN = kWKN;
  static_assert(kWKN || !kWOneDesc, "the one-descriptor form is for the KN layout");
  uint32_t wave_u;        // wave index, wave-uniform
  uint32_t x_off[kXJ];    // byte offsets of this lane's X chunks (depth 0 of the tile)
  uint32_t x_kchunk[kXJ]; // logical depth chunk (0..3) of each X load
  uint32_t w_off[kXJ];    // KN: offset within the stage's depth rows; NK: like x_off
  uint32_t w_kchunk[kXJ];
  uint32_t w_col[kXJ];    // KN: first feature, within the tile, of this lane's chunk
  const uint16_t* xbase;
  const uint16_t* wbase;
  int M, N, K, KT;          // KT: depth steps
  uint32_t xr_off;          // operand read offsets within a slot: X block 0
  uint32_t wr_off[2];       // W block 0 (KN: the two transposed halves)

  // Everything that does not depend on the output tile; tid is the thread index.
  __device__ __forceinline__ void init(const GemmProblem& p, int tid) {
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    wave_u = (uint32_t)wave;
    M = p.M;
    N = p.N;
    K = p.K;
    KT = (K + kBK - 1) / kBK;
    xbase = p.x;
    wbase = p.w;
    const uint32_t kb = (uint32_t)K * 2u;
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
        w_col[j] = 8u * wc;
        w_off[j] = ((uint32_t)wrow * (uint32_t)N + 8u * wc) * 2u;
        w_kchunk[j] = (uint32_t)wrow;
      } else {
        w_off[j] = x_off[j];
        w_kchunk[j] = c;
        w_col[j] = 0u;
      }
    }
    // operand lane l: row l % 16 of its block, depth 8 (l / 16) .. +7 of the step
    const int r16 = lane & 15, g = lane >> 4;
    xr_off = krow_off(wm * 128 + r16, g);
    if constexpr (kWKN) {
      // transposed read: in each 16-lane group, lane 4e+q points at depth row e of the
      // group's 4 rows, features 4q..4q+3; lane i receives feature i of all 4 rows.
      // Block i's chunk is that of block 0 OR 2 i (bits 1, 2 of block 0's chunk are
      // clear), so its offset is block 0's XOR 32 i: no bits of the row, the half-chunk
      // or the tile base carry into bits 5, 6.
      const int e = r16 >> 2, q = r16 & 3;
      const int nb = wn * kWaveN + 4 * q;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g + 4 * h + e;
        wr_off[h] = kTileBytes + nrow_off(row, nb >> 3) + (uint32_t)((nb >> 2) & 1) * 8u;
      }
    } else {
      // NK-W rows are features: block i is 16 rows (1 KiB) on, and the swizzle uses only
      // row bit 3
      wr_off[0] = kTileBytes + krow_off(wn * kWaveN + r16, g);
      wr_off[1] = 0;
    }
  }

  // Sources of tile number t at (m0, n0).
  __device__ __forceinline__ TileSrc src(int t, int m0, int n0) const {
    TileSrc s;
    const uint32_t kb = (uint32_t)K * 2u;
    s.xrs = rsrc_words(xbase + (size_t)m0 * K, (uint32_t)min(kBM, M - m0) * kb);
    if constexpr (kWOneDesc)
      s.wrs = rsrc_words(wbase + n0, ((uint32_t)K * (uint32_t)N - (uint32_t)n0) * 2u);
    else
      s.wrs = kWKN ? rsrc_words(wbase, 0u) : rsrc_words(wbase + (size_t)n0 * K, (uint32_t)min(kBN, N - n0) * kb);
    s.n0 = n0;
    s.kstart = k_rotation(t, KT);
#pragma unroll
    for (int j = 0; j < kXJ; ++j) s.w_col_ok[j] = !kWKN || n0 + (int)w_col[j] < N;
    return s;
  }

  // DMA load number j (0 .. kLoadsPerStep-1) of the tile's kt-th depth step (rotated)
  // into `slot`. Steps past the end (kt >= KT) issue out-of-range loads that only
  // zero-fill a slot nobody reads.
  __device__ __forceinline__ void issue_one(const TileSrc& s, char* slot, int kt, int j) const {
    const int ksr = kt + s.kstart;
    const int k0 = (kt >= KT) ? K : (ksr >= KT ? ksr - KT : ksr) * kBK;
    if (j < kXJ) {
      const uint32_t xs = lds_addr(slot) + wave_u * (kXJ * 1024u);
      const bool ok = k0 + 8 * (int)x_kchunk[j] < K;
      dma16(s.xrs, xs + j * 1024u, ok ? x_off[j] + (uint32_t)k0 * 2u : kOutOfRange);
    } else {
      const int jj = j - kXJ;
      const uint32_t ws = lds_addr(slot) + (uint32_t)kTileBytes + wave_u * (kXJ * 1024u);
      if constexpr (kWOneDesc) {
        dma16(s.wrs, ws + jj * 1024u, s.w_col_ok[jj] ? (uint32_t)k0 * (uint32_t)N * 2u + w_off[jj] : kOutOfRange);
      } else if constexpr (kWKN) {
        const int krows = max(0, min(kBK, K - k0));
        const i32x4_t wrs = rsrc_words(wbase + (size_t)min(k0, K - 1) * N + s.n0,
                                       krows ? ((uint32_t)krows * (uint32_t)N - (uint32_t)s.n0) * 2u : 0u);
        dma16(wrs, ws + jj * 1024u, s.w_col_ok[jj] ? w_off[jj] : kOutOfRange);
      } else {
        const bool ok = k0 + 8 * (int)w_kchunk[jj] < K;
        dma16(s.wrs, ws + jj * 1024u, ok ? w_off[jj] + (uint32_t)k0 * 2u : kOutOfRange);
      }
    }
  }

  // Opaque, wave-uniform slot base: keeps the compiler from hoisting one address
  // register per (slot, read) out of the loop.
  __device__ __forceinline__ static uint32_t opaque_base(const char* slot) {
    uint32_t base = lds_addr(slot);
    asm volatile("" : "+s"(base));
    return base;
  }
  // X operand block j (16 tokens) of a slot
  __device__ __forceinline__ bf16x8_t read_x(const char* slot, int j) const {
    return *(lds_b128_ptr)(uintptr_t)(opaque_base(slot) + xr_off + (uint32_t)j * 16u * 64u);
  }
  // W operand block i (16 features) of a slot
  __device__ __forceinline__ bf16x8_t read_w(const char* slot, int i) const {
    const uint32_t base = opaque_base(slot);
    if constexpr (kWKN) {
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_ptr)(uintptr_t)(base + (wr_off[0] ^ (32u * i))));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_ptr)(uintptr_t)(base + (wr_off[1] ^ (32u * i))));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *(lds_b128_ptr)(uintptr_t)(base + wr_off[0] + (uint32_t)i * 16u * 64u);
    }
  }
};

// Field-wise choice between two tiles' sources on a wave-uniform condition (kept in
// registers; a reference chosen at run time would put both structs in scratch memory).
__device__ __forceinline__ TileSrc pick(bool second, const TileSrc& a, const TileSrc& b) {
  TileSrc s;
  s.xrs.x = second ? b.xrs.x : a.xrs.x;
  s.xrs.y = second ? b.xrs.y : a.xrs.y;
  s.xrs.z = second ? b.xrs.z : a.xrs.z;
  s.xrs.w = second ? b.xrs.w : a.xrs.w;
  s.wrs.x = second ? b.wrs.x : a.wrs.x;
  s.wrs.y = second ? b.wrs.y : a.wrs.y;
  s.wrs.z = second ? b.wrs.z : a.wrs.z;
  s.wrs.w = second ? b.wrs.w : a.wrs.w;
  s.n0 = second ? b.n0 : a.n0;
  s.kstart = second ? b.kstart : a.kstart;
#pragma unroll
  for (int j = 0; j < kXJ; ++j) s.w_col_ok[j] = second ? b.w_col_ok[j] : a.w_col_ok[j];
  return s;
}

// X loads of depth steps kk (into slot a) and kk + 1 (slot b), row halves back to back.
template <class ML>
__device__ __forceinline__ void issue_x_pair(const ML& ml, const TileSrc& src, char* a, char* b, int kk) {
  ml.issue_one(src, a, kk, 0);
  ml.issue_one(src, b, kk + 1, 0);
  ml.issue_one(src, a, kk, 1);
  ml.issue_one(src, b, kk + 1, 1);
}

// Prologue: the loads the schedule would issue in its steps -3, -2, -1 (W of 0; X of 0
// and 1; W of 1; W of 2; X of 2 and 3), so that the loop's wait counts hold from step 0
// on; wait for step 0.
template <class ML>
__device__ __forceinline__ void mainloop_prologue(const ML& ml, const TileSrc& src, const LdsRing& lds) {
  ml.issue_one(src, lds.slot[0], 0, 2);
  ml.issue_one(src, lds.slot[0], 0, 3);
  issue_x_pair(ml, src, lds.slot[0], lds.slot[1], 0);
  ml.issue_one(src, lds.slot[1], 1, 2);
  ml.issue_one(src, lds.slot[1], 1, 3);
  ml.issue_one(src, lds.slot[2], 2, 2);
  ml.issue_one(src, lds.slot[2], 2, 3);
  issue_x_pair(ml, src, lds.slot[2], lds.slot[3], 2);
  wait_vmcnt<9>();  // 9 loads were issued after step 0's last one
  __builtin_amdgcn_s_barrier();
}

// Depth steps of the next tile that a persistent workgroup loads during the last steps
// of the current one (into the slots the current tile has finished with); the other
// three slots hold the epilogue's staging and row-exchange areas meanwhile.
constexpr int kNextSteps = 2;

// Start of a persistent workgroup's next tile, after its epilogue and a barrier: steps
// 0 and 1 are already in LDS; put the loads of step -1 (W of 2; X of 2 and 3) in flight.
template <class ML>
__device__ __forceinline__ void mainloop_resume(const ML& ml, const TileSrc& src, const LdsRing& lds) {
  ml.issue_one(src, lds.slot[2], 2, 2);
  ml.issue_one(src, lds.slot[2], 2, 3);
  issue_x_pair(ml, src, lds.slot[2], lds.slot[3], 2);
}

// The depth loop of one tile, after its prologue (or resume), over `steps` depth steps
// from the tile's first one (all of its ml.KT steps, or a slice of them in the split-depth
// schedule). With kPersist and a next tile, the loads of steps KT and KT+1 of the
// schedule are that tile's steps 0 and 1 (this needs KT >= 4, so that all of them fall
// inside this loop); otherwise loads past the end zero-fill free slots (or, past the end
// of a slice, load depth steps nobody reads). Returns once every load has landed and
// every wave is done reading operands.
template <bool kPersist, class ML>
__device__ __forceinline__ void mainloop_body(const ML& ml, const TileSrc& cur, const TileSrc& nxt,
                                              bool has_next, const LdsRing& lds, AccTile& acc, int steps) {
  constexpr bool kWKN = ML::kKN;
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = steps;
  constexpr int kH = kMJ / 2;                           // token blocks per half step
  constexpr int kMfmaH = kNI * kH;                      // MFMAs per half step

  // load j of schedule step kk: in a tail step (kTail) of a persistent workgroup it may
  // be a step of the next tile; elsewhere it is this tile's (or a zero fill)
  auto issue_at = [&](char* slot, int kk, int j, auto tail) {
    if constexpr (kPersist && decltype(tail)::value) {
      const bool nx = has_next && kk >= KT && kk < KT + kNextSteps;
      ml.issue_one(pick(nx, cur, nxt), slot, nx ? kk - KT : kk, j);
    } else {
      ml.issue_one(cur, slot, kk, j);
    }
  };
  const std::false_type steady, even;
  const std::true_type tail, odd;

  bf16x8_t a[kNI], b[kMJ];
#pragma unroll
  for (int i = 0; i < kNI; ++i) a[i] = ml.read_w(lds.slot[0], i);
#pragma unroll
  for (int j = 0; j < kH; ++j) b[j] = ml.read_x(lds.slot[0], j);

  // Step kt (ring slot S = kt mod 5). Loads: W of kt+3 each step; X of kt+3 and kt+4 on
  // odd steps. Issue order over the steps makes 8 loads follow the last one of step
  // kt+1 at an even step's wait, 5 at an odd step's. Every operand read lands in the
  // registers of a block no MFMA needs any more (X blocks 4..7 of this step in those of
  // the last step's, X blocks 0..3 of the next step in those of this step's, W block i
  // of the next step right after this step's last MFMA on W block i), so the operands
  // take 12 registers of 8 bf16, as many as the blocks in use.
  auto step = [&](const int S, const int kt, auto parity, auto kind) {
    constexpr bool kOdd = decltype(parity)::value;
#pragma unroll
    for (int j = kH; j < kMJ; ++j) b[j] = ml.read_x(lds.slot[S], j);
    // two waves share each SIMD: the one in its first-half MFMA run (and W issue) wins
    // issue arbitration over the other's reads and waits
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
      for (int j = 0; j < kH; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kH, 0);      // second-half X reads first
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaH, 0);  // then the first-half MFMAs
    // W half of step kt+3 into the slot of kt-2 (free since the previous barrier)
    issue_at(lds.slot[(S + 3) % kStages], kt + 3, 2, kind);
    issue_at(lds.slot[(S + 3) % kStages], kt + 3, 3, kind);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kOdd)
      wait_vmcnt<5>();  // this thread's loads of step kt+1 have landed
    else
      wait_vmcnt<8>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const char* next = lds.slot[(S + 1) % kStages];
#pragma unroll
    for (int r = 0; r < kMfmaH; ++r) {
      const int i = r / kH, j = kH + r % kH;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      // odd steps: X of kt+3 and kt+4 into the slots of kt-2 and kt-1 (free since the
      // previous barrier and this one), the two halves of each row back to back, one
      // load behind every other MFMA of the run's second half. A DMA issue stalls its wave
      // while the texture unit's command queue is full; issued late in the run the stall
      // falls where the wave has MFMAs queued and a wait ahead, not in front of 12 of them
      // (measured on MI355X against the loads behind the run's first four MFMAs,
      // interleaved, bit-identical: 2-4% faster on GEMM1, GEMM2, 8192^3 and the NK backward).
      // The persistent kernel keeps them behind the first four MFMAs: it holds the next
      // tile's sources across its loop, and with the loads that late the loop needs more
      // than its 256 registers (203 VGPRs spilled). Either way the loads come after the
      // step's barrier and before the next wait, so the ring's wait counts hold.
      constexpr int kX0 = kPersist ? 0 : kMfmaH - 8, kXStride = kPersist ? 1 : 2;
      if (kOdd && r >= kX0 && (r - kX0) % kXStride == 0 && (r - kX0) / kXStride < 4) {
        const int q = (r - kX0) / kXStride;
        issue_at(lds.slot[(S + 3 + (q & 1)) % kStages], kt + 3 + (q & 1), q >> 1, kind);
      }
      if (r < kH) {
        b[r] = ml.read_x(next, r);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      if (r % kH == kH - 1) {  // the last MFMA on W block i
        a[i] = ml.read_w(next, i);
        __builtin_amdgcn_sched_group_barrier(0x100, kWKN ? 2 : 1, 1);
      }
    }
    // nothing moves across steps: an operand read pulled ahead of the MFMAs still using
    // the registers it lands in would need registers of its own
    __builtin_amdgcn_sched_barrier(0);
  };

  int kt = 0;
  // ten steps per round: ring slot and parity both repeat. A persistent workgroup
  // leaves the last 4 to 13 steps, whose loads reach past this tile, to the tail.
  constexpr int kLook = kPersist ? 4 : 0;
  for (; kt + 2 * kStages + kLook <= KT; kt += 2 * kStages) {
    step(0, kt, even, steady);
    step(1, kt + 1, odd, steady);
    step(2, kt + 2, even, steady);
    step(3, kt + 3, odd, steady);
    step(4, kt + 4, even, steady);
    step(0, kt + 5, odd, steady);
    step(1, kt + 6, even, steady);
    step(2, kt + 7, odd, steady);
    step(3, kt + 8, even, steady);
    step(4, kt + 9, odd, steady);
  }
  // (each step its own block: as one straight block the tail does not fit the
  // register budget)
  auto rest = [&](auto kind) {
    if (kt < KT) step(0, kt, even, kind);
    if (kt + 1 < KT) step(1, kt + 1, odd, kind);
    if (kt + 2 < KT) step(2, kt + 2, even, kind);
    if (kt + 3 < KT) step(3, kt + 3, odd, kind);
    if (kt + 4 < KT) step(4, kt + 4, even, kind);
    if (kt + 5 < KT) step(0, kt + 5, odd, kind);
    if (kt + 6 < KT) step(1, kt + 6, even, kind);
    if (kt + 7 < KT) step(2, kt + 7, odd, kind);
    if (kt + 8 < KT) step(3, kt + 8, even, kind);
    if (kPersist && kt + 9 < KT) step(4, kt + 9, odd, kind);
    if (kPersist && kt + 10 < KT) step(0, kt + 10, even, kind);
    if (kPersist && kt + 11 < KT) step(1, kt + 11, odd, kind);
    if (kPersist && kt + 12 < KT) step(2, kt + 12, even, kind);
  };
  if constexpr (kPersist)
    rest(tail);
  else
    rest(steady);
  wait_vmcnt<0>();  // zero-fill loads (and the next tile's first steps) have landed
  __syncthreads();  // all operand reads are done before the free slots hold epilogue data
}

// The LDS of one workgroup as a ring whose logical slot s is physical slot
// (s + rot) mod 5, with the epilogue's areas in the three physical slots from e on
// (mod 5): staging of waves 0-3, staging of waves 4-7, row exchange.
__device__ __forceinline__ char* phys_slot(char* smem, int i) {
  return smem + (i >= kStages ? i - kStages : i) * kSlotBytes;
}
__device__ __forceinline__ LdsRing make_ring(char* smem, int rot, int e, int tid) {
  LdsRing r;
  r.tid = tid;
#pragma unroll
  for (int s = 0; s < kStages; ++s) r.slot[s] = phys_slot(smem, s + rot);
  r.stg[0] = phys_slot(smem, e);
  r.stg[1] = phys_slot(smem, e + 1);
  r.red = (float*)phys_slot(smem, e + 2);
  return r;
}

// ------------------------------------------------------------------------------------
// Epilogue. Accumulator block acc[i][j] of a lane covers features
//   n = n0 + wn*64 + 16 i + 4 (lane >> 4) + v  (register v = 0..3)
// for the token m = m0 + wm*128 + 16 j + (lane & 15): one lane spans 16 tokens of each
// feature run, which makes direct loads of per-element side inputs 8-byte gathers from
// 16 rows. So each wave first re-lays its 128 x 64 fp32 block out row-major through a
// private 8 KiB LDS area (32 tokens at a time) and then walks it with 16 lanes per
// token, 4 features per lane: side inputs (residual, gamma, rotary tables, saved activations) are read and
// outputs written as whole 128-byte row segments, and a row statistic is a 16-lane
// reduction. No barrier is needed between a wave's own staging writes and reads (one
// wave's LDS operations complete in order); the only workgroup barrier after the main
// loop is the one that combines the row statistics of the four feature-waves.
struct EpiLane {
  int lane, wave, wm, wn, m0, n0;
  __device__ __forceinline__ EpiLane(int m0_, int n0_, int tid)
      : lane(tid & 63), wave(tid >> 6), wm((tid >> 6) / kWavesN), wn((tid >> 6) % kWavesN), m0(m0_), n0(n0_) {}
  // first of the 4 features this lane holds in the row-major walk
  __device__ __forceinline__ int col4() const { return n0 + wn * kWaveN + 4 * (lane & 15); }
  // token of wave-local row r (0..127)
  __device__ __forceinline__ int token(int r) const { return m0 + wm * 128 + r; }
};

typedef __attribute__((address_space(3))) f32x4_t* lds_f32x4_ptr;

// Staging address of (row r in 0..31, 16-byte chunk c in 0..15), rows of 256 bytes.
// The accumulator writes put 8 consecutive rows at one chunk into each 8-lane group
// (gfx950 serves ds_write_b128 8 lanes at a time over 32 banks), so XOR-ing the chunk
// with r mod 8 makes them distinct; the row-major reads give rows r and r + 8 to the
// two halves of a 16-lane read group (see swz_k), which share that XOR and so take the
// two complementary halves of the banks.
__device__ __forceinline__ uint32_t stg_off(int r, int c) {
  return ((uint32_t)r << 8) | ((uint32_t)(c ^ (r & 7)) << 4);
}

__device__ __forceinline__ char* stage_base(const LdsRing& lds, int wave) {
  return (wave < 4 ? lds.stg[0] : lds.stg[1]) + (wave & 3) * kStgWaveBytes;
}

// Walk a wave's accumulators row-major: op.row(r, v, pre) gets wave-local row r
// (0..127), this lane's 4 fp32 values at features col4() .. col4() + 3, and what
// op.fetch(r) loaded for that row; it returns the row's statistic (kRowStat) and, for
// ops with kColStat, adds its per-feature contribution into a column accumulator kept
// here (returned: the sum over this lane's 32 rows). Side inputs are fetched one block
// (8 rows per lane) ahead of the block being walked, which bounds the registers they
// hold while the accumulators are still live; a row's loads are issued before the output
// stores that precede its use, so none queues behind them (the vector-memory counter
// waits on stores and loads alike).

// Type of an op's row statistic: Op::Stat if it declares one, else float.
template <class Op, class = void>
struct StatOf {
  typedef float type;
};
template <class Op>
struct StatOf<Op, std::void_t<typename Op::Stat>> {
  typedef typename Op::Stat type;
};

template <class Op>
__device__ __forceinline__ f32x4_t epilogue_rows(AccTile& acc, const LdsRing& lds, const EpiLane& L, Op& op) {
  f32x4_t col = {0.f, 0.f, 0.f, 0.f};  // column statistic of ops with kColStat (sum over this lane's rows)
  const uint32_t sb = lds_addr(stage_base(lds, L.wave));
  const int cq = L.lane & 15, rq = L.lane >> 4;
  typedef typename Op::Pre Pre;
  typedef typename StatOf<Op>::type Stat;
  // stage token blocks 2J, 2J + 1 (32 tokens) at staging rows 0 .. 31
  auto stage = [&](int J) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < kNI; ++i)
        *(lds_f32x4_ptr)(uintptr_t)(sb + stg_off(16 * h + (L.lane & 15), 4 * i + (L.lane >> 4))) = acc[i][2 * J + h];
  };
  // rows row0 + 8 rq + it (it = 0..7) of the staging area are wave rows r0 + 8 rq + it
  auto walk8 = [&](int row0, int r0, const Pre (&pre)[8], Stat (&stat)[8]) {
    constexpr int kRd = sizeof(Pre) <= 8 ? 8 : 4;  // rows whose LDS reads are in flight together
#pragma unroll
    for (int b = 0; b < 8 / kRd; ++b) {
      f32x4_t v[kRd];
#pragma unroll
      for (int q = 0; q < kRd; ++q) v[q] = *(lds_f32x4_ptr)(uintptr_t)(sb + stg_off(row0 + 8 * rq + kRd * b + q, cq));
#pragma unroll
      for (int q = 0; q < kRd; ++q) {
        const int r = r0 + 8 * rq + kRd * b + q;
        if constexpr (Op::kColStat)
          stat[kRd * b + q] = op.row(r, v[q], pre[kRd * b + q], col);
        else
          stat[kRd * b + q] = op.row(r, v[q], pre[kRd * b + q]);
      }
    }
  };
  auto record = [&](int r0, const Stat (&stat)[8]) {
    if constexpr (Op::kRowStat) {
      // lane 0 of each 16-lane row group records the wave's statistic of its rows
      if (cq == 0) {
        Stat* red = (Stat*)lds.red + (L.wm * kWavesN + L.wn) * 128 + r0 + 8 * rq;
#pragma unroll
        for (int it = 0; it < 8; ++it) red[it] = stat[it];
      }
    }
  };
  // blocks of 32 tokens, each staged on its own; the next block's side-input loads are
  // issued before this block's stores and are in flight while it is walked
  Pre pre[2][8];
#pragma unroll
  for (int it = 0; it < 8; ++it) pre[0][it] = op.fetch(8 * rq + it);
  constexpr int kBlocks = 128 / kStgRows;
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) {
    stage(j);
    if (j + 1 < kBlocks) {
#pragma unroll
      for (int it = 0; it < 8; ++it) pre[(j + 1) & 1][it] = op.fetch(32 * (j + 1) + 8 * rq + it);
    }
    Stat stat[8];
    walk8(0, 32 * j, pre[j & 1], stat);
    record(32 * j, stat);
  }
  return col;
}

struct NoPre {};

// Sum over the 16 lanes of a DPP row (fixed order: lane pairs, quads, halves, rows);
// every lane of the row gets the total.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Row statistic: op.row returns its row's total over the wave's 64 features (sum16),
// which epilogue_rows records per (wave, row); after all waves have done so, the
// tile's value per token is the sum over the four feature-waves wn = 0, 1, 2, 3 in that
// order, stored at partials[m * nb + tile].
__device__ __forceinline__ void store_row_partials(const LdsRing& lds, const EpiLane& L, float* __restrict__ partials,
                                                   int nb, int M) {
  __syncthreads();
  const int t = lds.tid;
  if (t < kBM) {
    const int wm = t >> 7, r = t & 127;
    const int m = L.m0 + t;
    const float* red = lds.red + wm * kWavesN * 128 + r;
    const float s = ((red[0] + red[128]) + red[256]) + red[384];
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

// Side inputs of the row-major walk are read through raw buffer descriptors over the
// wave's own 128 rows: rows past M fall outside the range and read as zero, and a lane
// whose features lie past the width uses an out-of-range offset, so the loads need no
// branches (branch-wrapped loads leave the compiler only full vector-memory waits).
struct WaveRowsBf16 {  // [M, ld] bf16, this lane's 4 features at column n
  __amdgpu_buffer_rsrc_t rs;
  uint32_t pitch, coff;
  __device__ __forceinline__ WaveRowsBf16(const uint16_t* base, const EpiLane& L, int M, int ld, int n, bool nok) {
    const int r0 = L.m0 + L.wm * 128;
    const int rows = base ? max(0, min(128, M - r0)) : 0;  // 128 * 2^22 * 2 bytes < 2^31
    rs = make_rsrc(base ? base + (size_t)max(r0, 0) * ld : base, (uint32_t)rows * (uint32_t)ld * 2u);
    pitch = (uint32_t)ld * 2u;
    coff = nok ? (uint32_t)n * 2u : kOutOfRange;
  }
  __device__ __forceinline__ u32x2_t load4(int r) const {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, coff == kOutOfRange ? kOutOfRange : (uint32_t)r * pitch + coff, 0,
                                                0);
  }
  __device__ __forceinline__ u32x4_t load8(int r) const {  // 8 features starting at column n
    return __builtin_amdgcn_raw_buffer_load_b128(rs, coff == kOutOfRange ? kOutOfRange : (uint32_t)r * pitch + coff,
                                                 0, 0);
  }
};
struct WaveRowsF32 {  // [M] fp32, one value per row
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ WaveRowsF32(const float* base, const EpiLane& L, int M) {
    const int r0 = L.m0 + L.wm * 128;
    const int rows = base ? max(0, min(128, M - r0)) : 0;
    rs = make_rsrc(base ? base + max(r0, 0) : base, (uint32_t)rows * 4u);
  }
  __device__ __forceinline__ float load(int r) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)r * 4u, 0, 0));
  }
};
// Output rows of the wave's 128 tokens in an [M, ld] bf16 array, through a raw buffer
// descriptor: rows past M lie outside its range, and a lane whose features lie past the
// width starts from an out-of-range column offset (2^31; adding a row offset below 2^30
// keeps it out of every range), so those stores are dropped by the hardware and the
// stores need no branch. Outputs of the same shape share one row offset (row_off).
// The stores are non-temporal (cache policy nt): a tile's outputs are not read again by
// this kernel, and streaming them keeps the operand panels that other tiles still read
// in L2 and the Infinity Cache (measured on MI355X: GEMM1 -1.8% / -2.3% time, GEMM2
// -1.2% / -0.4%, interleaved against normal stores on two boxes).
struct WaveRowsOutBf16 {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t pitch, coff;
  __device__ __forceinline__ WaveRowsOutBf16(uint16_t* base, const EpiLane& L, int M, int ld, int n, bool nok) {
    const int r0 = L.m0 + L.wm * 128;
    const int rows = max(0, min(128, M - r0));  // 128 * 2^22 * 2 bytes < 2^31
    rs = make_rsrc(base + (size_t)max(r0, 0) * ld, (uint32_t)rows * (uint32_t)ld * 2u);
    pitch = (uint32_t)ld * 2u;
    coff = nok ? (uint32_t)n * 2u : kOutOfRange;
  }
  __device__ __forceinline__ uint32_t row_off(int r) const { return coff + (uint32_t)r * pitch; }
  // bf16 of (a, b, c, d) at byte offset `off` (row_off of this or a same-shaped output)
  __device__ __forceinline__ void store4_at(uint32_t off, float a, float b, float c, float d) const {
    u32x2_t v;
    v.x = pack_bf16x2(a, b);
    v.y = pack_bf16x2(c, d);
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, kCachePolicyNT);
  }
  __device__ __forceinline__ void store4(int r, float a, float b, float c, float d) const {
    store4_at(row_off(r), a, b, c, d);
  }
  // bf16 of (a, b) at byte offset `off`
  __device__ __forceinline__ void store2_at(uint32_t off, float a, float b) const {
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a, b), rs, off, 0, kCachePolicyNT);
  }
  // 16 bytes (8 bf16, already packed) at byte offset `off`
  __device__ __forceinline__ void store8_at(uint32_t off, const u32x4_t& v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, kCachePolicyNT);
  }
};

__device__ __forceinline__ void store_bf16x4(uint16_t* __restrict__ base, size_t idx, float a, float b, float c,
                                             float d) {
  u32x2_t v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  __builtin_nontemporal_store(v, (u32x2_t*)(base + idx));
}

// ---------------------------------------------------------------- plain store (baseline)
struct EpiStore {
  struct Args {
    uint16_t* out;
  };
  struct Op {
    WaveRowsOutBf16 out;
    static constexpr bool kRowStat = false;
    static constexpr bool kColStat = false;
    typedef NoPre Pre;
    __device__ __forceinline__ Pre fetch(int) const { return Pre{}; }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre&) {
      out.store4(r, v.x, v.y, v.z, v.w);
      return 0.f;
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    Op op{WaveRowsOutBf16(a.out, L, p.M, p.N, n, n < p.N)};
    epilogue_rows(acc, lds, L, op);
  }
};

// ------------------------------------- GEMM1: residual + gamma side output + partials
// h1 = acc + z (stored), h2 = h1 * gamma (stored), P[m, tile] = sum h1^2 over the tile
// (the fp32 h1, before rounding to bf16).
struct EpiResidualRmsPartials {
  struct Args {
    const uint16_t* z;
    const uint16_t* gamma;
    uint16_t* h1;
    uint16_t* h2;
    float* partials;
    int nb;
  };
  struct Op {
    float g0, g1, g2, g3;
    WaveRowsBf16 z;
    WaveRowsOutBf16 h1o, h2o;
    static constexpr bool kRowStat = true;
    static constexpr bool kColStat = false;
    typedef u32x2_t Pre;
    __device__ __forceinline__ Pre fetch(int r) const { return z.load4(r); }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre& zz) {
      const float h0 = v.x + bf16_lo(zz.x), h1 = v.y + bf16_hi(zz.x);
      const float h2 = v.z + bf16_lo(zz.y), h3 = v.w + bf16_hi(zz.y);
      const uint32_t off = h1o.row_off(r);  // h1 and h2 have the same shape
      h1o.store4_at(off, h0, h1, h2, h3);
      h2o.store4_at(off, h0 * g0, h1 * g1, h2 * g2, h3 * g3);
      return sum16((h0 * h0 + h1 * h1) + (h2 * h2 + h3 * h3));
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    const bool nok = n < p.N;
    const u32x2_t gg = load_bf16x4(a.gamma, (size_t)n, nok);
    Op op{bf16_lo(gg.x), bf16_hi(gg.x), bf16_lo(gg.y), bf16_hi(gg.y), WaveRowsBf16(a.z, L, p.M, p.N, n, nok),
          WaveRowsOutBf16(a.h1, L, p.M, p.N, n, nok), WaveRowsOutBf16(a.h2, L, p.M, p.N, n, nok)};
    epilogue_rows(acc, lds, L, op);
    store_row_partials(lds, L, a.partials, a.nb, p.M);
  }
};

// ------------------------------------------------ GEMM2: deferred row scale y = r[m] acc
struct EpiRowScale {
  struct Args {
    const float* r;
    uint16_t* y;
  };
  struct Op {
    WaveRowsF32 rv;
    WaveRowsOutBf16 out;
    static constexpr bool kRowStat = false;
    static constexpr bool kColStat = false;
    typedef float Pre;
    __device__ __forceinline__ Pre fetch(int r) const { return rv.load(r); }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre& s) {
      out.store4(r, s * v.x, s * v.y, s * v.z, s * v.w);
      return 0.f;
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    Op op{WaveRowsF32(a.r, L, p.M), WaveRowsOutBf16(a.y, L, p.M, p.N, n, n < p.N)};
    epilogue_rows(acc, lds, L, op);
  }
};

// ------------------------------------------------------- QKV projection + RoPE on Q, K
// A lane's 4 features are two (even, odd) pairs of one head (4 | head_dim), rotated by
// the angles of pair indices pp, pp + 1 at the token's position. With `inverse` set the
// rotation is by the negated angle: the RoPE backward, applied in the epilogue of the
// GEMM that produces the gradient of the rotated Q and K.
struct EpiRope {
  struct Args {
    const float* cos_t;
    const float* sin_t;
    uint16_t* out;
    int n_rot;  // n_q + n_k: columns [0, n_rot) are rotated
    int head_dim;
    int seq_len;
    int pos_offset;
    int inverse;  // 0: forward rotation, 1: rotation by the negated angle
  };
  // kShort: seq_len < 128, so a wave's 128 rows may wrap the position more than once.
  template <bool kShort>
  struct Op {
    const EpiLane& L;
    const Args& a;
    __amdgpu_buffer_rsrc_t ct, st;  // the cos and sin tables, [seq_len, head_dim / 2] fp32
    WaveRowsOutBf16 out;
    int half, pp, pos0;
    bool rot;
    static constexpr bool kRowStat = false;
    static constexpr bool kColStat = false;
    struct Pre {
      float2 c, s;
    };
    __device__ __forceinline__ Pre fetch(int r) const {
      // (m + pos_offset) mod seq_len for wave row r: pos0 + r < pos0 + 128, so one
      // subtraction wraps it when seq_len >= 128. Every lane and row reads a valid table
      // entry (also rows past M and unrotated columns, whose values are not used).
      int pos = pos0 + r;
      if constexpr (kShort) {
        pos %= a.seq_len;
      } else {
        pos = pos >= a.seq_len ? pos - a.seq_len : pos;
      }
      const uint32_t off = (uint32_t)(pos * half + pp) * 4u;
      Pre t;
      t.c = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ct, off, 0, 0));
      t.s = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(st, off, 0, 0));
      return t;
    }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre& t) {
      const float2 c = t.c;
      const float2 s = a.inverse ? make_float2(-t.s.x, -t.s.y) : t.s;
      const float re0 = v.x * c.x - v.y * s.x, ro0 = v.x * s.x + v.y * c.x;
      const float re1 = v.z * c.y - v.w * s.y, ro1 = v.z * s.y + v.w * c.y;
      out.store4(r, rot ? re0 : v.x, rot ? ro0 : v.y, rot ? re1 : v.z, rot ? ro1 : v.w);
      return 0.f;
    }
  };
  template <bool kShort>
  __device__ __forceinline__ static void run(AccTile& acc, const Args& a, const GemmProblem& p, const EpiLane& L,
                                             const LdsRing& lds) {
    const int n = L.col4();
    const int half = a.head_dim >> 1;
    const int pos0 = (int)(((long long)L.token(0) + a.pos_offset) % a.seq_len);
    const uint32_t tbytes = (uint32_t)a.seq_len * (uint32_t)half * 4u;
    Op<kShort> op{L, a, make_rsrc(a.cos_t, tbytes), make_rsrc(a.sin_t, tbytes),
                  WaveRowsOutBf16(a.out, L, p.M, p.N, n, n < p.N), half, (n % a.head_dim) >> 1, pos0, n < a.n_rot};
    epilogue_rows(acc, lds, L, op);
  }
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    if (a.seq_len >= 128)
      run<false>(acc, a, p, L, lds);
    else
      run<true>(acc, a, p, L, lds);
  }
};

// ---------------------------------------------- SwiGLU: out[m, j] = silu(G_j) * U_j
// sigmoid(g) = 1 / (1 + e^-g) through the hardware reciprocal (about 1 ulp, far below the
// bf16 rounding of the output); g -> -inf gives rcp(inf) = 0 exactly.
__device__ __forceinline__ float sigmoid_f32(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f32(float g) { return g * sigmoid_f32(g); }

struct EpiSwiGLU {
  struct Args {
    uint16_t* out;
    int F;  // output width (= N / 2)
  };
  struct Op {
    WaveRowsOutBf16 out;  // [M, F]: this lane's two outputs at column n / 2
    static constexpr bool kRowStat = false;
    static constexpr bool kColStat = false;
    typedef NoPre Pre;
    __device__ __forceinline__ Pre fetch(int) const { return Pre{}; }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre&) {
      out.store2_at(out.row_off(r), silu_f32(v.x) * v.y, silu_f32(v.z) * v.w);
      return 0.f;
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    Op op{WaveRowsOutBf16(a.out, L, p.M, a.F, n >> 1, n < p.N)};
    epilogue_rows(acc, lds, L, op);
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
  struct Op {
    WaveRowsBf16 hv;      // h2, this lane's 4 features (rows past M and features past N read zero)
    WaveRowsOutBf16 dho;  // dh2, same positions (those stores are dropped)
    static constexpr bool kRowStat = true;
    static constexpr bool kColStat = false;
    typedef u32x2_t Pre;
    __device__ __forceinline__ Pre fetch(int r) const { return hv.load4(r); }
    __device__ __forceinline__ float row(int r, const f32x4_t& v, const Pre& hh) {
      const float d = (v.x * bf16_lo(hh.x) + v.y * bf16_hi(hh.x)) + (v.z * bf16_lo(hh.y) + v.w * bf16_hi(hh.y));
      dho.store4(r, v.x, v.y, v.z, v.w);
      return sum16(d);
    }
  };
  __device__ __forceinline__ static void apply(AccTile& acc, const Args& a, const GemmProblem& p, int m0, int n0,
                                               const LdsRing& lds) {
    const EpiLane L(m0, n0, lds.tid);
    const int n = L.col4();
    Op op{WaveRowsBf16(a.h2, L, p.M, p.N, n, n < p.N), WaveRowsOutBf16(a.dh2, L, p.M, p.N, n, n < p.N)};
    epilogue_rows(acc, lds, L, op);
    store_row_partials(lds, L, a.partials, a.nb, p.M);
  }
};

__host__ __device__ inline int gemm_grid(int M, int N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

// One workgroup per output tile. kWOneDesc (KN only): the one-descriptor form of the
// W loads, for shapes where kn_one_descriptor_fits.
template <bool kWKN, class Epi, bool kWOneDesc = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_epilogue_kernel(GemmProblem p, typename Epi::Args ea) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kSlotBytes];
  const LdsRing lds = make_ring(smem, 0, 0, threadIdx.x);
  const int t = blockIdx.x;
  int m0, n0;
  tile_coords(p.M, p.N, p.K, p.group_m, t, m0, n0);
  Mainloop<kWKN, kWOneDesc> ml;
  ml.init(p, threadIdx.x);
  const TileSrc src = ml.src(t, m0, n0);
  AccTile acc;
  mainloop_prologue(ml, src, lds);
  mainloop_body<false>(ml, src, src, false, lds, acc, ml.KT);
  Epi::apply(acc, ea, p, m0, n0, lds);
}

// Persistent form: one workgroup per CU walks tiles t = blockIdx.x, + gridDim.x, ...
// (tile t stays on XCD t mod 8 when gridDim.x is a multiple of 8, as in the form
// above). The DMA ring runs on across tiles: the last steps of a tile load the first
// two depth steps of the next, whose latency the epilogue then covers, and no
// workgroup launch separates the tiles. Needs K / 32 >= 4. Results are bit-identical
// to the one-workgroup-per-tile form (same tile sums in the same order). It keeps the
// per-step KN-W descriptors: with the one-descriptor form its loop needs more than the
// 256 registers of two waves per SIMD and spills.
template <bool kWKN, class Epi>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_persistent_kernel(GemmProblem p, typename Epi::Args ea) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kSlotBytes];
  const int tiles = gemm_grid(p.M, p.N);
  const int KT = (p.K + kBK - 1) / kBK;
  const int adv = KT % kStages;  // ring advance per tile
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int t = blockIdx.x, rot = 0;
  int m0, n0;
  tile_coords(p.M, p.N, p.K, p.group_m, t, m0, n0);
  bool first = true;
  TileSrc cur;
  while (true) {
    // Every lane-dependent offset (the main loop's DMA and read offsets, the epilogue's
    // staging addresses) is rebuilt for each tile from a thread index the compiler
    // cannot hoist (the lane id from mbcnt in volatile asm): hoisted out of the tile
    // loop, they would stay live across the main loop and push it past the register
    // budget.
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    const int tid = wave * 64 + lane;
    Mainloop<kWKN> ml;
    ml.init(p, tid);
    if (first) {
      cur = ml.src(t, m0, n0);
      mainloop_prologue(ml, cur, make_ring(smem, 0, 0, tid));
      first = false;
    } else {
      mainloop_resume(ml, cur, make_ring(smem, rot, 0, tid));
    }
    const int tn = t + (int)gridDim.x;
    const bool has_next = tn < tiles;
    int mn = m0, nn = n0;
    int Mo = p.M, No = p.N;  // opaque copies: the division is redone per tile, not hoisted
    asm volatile("" : "+s"(Mo), "+s"(No));
    if (has_next) tile_coords(Mo, No, p.K, p.group_m, tn, mn, nn);
    const TileSrc nxt = ml.src(has_next ? tn : t, mn, nn);
    // the next tile's steps 0, 1 land in physical slots rot + KT, rot + KT + 1 (mod 5);
    // the epilogue takes the three after them
    int e = rot + adv + kNextSteps;  // at most 10
    e = e >= kStages ? e - kStages : e;
    e = e >= kStages ? e - kStages : e;
    const LdsRing lds = make_ring(smem, rot, e, tid);
    AccTile acc;
    mainloop_body<true>(ml, cur, nxt, has_next, lds, acc, ml.KT);
    Epi::apply(acc, ea, p, m0, n0, lds);
    if (!has_next) break;
    t = tn;
    m0 = mn;
    n0 = nn;
    cur = nxt;
    rot += adv;
    rot = rot >= kStages ? rot - kStages : rot;
    __syncthreads();  // every wave is done with the epilogue's areas before steps 2, 3 land there
  }
}

// Persistent launches need at least this many depth steps (the next tile's first two
// steps are loaded by the last four of the current one).
constexpr int kPersistMinSteps = 4;

}  // namespace coda
