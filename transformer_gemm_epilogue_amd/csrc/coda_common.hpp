// Shared device helpers for the gfx950 (CDNA4) GEMM-epilogue kernels: vector types,
// raw buffer descriptors, and bf16 packing. Written for gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace coda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Word 3 of a gfx9-family raw buffer descriptor (32-bit data format, no swizzle).
constexpr uint32_t kBufferWord3 = 0x00020000u;
// A byte offset that lies beyond every buffer range built in this library (ranges are
// capped below 2^31), so a load from it returns zero and a store to it is dropped.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy operand of the buffer load/store builtins on gfx950: bit 1 is nt
// (non-temporal: stream the line, keep it from displacing reused data).
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kBufferWord3);
}

__device__ __forceinline__ u32x4_t buffer_load_16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace coda
