// Host-side argument checks shared by the C-ABI entry points. Every check runs before
// anything is enqueued, so a failing call leaves device memory untouched.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "coda.h"

namespace coda {

constexpr int kMaxDim = 1 << 22;   // bound on K and output widths (keeps buffer ranges < 2^31)
constexpr int kMaxRows = 1 << 24;  // bound on M (with kMaxDim, fewer than 2^30 output tiles)

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline int check_depth_or_width(int v) {
  if (v < 8 || v > kMaxDim || (v % 8) != 0) return CODA_ERR_SHAPE;
  return CODA_OK;
}

inline int check_rows(int M) { return (M < 0 || M > kMaxRows) ? CODA_ERR_SHAPE : CODA_OK; }

// Byte range of one argument buffer, for the rule that output buffers overlap neither
// the inputs nor each other (a NULL or empty range overlaps nothing).
struct Span {
  const void* p;
  uint64_t bytes;
};
inline Span bf16_span(const void* p, long long rows, long long cols = 1) {
  return Span{p, (uint64_t)rows * (uint64_t)cols * 2u};
}
inline Span f32_span(const void* p, long long rows, long long cols = 1) {
  return Span{p, (uint64_t)rows * (uint64_t)cols * 4u};
}
inline bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uint64_t a0 = (uint64_t)(uintptr_t)a.p, b0 = (uint64_t)(uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}
// CODA_ERR_ARG if an output overlaps another output or an input (inputs are only read,
// so they may alias each other).
inline int check_disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (const Span* o = outs.begin(); o != outs.end(); ++o) {
    for (const Span* o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return CODA_ERR_ARG;
    for (const Span& i : ins)
      if (overlap(*o, i)) return CODA_ERR_ARG;
  }
  return CODA_OK;
}

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CODA_OK : CODA_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

#define CODA_TRY(expr)            \
  do {                            \
    const int _st = (expr);       \
    if (_st != CODA_OK) return _st; \
  } while (0)

#define CODA_NONNULL(p) \
  do {                  \
    if (!(p)) return CODA_ERR_NULL; \
  } while (0)

#define CODA_ALIGN16(p) \
  do {                  \
    if (!::coda::aligned((p), 16)) return CODA_ERR_ALIGN; \
  } while (0)

}  // namespace coda
