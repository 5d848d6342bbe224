// A consumer of libcoda.so with neither Python nor torch: device buffers from hipMalloc, the
// forward GEMM-RMSNorm-GEMM rewrite (coda_gemm_rmsnorm_fwd, its partials in a buffer of
// coda_rowstat_num_partials columns) and GEMM + SwiGLU (coda_gemm_swiglu) on the null
// stream, on bf16 inputs read from a file; the outputs are written to another file.
// tests/test_gpu_c_abi_program.py writes the inputs from the seeded workload generators,
// runs this program as a child process and checks what it wrote.
//
// usage: fwd_program <inputs> <outputs> M K D N1 eps F
// inputs: x [M,K], w0 [K,D], z [M,D], gamma [D], w1 [D,N1], then xs [M,K], ws [K,2F]
// (bf16 bits, in that order); outputs: h1, h2 [M,D] bf16, partials [M,nb] fp32,
// r [M] fp32, y [M,N1] bf16, then the SwiGLU output [M,F] bf16.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "coda.h"

#define CHECK_HIP(x)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                     \
      return 2;                                                                          \
    }                                                                                    \
  } while (0)
#define CHECK_CODA(x)                                                                    \
  do {                                                                                   \
    int s_ = (x);                                                                        \
    if (s_ != CODA_OK) {                                                                 \
      fprintf(stderr, "%s returned %d (%s)\n", #x, s_, coda_status_string(s_));          \
      return 3;                                                                          \
    }                                                                                    \
  } while (0)

namespace {

struct Buf {
  void* dev = nullptr;
  size_t bytes = 0;
};

int upload(FILE* f, size_t bytes, Buf* b) {
  std::vector<char> host(bytes);
  if (fread(host.data(), 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    return 1;
  }
  b->bytes = bytes;
  CHECK_HIP(hipMalloc(&b->dev, bytes));
  CHECK_HIP(hipMemcpy(b->dev, host.data(), bytes, hipMemcpyHostToDevice));
  return 0;
}

int download(FILE* f, const Buf& b) {
  std::vector<char> host(b.bytes);
  CHECK_HIP(hipMemcpy(host.data(), b.dev, b.bytes, hipMemcpyDeviceToHost));
  if (fwrite(host.data(), 1, b.bytes, f) != b.bytes) {
    fprintf(stderr, "short write\n");
    return 1;
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 9) {
    fprintf(stderr, "usage: %s <inputs> <outputs> M K D N1 eps F\n", argv[0]);
    return 1;
  }
  const int M = atoi(argv[3]), K = atoi(argv[4]), D = atoi(argv[5]), N1 = atoi(argv[6]);
  const float eps = (float)atof(argv[7]);
  const int F = atoi(argv[8]);
  int nb = 0;
  CHECK_CODA(coda_rowstat_num_partials(D, &nb));
  printf("coda ABI %d, M=%d K=%d D=%d N1=%d F=%d nb=%d\n", coda_abi_version(), M, K, D, N1, F, nb);
  fflush(stdout);
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 1;
  Buf x, w0, z, g, w1, xs, ws;
  const size_t b16 = 2;
  if (upload(in, (size_t)M * K * b16, &x) || upload(in, (size_t)K * D * b16, &w0) ||
      upload(in, (size_t)M * D * b16, &z) || upload(in, (size_t)D * b16, &g) ||
      upload(in, (size_t)D * N1 * b16, &w1) || upload(in, (size_t)M * K * b16, &xs) ||
      upload(in, (size_t)K * 2 * F * b16, &ws))
    return 1;
  fclose(in);
  Buf h1, h2, part, r, y, sw;
  h1.bytes = h2.bytes = (size_t)M * D * b16;
  part.bytes = (size_t)M * nb * 4;
  r.bytes = (size_t)M * 4;
  y.bytes = (size_t)M * N1 * b16;
  sw.bytes = (size_t)M * F * b16;
  for (Buf* b : {&h1, &h2, &part, &r, &y, &sw}) CHECK_HIP(hipMalloc(&b->dev, b->bytes));
  CHECK_CODA(coda_gemm_rmsnorm_fwd((const uint16_t*)x.dev, (const uint16_t*)w0.dev, (const uint16_t*)z.dev,
                                   (const uint16_t*)g.dev, (const uint16_t*)w1.dev, M, K, D, N1, eps,
                                   (uint16_t*)h1.dev, (uint16_t*)h2.dev, (float*)part.dev, (float*)r.dev,
                                   (uint16_t*)y.dev, NULL));
  CHECK_CODA(coda_gemm_swiglu((const uint16_t*)xs.dev, (const uint16_t*)ws.dev, M, K, F, (uint16_t*)sw.dev, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  FILE* out = fopen(argv[2], "wb");
  if (!out) return 1;
  for (const Buf* b : {&h1, &h2, &part, &r, &y, &sw})
    if (download(out, *b)) return 1;
  fclose(out);
  for (Buf* b : {&x, &w0, &z, &g, &w1, &xs, &ws, &h1, &h2, &part, &r, &y, &sw}) CHECK_HIP(hipFree(b->dev));
  printf("done\n");
  return 0;
}
