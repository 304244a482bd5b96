// Activations as a sum of three MX fp8 terms, for the MX-scaled expert GEMM.
//
// Each run of 32 consecutive K values of a row (one MX block) is written as
// a ~= s1*q1 + s2*q2 + s3*q3 with q_i e4m3 (OCP) bytes and s_i = 2^(e_i) power-
// of-two block scales (e8m0 bytes e_i + 127): q1 rounds a / s1 to nearest
// even, q2 the exact residual a - s1*q1 on its own scale, q3 the next.  The
// scale of a term is the smallest power of two that keeps the block's largest
// magnitude within the e4m3 range (448).  Each term carries about four
// significant bits, so three terms leave a residual near 2^-12 of the block
// maximum.
//
// Layout (ws): q [3][rows][K] bytes, then scales [3][rows][K/32] bytes.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// e4m3 (OCP, finite) byte -> float, exact
MOE_DEV float e4m3_to_float(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -v : v;
}

// exponent e of the block scale 2^e: max / 2^e <= 448 with e as small as possible
MOE_DEV int block_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  const uint32_t bits = __float_as_uint(amax);
  int ex = (int)((bits >> 23) & 0xFFu) - 127;  // amax = 1.m * 2^ex (normal inputs)
  if (ex < -126) return -127;
  // 1.m * 2^ex / 2^(ex - 8) = 1.m * 256 <= 448 iff 1.m <= 1.75
  int e = ex - 8;
  if ((bits & 0x7FFFFFu) > 0x600000u) e += 1;  // 1.m > 1.75
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// One thread per (row, block of 32): 128 bytes in, 3 x 32 bytes + 3 scale bytes out.
__global__ __launch_bounds__(256) void mx8_split_kernel(const float *__restrict__ A, long long lda, int rows,
                                                        int K, uint8_t *__restrict__ q,
                                                        uint8_t *__restrict__ sc) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int nb = K / 32;
  if (i >= (long long)rows * nb) return;
  const long long row = i / nb;
  const int blk = (int)(i - row * nb);
  const f32x4_t *src = reinterpret_cast<const f32x4_t *>(A + row * lda + blk * 32);
  float a[32];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const f32x4_t x = src[v];
    a[4 * v] = x[0];
    a[4 * v + 1] = x[1];
    a[4 * v + 2] = x[2];
    a[4 * v + 3] = x[3];
  }
  const long long plane = (long long)rows * K, splane = (long long)rows * nb;
#pragma unroll
  for (int term = 0; term < 3; ++term) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(a[e]));
    const int ex = block_exp(amax);
    const float down = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex (ex in -126..127)
    const float up = ex >= -126 ? __uint_as_float((uint32_t)(ex + 127) << 23) : 0x1p-127f;
    uint32_t packed[8];
#pragma unroll
    for (int e = 0; e < 32; e += 4) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(a[e] * down, a[e + 1] * down, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(a[e + 2] * down, a[e + 3] * down, w, true);
      packed[e / 4] = (uint32_t)w;
#pragma unroll
      for (int u = 0; u < 4; ++u) a[e + u] -= e4m3_to_float(((uint32_t)w >> (8 * u)) & 0xFFu) * up;
    }
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(q + term * plane + row * K + blk * 32);
    dst[0] = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
    dst[1] = u32x4_t{packed[4], packed[5], packed[6], packed[7]};
    sc[term * splane + row * nb + blk] = (uint8_t)(ex + 127);
  }
}

}  // namespace

size_t mx8_split_bytes(long long rows, int K) { return (size_t)rows * K * 3 + (size_t)rows * (K / 32) * 3; }

hipError_t launch_mx8_split(const float *A, long long lda, int rows, int K, uint8_t *ws, hipStream_t st) {
  const long long n = (long long)rows * (K / 32);
  uint8_t *q = ws;
  uint8_t *sc = ws + (size_t)rows * K * 3;
  hipLaunchKernelGGL(mx8_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A, lda, rows, K, q,
                     sc);
  return hipGetLastError();
}

}  // namespace moe
