// Activations as a sum of three MX terms, for the MX-scaled expert GEMM:
// fp8 (e4m3) terms, or fp6 (e2m3) terms that the MFMA runs at the fp4 rate.
//
// fp8:
// Each run of 32 consecutive K values of a row (one MX block) is written as
// a ~= s1*q1 + s2*q2 + s3*q3 with q_i e4m3 (OCP) bytes and s_i = 2^(e_i) power-
// of-two block scales (e8m0 bytes e_i + 127): q1 rounds a / s1 to nearest
// even, q2 the exact residual a - s1*q1 on its own scale, q3 the next.  The
// scale of a term is the smallest power of two that keeps the block's largest
// magnitude within the e4m3 range (448).  Each term carries about four
// significant bits, so three terms leave a residual near 2^-12 of the block
// maximum.
//
// Layout (ws): q [3][rows][K] bytes, then scales [3][rows][K/32] bytes.  Row r
// of the planes is row r of the activations, or row map[r] / div of them when
// a gather map is given.
//
// fp6: the same three-term recursion with e2m3 (OCP MX) codes: 1 sign, 2
// exponent (bias 1) and 3 mantissa bits, magnitudes m/8 for exponent 0 and
// (1 + m/8) 2^(e-1) otherwise, largest 7.5.  The scale of a term is the
// smallest power of two that keeps the block's largest magnitude within 7.5.
// A block's 32 codes are packed LSB first, code i in bits 6i .. 6i+5 of six
// dwords, which is the operand layout of the MX MFMA (32 consecutive K per
// lane group).  Each block takes a 32-byte slot of the q planes (24 bytes of
// codes, then 8 zero bytes), so the planes keep the fp8 size and stride.
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
                                                        int K, const int32_t *__restrict__ map, int div,
                                                        uint8_t *__restrict__ q, uint8_t *__restrict__ sc) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int nb = K / 32;
  if (i >= (long long)rows * nb) return;
  const long long row = i / nb;
  const int blk = (int)(i - row * nb);
  const long long arow = map ? (long long)(map[row] / div) : row;
  const f32x4_t *src = reinterpret_cast<const f32x4_t *>(A + arow * lda + blk * 32);
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

// exponent e of the e2m3 block scale 2^e: max / 2^e <= 7.5 with e as small as possible
MOE_DEV int block_exp6(float amax) {
  if (!(amax > 0.f)) return -127;
  const uint32_t bits = __float_as_uint(amax);
  int ex = (int)((bits >> 23) & 0xFFu) - 127;
  if (ex < -126) return -127;
  // 1.m * 2^ex / 2^(ex - 2) = 1.m * 4 <= 7.5 iff 1.m <= 1.875
  int e = ex - 2;
  if ((bits & 0x7FFFFFu) > 0x700000u) e += 1;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// e2m3 code of v (|v| <= 7.5), round to nearest even, and its value.  On
// [0, 2) the grid step is 1/8, on [2, 4) 1/4, on [4, 8) 1/2; with E the
// binade (0, 1, 2) the code is rne(|v| 2^(3-E)) + 8E, which carries into
// the next binade correctly when the rounding goes up.
MOE_DEV uint32_t to_e2m3(float v, float &q) {
  const float av = fabsf(v);
  const int E = av >= 4.f ? 2 : (av >= 2.f ? 1 : 0);
  const float up = E == 2 ? 2.f : (E == 1 ? 4.f : 8.f);
  const float step = E == 2 ? 0.5f : (E == 1 ? 0.25f : 0.125f);
  const float r = __builtin_rintf(av * up);
  const uint32_t mag = (uint32_t)r + 8u * (uint32_t)E;
  q = copysignf(r * step, v);
  return (v < 0.f && mag) ? (mag | 32u) : mag;
}

// One thread per (row, block of 32): 128 bytes in, 3 x 32 bytes + 3 scale bytes out.
__global__ __launch_bounds__(256) void mx6_split_kernel(const float *__restrict__ A, long long lda, int rows,
                                                        int K, const int32_t *__restrict__ map, int div,
                                                        uint8_t *__restrict__ q, uint8_t *__restrict__ sc) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int nb = K / 32;
  if (i >= (long long)rows * nb) return;
  const long long row = i / nb;
  const int blk = (int)(i - row * nb);
  const long long arow = map ? (long long)(map[row] / div) : row;
  const f32x4_t *src = reinterpret_cast<const f32x4_t *>(A + arow * lda + blk * 32);
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
    const int ex = block_exp6(amax);
    const float down = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex (ex in -126..127)
    const float up = ex >= -126 ? __uint_as_float((uint32_t)(ex + 127) << 23) : 0x1p-127f;
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      float qv;
      const uint32_t c = to_e2m3(a[e] * down, qv);
      a[e] -= qv * up;
      const int bit = 6 * e, word = bit >> 5, off = bit & 31;
      w[word] |= c << off;
      if (off > 26) w[word + 1] |= c >> (32 - off);
    }
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(q + term * plane + row * K + blk * 32);
    dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4_t{w[4], w[5], 0u, 0u};
    sc[term * splane + row * nb + blk] = (uint8_t)(ex + 127);
  }
}

}  // namespace

size_t mx8_split_bytes(long long rows, int K) { return (size_t)rows * K * 3 + (size_t)rows * (K / 32) * 3; }

hipError_t launch_mx_split(bool fp6, const float *A, long long lda, int rows, int K, const int32_t *map, int div,
                           uint8_t *ws, hipStream_t st) {
  const long long n = (long long)rows * (K / 32);
  uint8_t *q = ws;
  uint8_t *sc = ws + (size_t)rows * K * 3;
  if (fp6)
    hipLaunchKernelGGL(mx6_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A, lda, rows, K, map,
                       div, q, sc);
  else
    hipLaunchKernelGGL(mx8_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A, lda, rows, K, map,
                       div, q, sc);
  return hipGetLastError();
}

}  // namespace moe
