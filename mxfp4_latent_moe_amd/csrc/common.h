// Shared device helpers for the gfx950 kernels: vector types, MFMA, bf16
// splitting, MXFP4 nibble conversion, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define MOE_DEV __device__ __forceinline__

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).
// Lane l holds A row (l % 16), B column (l % 16), each with 8 consecutive K
// values of K-block (l / 16); D column (l % 16), rows 4*(l/16) .. +3.
MOE_DEV f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round to nearest even (gfx950 v_cvt_pk_bf16_f32).
MOE_DEV __bf16 to_bf16(float x) { return (__bf16)x; }
MOE_DEV float from_bf16(__bf16 x) { return (float)x; }

// a = hi + lo with hi = bf16(a) and lo = bf16(a - hi); a - hi is exact in fp32.
MOE_DEV void split_bf16(float a, __bf16 &hi, __bf16 &lo) {
  hi = to_bf16(a);
  lo = to_bf16(a - from_bf16(hi));
}

// Eight e2m1 codes (one dword, element 2b in the low nibble of byte b) times
// 2^(e-127) as eight bf16 values in element order.  The scale argument is the
// float whose bit pattern is e << 23, i.e. exactly 2^(e-127) for e in 1..254.
MOE_DEV bf16x8_t fp4x8_to_bf16(uint32_t q, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

MOE_DEV float e8m0_to_float(uint32_t e) { return __uint_as_float(e << 23); }

// Affine 2-bit codes (element i of a dword in bits 2i .. 2i+1) as exact bf16
// integers q through the fp4 convert: masked into the low half of a nibble,
// code q reads as the e2m1 value q / 2, and the convert's scale 2 (a power of
// two: the convert takes only the exponent of its scale) gives q.
// y = d & 0x33333333 holds codes 4b and 4b+2 in byte b, z = (d >> 2) &
// 0x33333333 codes 4b+1 and 4b+3.  Bytes B and B+1 of y and z give the eight
// codes 4B .. 4B+7 in the order 0, 2, 1, 3, 4, 6, 5, 7 (relative to 4B); the
// activations are staged in that same order, so the products pair up.
template <int B>
MOE_DEV bf16x8_t aff2x8_to_bf16(uint32_t y, uint32_t z) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y, 2.0f, B);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(z, 2.0f, B);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y, 2.0f, B + 1);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(z, 2.0f, B + 1);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}
// Slot i of an octet of activations staged for affine weights holds element
// aff2_perm(i) of the octet (the order aff2x8_to_bf16 produces).
MOE_DEV constexpr int aff2_perm(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }
// Affine K layout of one 128-wide K step (two 64-element groups h): MFMA
// instruction j = 2h + jj covers group h only; in it, lane group kg takes the
// 8 elements 64h + 16kg + 8jj .. +7, i.e. half jj of the step's dword 4h + kg
// of codes, and the activations of octet 8h + 2kg + jj.
MOE_DEV constexpr int aff2_octet(int h, int kg, int jj) { return 8 * h + 2 * kg + jj; }
// fp32 value of the bf16 in the low 16 bits of a pattern
MOE_DEV float bf16_lo_to_float(uint32_t bits) { return __uint_as_float(bits << 16); }

// tanh x in fp32 as a fraction num / den, from two identities: the odd
// Taylor series of tanh (Bernoulli-number coefficients, terms to x^11) over 1
// for |x| < 0.4, where the first omitted term is below 1e-7 of the value, and
// sign(x) (1 - e) over (1 + e) with e = exp(-2|x|) above, where 1 - e does not
// cancel.  The exponential is the hardware one (about 1 ulp); after one
// hardware reciprocal the worst relative error over the fp32 range is about
// 2.4e-7.
MOE_DEV void tanh_frac_f32(float x, float &num, float &den) {
  const float ax = fabsf(x);
  const float x2 = x * x;
  float p = -1382.0f / 155925.0f;
  p = fmaf(p, x2, 62.0f / 2835.0f);
  p = fmaf(p, x2, -17.0f / 315.0f);
  p = fmaf(p, x2, 2.0f / 15.0f);
  p = fmaf(p, x2, -1.0f / 3.0f);
  const float series = fmaf(x * x2, p, x);
  const float e = __builtin_amdgcn_exp2f(ax * -2.8853900817779268f);  // exp(-2|x|) as 2^(-2|x| log2 e)
  const bool small = ax < 0.4f;
  num = small ? series : copysignf(1.0f - e, x);
  den = small ? 1.0f : 1.0f + e;
}

// SiTU-GLU in fp32: beta*tanh(g/beta)*sigmoid(g) * beta_lin*tanh(u/beta_lin),
// with sigmoid(g) = 1 / (1 + exp(-g)).  The three denominators share one
// hardware reciprocal: for g below about -88, 1 + exp(-g) is +inf and the
// result is 0, the limit of the product.
MOE_DEV float situ_glu(float g, float u, float beta, float beta_lin) {
  float ng, dg, nu, du;
  tanh_frac_f32(g * __builtin_amdgcn_rcpf(beta), ng, dg);
  tanh_frac_f32(u * __builtin_amdgcn_rcpf(beta_lin), nu, du);
  const float ds = 1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return (beta * ng) * (beta_lin * nu) * __builtin_amdgcn_rcpf(dg * du * ds);
}

MOE_DEV int lane_id() { return threadIdx.x & 63; }

// Raw buffer resource over [base, base + bytes): loads outside it return 0.
// Word 3 is the gfx9-family raw-buffer format (32-bit data format, no swizzle).
MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
MOE_DEV u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
MOE_DEV uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
MOE_DEV u32x2_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// Work-item decode shared by the GEMM kernels.  The grid is sized for the
// worst case; the real items are the first `total` logical ids.  Blocks are
// handed to the 8 XCDs round-robin, so block b gets logical id
// (b % 8) * (T8 / 8) + b / 8 with T8 = total rounded up to 8: every XCD gets an
// equal share of the real items and consecutive logical ids (the weight
// blocks of one row chunk) run on the same XCD.  Returns -1 for no work.
MOE_DEV int xcd_logical(int total) {
  const int t8 = (total + 7) & ~7;
  const int b = blockIdx.x;
  if (b >= t8) return -1;
  const int logical = (b & 7) * (t8 >> 3) + (b >> 3);
  return logical < total ? logical : -1;
}

// ---- direct-to-LDS loads and hand-scheduled LDS reads
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits until at most n vector memory operations are outstanding
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// fn(integral_constant<0>) .. fn(integral_constant<N - 1>), in order
template <int N, typename Fn>
MOE_DEV void static_for(Fn &&fn) {
  if constexpr (N > 0) {
    static_for<N - 1>(fn);
    fn(std::integral_constant<int, N - 1>{});
  }
}

MOE_DEV uint32_t lds_addr(const uint8_t *p) { return (uint32_t)(uintptr_t)(const lds_void *)p; }
