// Weighted combine of the expert outputs and RMSNorm on the combined latent.
//
// kimi-k3-mlx README, REAP section, caveat paragraph: K3's LatentMoE applies
// RMSNorm to the combined expert output before up_proj.  One workgroup per
// token: y = sum_j w_j * Y[pair_pos[t*k+j]] in fixed slot order, then
// y * (1 / sqrt(mean(y^2) + eps)) * gamma with a fixed-order reduction.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// One workgroup of 1024 threads per token: each thread owns 4 columns (one
// pass covers L <= 4096), loads its k rows in batches of 8 before summing them
// in order j = 0..k-1, and the sum of squares goes through a fixed-order
// reduction over the 16 waves.
//
// REAP: the same pass also takes each row's sum of squares (the unweighted
// expert output e_j(x)), reduces it per row over the wavefronts in a fixed
// order and writes g * ||e_j(x)||_2 to contrib at the row's sorted position
// (kimi-k3-mlx README, REAP section).  That needs every column of a row in one
// pass, so L <= 4096; the combined output is computed exactly as without it.
template <bool REAP>
__global__ __launch_bounds__(1024) void combine_norm_kernel(const float *__restrict__ Y,
                                                            const int32_t *__restrict__ pair_pos,
                                                            const float *__restrict__ w,
                                                            const uint16_t *__restrict__ gamma,
                                                            int k, int L, float eps,
                                                            float *__restrict__ yn,
                                                            float *__restrict__ contrib) {
  constexpr int NTHR = 1024, B = 8, NWV = NTHR / 64;
  __shared__ long long rows[32];
  __shared__ float wts[32];
  __shared__ float red[NWV];
  __shared__ float rsq[REAP ? 32 : 1][NWV];  // per row, per wave: partial sums of squares
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    rows[tid] = pair_pos[(long long)t * k + tid];
    wts[tid] = w ? w[(long long)t * k + tid] : 1.0f;
  }
  __syncthreads();
  float *out = yn + (long long)t * L;
  float ss = 0.f;
  // y_t over this thread's columns: k rows loaded in batches of B, summed in
  // order j = 0..k-1 (the same arithmetic with and without REAP)
  auto combine = [&](int c, bool in) {
    f32x4_t y = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += B) {
      f32x4_t v[B];
#pragma unroll
      for (int jj = 0; jj < B; ++jj) {
        v[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (in && j0 + jj < k) v[jj] = *reinterpret_cast<const f32x4_t *>(Y + rows[j0 + jj] * L + c);
      }
#pragma unroll
      for (int jj = 0; jj < B; ++jj)
        if (j0 + jj < k) y += wts[j0 + jj] * v[jj];
      if constexpr (REAP) {
        // every lane takes part (lanes past L hold zeros), so the wave sums are whole
#pragma unroll
        for (int jj = 0; jj < B; ++jj) {
          if (j0 + jj >= k) break;
          float q = v[jj][0] * v[jj][0] + v[jj][1] * v[jj][1] + v[jj][2] * v[jj][2] + v[jj][3] * v[jj][3];
#pragma unroll
          for (int d = 32; d >= 1; d >>= 1) q += __shfl_xor(q, d, 64);
          if ((tid & 63) == 0) rsq[j0 + jj][tid >> 6] = q;
        }
      }
    }
    if (in) {
      *reinterpret_cast<f32x4_t *>(out + c) = y;
      ss += y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
    }
  };
  if constexpr (REAP) {
    combine(tid * 4, tid * 4 < L);  // one pass: L <= 4 * NTHR
  } else {
    for (int c = tid * 4; c < L; c += NTHR * 4) combine(c, true);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if constexpr (REAP) {
    if (tid < k) {
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < NWV; ++i) q += rsq[tid][i];
      contrib[rows[tid]] = wts[tid] * __builtin_sqrtf(q);
    }
  }
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NTHR / 64; ++i) tot += red[i];
  const float scale = 1.0f / sqrtf(tot / (float)L + eps);
  for (int c = tid * 4; c < L; c += NTHR * 4) {
    f32x4_t y = *reinterpret_cast<const f32x4_t *>(out + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = y[e] * scale * __uint_as_float((uint32_t)gamma[c + e] << 16);
    *reinterpret_cast<f32x4_t *>(out + c) = y;
  }
}

// The plain combine (no REAP sums) writing y_n as bf16 planes: with L <= 4096
// a thread's four columns stay in registers through the reduction, so y_n is
// written once, as the next GEMM's operands.  Same arithmetic as
// combine_norm_kernel<false>.
__global__ __launch_bounds__(1024) void combine_norm_planes_kernel(const float *__restrict__ Y,
                                                                   const int32_t *__restrict__ pair_pos,
                                                                   const float *__restrict__ w,
                                                                   const uint16_t *__restrict__ gamma, int k,
                                                                   int L, float eps, __bf16 *__restrict__ hi,
                                                                   __bf16 *__restrict__ lo) {
  constexpr int NTHR = 1024, B = 8, NWV = NTHR / 64;
  __shared__ long long rows[32];
  __shared__ float wts[32];
  __shared__ float red[NWV];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    rows[tid] = pair_pos[(long long)t * k + tid];
    wts[tid] = w ? w[(long long)t * k + tid] : 1.0f;
  }
  __syncthreads();
  const int c = tid * 4;
  const bool in = c < L;
  f32x4_t y = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += B) {
    f32x4_t v[B];
#pragma unroll
    for (int jj = 0; jj < B; ++jj) {
      v[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (in && j0 + jj < k) v[jj] = *reinterpret_cast<const f32x4_t *>(Y + rows[j0 + jj] * L + c);
    }
#pragma unroll
    for (int jj = 0; jj < B; ++jj)
      if (j0 + jj < k) y += wts[j0 + jj] * v[jj];
  }
  float ss = in ? y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3] : 0.f;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NWV; ++i) tot += red[i];
  const float scale = 1.0f / sqrtf(tot / (float)L + eps);
  if (!in) return;
  bf16x4_t h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = y[e] * scale * __uint_as_float((uint32_t)gamma[c + e] << 16);
    __bf16 vh, vl;
    split_bf16(v, vh, vl);
    h[e] = vh;
    l[e] = vl;
  }
  const long long o = (long long)t * L + c;
  *reinterpret_cast<bf16x4_t *>(hi + o) = h;
  if (lo != nullptr) *reinterpret_cast<bf16x4_t *>(lo + o) = l;
}

}  // namespace

hipError_t launch_combine_norm_planes(const float *Y, const int32_t *pair_pos, const float *w,
                                      const uint16_t *gamma, int T, int k, int L, float eps, uint16_t *hi,
                                      uint16_t *lo, hipStream_t st) {
  if (L > 4096 || L % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_norm_planes_kernel, dim3(T), dim3(1024), 0, st, Y, pair_pos, w, gamma, k, L, eps,
                     reinterpret_cast<__bf16 *>(hi), reinterpret_cast<__bf16 *>(lo));
  return hipGetLastError();
}

hipError_t launch_combine_norm(const float *Y, const int32_t *pair_pos, const float *w,
                               const uint16_t *gamma, int T, int k, int L, float eps, float *yn,
                               float *contrib, hipStream_t st) {
  if (contrib != nullptr) {
    if (L > 4096) return hipErrorInvalidValue;  // the REAP pass needs a row in one pass
    hipLaunchKernelGGL(combine_norm_kernel<true>, dim3(T), dim3(1024), 0, st, Y, pair_pos, w, gamma, k, L,
                       eps, yn, contrib);
  } else {
    hipLaunchKernelGGL(combine_norm_kernel<false>, dim3(T), dim3(1024), 0, st, Y, pair_pos, w, gamma, k, L,
                       eps, yn, contrib);
  }
  return hipGetLastError();
}

}  // namespace moe
