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

__global__ __launch_bounds__(256) void combine_norm_kernel(const float *__restrict__ Y,
                                                           const int32_t *__restrict__ pair_pos,
                                                           const float *__restrict__ w,
                                                           const uint16_t *__restrict__ gamma,
                                                           int k, int L, float eps,
                                                           float *__restrict__ yn) {
  __shared__ long long rows[32];
  __shared__ float wts[32];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    rows[tid] = pair_pos[(long long)t * k + tid];
    wts[tid] = w ? w[(long long)t * k + tid] : 1.0f;
  }
  __syncthreads();
  float *out = yn + (long long)t * L;
  float ss = 0.f;
  for (int c = tid * 4; c < L; c += 1024) {
    f32x4_t y = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t *>(Y + rows[j] * L + c);
      y += wts[j] * v;
    }
    *reinterpret_cast<f32x4_t *>(out + c) = y;
    ss += y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float scale = 1.0f / sqrtf(tot / (float)L + eps);
  for (int c = tid * 4; c < L; c += 1024) {
    f32x4_t y = *reinterpret_cast<const f32x4_t *>(out + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = y[e] * scale * __uint_as_float((uint32_t)gamma[c + e] << 16);
    *reinterpret_cast<f32x4_t *>(out + c) = y;
  }
}

}  // namespace

hipError_t launch_combine_norm(const float *Y, const int32_t *pair_pos, const float *w,
                               const uint16_t *gamma, int T, int k, int L, float eps, float *yn,
                               hipStream_t st) {
  hipLaunchKernelGGL(combine_norm_kernel, dim3(T), dim3(256), 0, st, Y, pair_pos, w, gamma, k, L, eps,
                     yn);
  return hipGetLastError();
}

}  // namespace moe
