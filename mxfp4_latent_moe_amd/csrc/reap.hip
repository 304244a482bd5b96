// REAP expert saliency over a calibration batch: per expert j, the sum over
// the tokens routed to it of g_j(x) * ||e_j(x)||_2 and the number of such
// tokens (kimi-k3-mlx README, REAP section).  The expert outputs are the
// grouped down GEMM's un-weighted rows Y [P, L] in expert-sorted order, so
// expert j owns rows offsets[j] .. offsets[j+1].
//
// Two passes, both deterministic (no atomics):
//  * one wave per sorted row: ||Y_p||_2 (fp32 sum of squares in a fixed lane
//    order and tree) times the row's routing weight -> c[p];
//  * one wave per expert: the fp64 sum of c over its segment (lane-strided
//    partial sums, then a fixed tree), added to or written into sal_sum[j],
//    and the segment length into counts[j].
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

MOE_DEV float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
MOE_DEV double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void reap_rows_kernel(const float *__restrict__ Y, int P, int L,
                                                        const float *__restrict__ pair_weight,
                                                        const int32_t *__restrict__ sorted_pair,
                                                        float *__restrict__ contrib) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= P) return;
  const f32x4_t *row = reinterpret_cast<const f32x4_t *>(Y + (long long)p * L);
  float sq = 0.f;
  for (int i = lane; i < L / 4; i += 64) {
    const f32x4_t v = row[i];
    sq = fmaf(v[0], v[0], sq);
    sq = fmaf(v[1], v[1], sq);
    sq = fmaf(v[2], v[2], sq);
    sq = fmaf(v[3], v[3], sq);
  }
  sq = wave_sum_f32(sq);
  if (lane == 0) {
    const float g = pair_weight != nullptr ? pair_weight[sorted_pair[p]] : 1.f;
    contrib[p] = g * __builtin_sqrtf(sq);
  }
}

__global__ __launch_bounds__(256) void reap_experts_kernel(const float *__restrict__ contrib,
                                                           const int32_t *__restrict__ offsets, int E,
                                                           double *__restrict__ sal_sum,
                                                           long long *__restrict__ counts, int accumulate) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  double s = 0.0;
  for (int p = r0 + lane; p < r1; p += 64) s += (double)contrib[p];
  s = wave_sum_f64(s);
  if (lane == 0) {
    sal_sum[e] = accumulate ? sal_sum[e] + s : s;
    counts[e] = accumulate ? counts[e] + (long long)(r1 - r0) : (long long)(r1 - r0);
  }
}

}  // namespace

hipError_t launch_reap(const float *Y, int P, int L, const float *pair_weight, const int32_t *sorted_pair,
                       const int32_t *offsets, int E, double *sal_sum, long long *counts, int accumulate,
                       float *contrib, hipStream_t st) {
  if (P > 0) {
    hipLaunchKernelGGL(reap_rows_kernel, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, st, Y, P, L, pair_weight,
                       sorted_pair, contrib);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_reap_experts(contrib, offsets, E, sal_sum, counts, accumulate, st);
}

hipError_t launch_reap_experts(const float *contrib, const int32_t *offsets, int E, double *sal_sum,
                               long long *counts, int accumulate, hipStream_t st) {
  hipLaunchKernelGGL(reap_experts_kernel, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, st, contrib, offsets, E,
                     sal_sum, counts, accumulate);
  return hipGetLastError();
}

}  // namespace moe
