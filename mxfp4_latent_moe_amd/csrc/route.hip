// Biased top-k selection of the sigmoid router, one wavefront per token.
//
// kimi-k3-mlx README, Architecture table, MoE row: sigmoid router over the
// experts plus the aux-loss-free e_score_correction_bias, top-16.  The bias
// takes part in the selection only; the weights are the selected sigmoid
// scores divided by their sum.  Order: larger biased score first, then the
// lower expert index (NaN ranks last).  Output slots hold the selected ids in
// ascending order.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int SLOTS = 16;  // experts per lane: E <= 64 * SLOTS = 1024

MOE_DEV float sigmoid(float l) { return 1.0f / (1.0f + expf(-l)); }

// Order-preserving map of a biased score to 32 bits (NaN ranks as -inf).
MOE_DEV uint32_t ordered(float b) {
  if (b != b) b = -INFINITY;
  const uint32_t u = __float_as_uint(b);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float unordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// One DPP move of a 64-bit value within rows of 16 lanes.
template <int CTRL>
MOE_DEV uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
MOE_DEV uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
MOE_DEV uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave, the same value in every lane: quad swaps and row
// mirrors reduce each row of 16, then the four row results are read out.
MOE_DEV uint64_t wave_max64(uint64_t k) {
  k = max64(k, dpp64<0xB1>(k));   // quad_perm [1,0,3,2]
  k = max64(k, dpp64<0x4E>(k));   // quad_perm [2,3,0,1]
  k = max64(k, dpp64<0x141>(k));  // row_half_mirror
  k = max64(k, dpp64<0x140>(k));  // row_mirror
  return max64(max64(readlane64(k, 0), readlane64(k, 16)), max64(readlane64(k, 32), readlane64(k, 48)));
}

// Biased top-k, one wavefront per token.  Each candidate is the 64-bit key
// (ordered biased score, inverted expert id): the larger key is the larger
// score, then the lower id, and keys are unique.  Round r takes the wave
// maximum; the lane that owned it drops that slot and rescans its own.
// Logits are the sum of `splits` partial products in split order.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ partial, int splits,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, float *__restrict__ gap) {
  __shared__ int sel_lds[4][32];
  __shared__ float sc_lds[4][32];
  __shared__ float sorted_lds[4][32];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool live = t < T;
  const long long tt = live ? t : 0;

  uint64_t key[SLOTS];
  float sc[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0;
    sc[i] = 0.f;
    if (e < E) {
      float l = 0.f;
      for (int q = 0; q < splits; ++q) l += partial[((long long)q * T + tt) * E + e];
      sc[i] = sigmoid(l);
      key[i] = ((uint64_t)ordered(sc[i] + bias[e]) << 32) | (uint32_t)(~e);
    }
  }
  uint32_t taken = 0;
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) best = max64(best, key[i]);

  uint32_t kth = 0, kp1 = 0;
  const int rounds = (k < E) ? k + 1 : k;
  for (int r = 0; r < rounds; ++r) {
    const uint64_t K = wave_max64(best);
    const int e = (int)(~(uint32_t)K);
    if (r < k) {
      if (r == k - 1) kth = (uint32_t)(K >> 32);
    } else {
      kp1 = (uint32_t)(K >> 32);
    }
    if ((e & 63) == lane) {
      const int slot = e >> 6;
      float s_won = 0.f;
      best = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (i == slot) {
          taken |= 1u << i;
          s_won = sc[i];
        }
        if (!((taken >> i) & 1u)) best = max64(best, key[i]);
      }
      if (r < k) {
        sel_lds[wave][r] = e;
        sc_lds[wave][r] = s_won;
      }
    }
  }
  __syncthreads();

  // ascending order of the selected ids: rank = number of smaller selected ids
  if (lane < k) {
    const int my = sel_lds[wave][lane];
    int rank = 0;
    for (int q = 0; q < k; ++q) rank += (sel_lds[wave][q] < my) ? 1 : 0;
    sorted_lds[wave][rank] = sc_lds[wave][lane];
    if (live) ids[tt * k + rank] = my;
  }
  __syncthreads();
  if (!live) return;
  float sum = 0.f;
  for (int q = 0; q < k; ++q) sum += sorted_lds[wave][q];
  if (lane < k) w[tt * k + lane] = sorted_lds[wave][lane] / sum;
  if (lane == 0 && gap != nullptr) gap[t] = (k < E) ? unordered(kth) - unordered(kp1) : INFINITY;
}

}  // namespace

hipError_t launch_topk(const float *partial, int splits, const float *bias, int T, int E, int k,
                       int32_t *ids, float *w, float *gap, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, partial, splits, bias, T, E, k, ids,
                     w, gap);
  return hipGetLastError();
}

}  // namespace moe
