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

MOE_DEV bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

MOE_DEV float sigmoid(float l) { return 1.0f / (1.0f + expf(-l)); }

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, float *__restrict__ gap) {
  __shared__ int sel_lds[4][32];
  __shared__ float s_lds[4][32];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool live = t < T;
  const float *lr = logits + (long long)(live ? t : 0) * E;

  float v[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + 64 * i;
    float b = -INFINITY;
    if (e < E) {
      b = sigmoid(lr[e]) + bias[e];
      if (b != b) b = -INFINITY;
    }
    v[i] = b;
  }
  uint32_t taken = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  auto rescan = [&]() {
    bv = -INFINITY;
    bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
  };
  rescan();

  int my_sel = 0x7fffffff;
  float kth = 0.f, kp1 = -INFINITY;
  const int rounds = (k < E) ? k + 1 : k;
  for (int r = 0; r < rounds; ++r) {
    float wv = bv;
    int wi = bi;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(wv, d, 64);
      const int oi = __shfl_xor(wi, d, 64);
      if (better(ov, oi, wv, wi)) {
        wv = ov;
        wi = oi;
      }
    }
    if (r < k) {
      if (lane == r) my_sel = wi;
      if (r == k - 1) kth = wv;
    } else {
      kp1 = wv;
    }
    if ((wi & 63) == lane) {
      taken |= 1u << (wi >> 6);
      rescan();
    }
  }

  // ascending order of the selected ids: rank = number of smaller selected ids
  int rank = 0;
  for (int q = 0; q < k; ++q) {
    const int o = __shfl(my_sel, q, 64);
    rank += (o < my_sel) ? 1 : 0;
  }
  if (lane < k) {
    sel_lds[wave][rank] = my_sel;
    s_lds[wave][rank] = sigmoid(lr[my_sel]);
  }
  __syncthreads();
  if (!live) return;
  float sum = 0.f;
  for (int q = 0; q < k; ++q) sum += s_lds[wave][q];
  if (lane < k) {
    ids[(long long)t * k + lane] = sel_lds[wave][lane];
    w[(long long)t * k + lane] = s_lds[wave][lane] / sum;
  }
  if (lane == 0 && gap != nullptr) gap[t] = (k < E) ? kth - kp1 : INFINITY;
}

}  // namespace

hipError_t launch_topk(const float *logits, const float *bias, int T, int E, int k, int32_t *ids,
                       float *w, float *gap, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, bias, T, E, k, ids, w,
                     gap);
  return hipGetLastError();
}

}  // namespace moe
