// Biased top-k selection of the sigmoid router, one wavefront per token.
//
// kimi-k3-mlx README, Architecture table, MoE row: sigmoid router over the
// experts plus the aux-loss-free e_score_correction_bias, top-16.  The bias
// takes part in the selection only; the weights are the selected sigmoid
// scores divided by their sum.  Order: larger biased score first, then the
// lower expert index (NaN ranks last).  Output slots hold the selected ids in
// ascending order.
//
// Capped promotion (Kimi-K3-Alis-MLX-Dynamic card, Build recipe: the serving
// configuration keeps at most moe_k_hi promoted MXFP4 experts per token and
// drops the contribution of the later ones): with a promoted mask given, a
// selected promoted expert that has k_hi selected promoted experts ahead of
// it in routing order gets weight 0.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int SLOTS = 16;  // experts per lane: E <= 64 * SLOTS = 1024
// token counts up to this take one work-group per token (topk_token_kernel)
#ifndef TOPK_TOKEN_MAX_T
#define TOPK_TOKEN_MAX_T 256
#endif

// Order-preserving map of a biased score onto uint32 (larger score, larger
// key); -0 is folded onto +0 so the two compare equal, as floats do.
MOE_DEV uint32_t order_key(float b) {
  uint32_t u = __float_as_uint(b);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float key_value(uint32_t key) { return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key); }

MOE_DEV float sigmoid(float l) { return 1.0f / (1.0f + expf(-l)); }

// lanes below this one with their bit set in m
MOE_DEV int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The k-th largest key of a wavefront's SLOTS x 64 keys and the selection
// (see above): the selected ids, scores and keys go to sel / s / kl in
// ascending id order; th is the k-th largest key, kp1 the (k+1)-th.
MOE_DEV void select_topk(const uint32_t (&key)[SLOTS], const float (&sg)[SLOTS], int k, int lane, int *sel,
                         float *s, uint32_t *kl, uint32_t &th_out, uint32_t &kp1_out) {
  auto count_ge = [&](uint32_t c) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) n += __popcll(__ballot(key[i] >= c));
    return n;
  };
  uint32_t th = 0u;  // the largest c with at least k keys >= c: the k-th largest key
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = th | (1u << bit);
    if (count_ge(c) >= k) th = c;
  }
  int above = 0, at_or_above = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    above += __popcll(__ballot(key[i] > th));
    at_or_above += __popcll(__ballot(key[i] >= th));
  }
  // (k+1)-th largest: th again if more keys equal it, else the largest key below it
  uint32_t below = 0u;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) below = max(below, key[i] < th ? key[i] : 0u);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) below = max(below, (uint32_t)__shfl_xor((int)below, d, 64));
  kp1_out = at_or_above > k ? th : below;
  th_out = th;

  int need = k - above;  // keys equal to th that are selected, lowest indices first
  int pos = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const uint64_t eq = __ballot(key[i] == th);
    const bool pick = key[i] > th || (key[i] == th && lanes_below(eq) < need);
    need -= min(__popcll(eq), max(need, 0));
    const uint64_t m = __ballot(pick);
    if (pick) {
      const int q = pos + lanes_below(m);
      sel[q] = lane + 64 * i;
      s[q] = sg[i];
      kl[q] = key[i];
    }
    pos += __popcll(m);
  }
}

// Weights of token t from its selection (after a barrier that makes the
// selection visible): the selected sigmoid scores over their sum, with the
// capped-promotion rule when a promoted mask is given.
MOE_DEV void write_topk(int t, int k, int lane, const int *sel, const float *s, const uint32_t *kl,
                        const uint8_t *promoted, int k_hi, int32_t *ids, float *w) {
  float sum = 0.f;
  for (int q = 0; q < k; ++q) sum += s[q];
  if (lane < k) {
    const int id = sel[lane];
    float wt = s[lane] / sum;
    if (promoted != nullptr && promoted[id]) {
      // capped promotion: a promoted expert with k_hi selected promoted experts
      // ahead of it in routing order (larger key, or equal key and lower id)
      // has its contribution dropped; the other weights stay as they are
      const uint32_t my = kl[lane];
      int ahead = 0;
      for (int q = 0; q < k; ++q) {
        const int o = sel[q];
        const uint32_t ok = kl[q];
        ahead += (promoted[o] && (ok > my || (ok == my && o < id))) ? 1 : 0;
      }
      if (ahead >= k_hi) wt = 0.f;
    }
    ids[(long long)t * k + lane] = id;
    w[(long long)t * k + lane] = wt;
  }
}

// Lane l holds experts l + 64 i.  The k-th largest key is found by a binary
// descent over its 32 bits, each step counting the keys at or above the
// candidate with one ballot per slot (no cross-lane data movement).  The
// selection is every key above it plus, among the keys equal to it, the
// lowest expert indices; expert index order is slot-major, lane-minor, so
// walking the slots in order with a per-slot prefix count resolves the ties
// and also emits the selected ids in ascending order.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   const float *__restrict__ partial, int splits,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, float *__restrict__ gap,
                                                   const uint8_t *__restrict__ promoted, int k_hi) {
  __shared__ int sel_lds[4][32];
  __shared__ float s_lds[4][32];
  __shared__ uint32_t key_lds[4][32];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool live = t < T;
  const float *lr = logits + (long long)(live ? t : 0) * E;

  // logits: read, or summed here from the router's split-K partials in split
  // order from zero (the same additions a separate finalize pass makes)
  float lg[SLOTS];
  if (partial != nullptr) {
    const float *pt = partial + (long long)(live ? t : 0) * E;
    const long long sstride = (long long)T * E;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) lg[i] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 4) {
      float v[4][SLOTS];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
          const int e = lane + 64 * i;
          v[u][i] = (s0 + u < splits && e < E) ? pt[(s0 + u) * sstride + e] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (s0 + u < splits) {
#pragma unroll
          for (int i = 0; i < SLOTS; ++i) lg[i] += v[u][i];
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int e = lane + 64 * i;
      lg[i] = e < E ? lr[e] : 0.f;
    }
  }

  uint32_t key[SLOTS];  // 0 for slots past E: below every real expert
  float sg[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0u;
    sg[i] = 0.f;
    if (e < E) {
      sg[i] = sigmoid(lg[i]);
      float b = sg[i] + bias[e];
      if (b != b) b = -INFINITY;
      key[i] = order_key(b);
    }
  }
  uint32_t th, kp1;
  select_topk(key, sg, k, lane, sel_lds[wave], s_lds[wave], key_lds[wave], th, kp1);
  __syncthreads();
  if (!live) return;
  write_topk(t, k, lane, sel_lds[wave], s_lds[wave], key_lds[wave], promoted, k_hi, ids, w);
  if (lane == 0 && gap != nullptr) gap[t] = (k < E) ? key_value(th) - key_value(kp1) : INFINITY;
}


// The same selection with one work-group per token, for small token counts:
// the four wavefronts add the router's split-K partials of a quarter of the
// experts each (every partial of a thread's experts requested at once, added
// in split order from zero as above, so the logits are bitwise the same),
// the keys meet in LDS, and wavefront 0 selects from them in the lane/slot
// layout of topk_kernel.  Per token the partials then take one memory round
// trip instead of splits / 4.
__global__ __launch_bounds__(256) void topk_token_kernel(const float *__restrict__ logits,
                                                         const float *__restrict__ partial, int splits,
                                                         const float *__restrict__ bias, int T, int E, int k,
                                                         int32_t *__restrict__ ids, float *__restrict__ w,
                                                         float *__restrict__ gap,
                                                         const uint8_t *__restrict__ promoted, int k_hi) {
  constexpr int PER = 64 * SLOTS / 256;  // experts per thread: tid + 256 u
  constexpr int SB = 8;                  // partials requested per round
  __shared__ uint32_t s_key[64 * SLOTS];
  __shared__ float s_sg[64 * SLOTS];
  __shared__ int sel_lds[32];
  __shared__ float s_lds[32];
  __shared__ uint32_t key_lds[32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t = blockIdx.x;

  float lg[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) lg[u] = 0.f;
  if (partial != nullptr) {
    const float *pt = partial + (long long)t * E;
    const long long sstride = (long long)T * E;
    for (int s0 = 0; s0 < splits; s0 += SB) {
      float v[SB][PER];
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int e = tid + 256 * u;
          v[b][u] = (s0 + b < splits && e < E) ? pt[(s0 + b) * sstride + e] : 0.f;
        }
#pragma unroll
      for (int b = 0; b < SB; ++b)
        if (s0 + b < splits) {
#pragma unroll
          for (int u = 0; u < PER; ++u) lg[u] += v[b][u];
        }
    }
  } else {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u;
      lg[u] = e < E ? logits[(long long)t * E + e] : 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + 256 * u;
    uint32_t key = 0u;  // slots past E: below every real expert
    float sg = 0.f;
    if (e < E) {
      sg = sigmoid(lg[u]);
      float b = sg + bias[e];
      if (b != b) b = -INFINITY;
      key = order_key(b);
    }
    s_key[e] = key;
    s_sg[e] = sg;
  }
  __syncthreads();
  uint32_t th = 0u, kp1 = 0u;
  if (wave == 0) {
    uint32_t key[SLOTS];
    float sg[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      key[i] = s_key[lane + 64 * i];
      sg[i] = s_sg[lane + 64 * i];
    }
    select_topk(key, sg, k, lane, sel_lds, s_lds, key_lds, th, kp1);
  }
  __syncthreads();
  if (wave != 0) return;
  write_topk(t, k, lane, sel_lds, s_lds, key_lds, promoted, k_hi, ids, w);
  if (lane == 0 && gap != nullptr) gap[t] = (k < E) ? key_value(th) - key_value(kp1) : INFINITY;
}
}  // namespace

hipError_t launch_topk(const float *logits, const float *partial, int splits, const float *bias, int T, int E,
                       int k, int32_t *ids, float *w, float *gap, const uint8_t *promoted, int k_hi,
                       hipStream_t st) {
  if (T <= TOPK_TOKEN_MAX_T) {
    hipLaunchKernelGGL(topk_token_kernel, dim3(T), dim3(256), 0, st, logits, partial, splits, bias, T, E, k, ids, w,
                       gap, promoted, k_hi);
  } else {
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, partial, splits, bias, T, E, k,
                       ids, w, gap, promoted, k_hi);
  }
  return hipGetLastError();
}

}  // namespace moe
