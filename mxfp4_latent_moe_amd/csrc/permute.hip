// Stable counting sort of the (token, slot) pairs by expert id.
//
// kimi-k3-mlx README, REAP section, two-bank paragraph: once the pairs are
// sorted by expert index each expert owns a contiguous slice of rows.  Pair
// p = t*k + j; inside an expert's slice the pairs keep their order, so tokens
// ascend.  Three passes, none with an order-dependent result (one workgroup
// runs all three when the tokens fit one block):
//   1. per block of 64 tokens, a histogram of expert ids (LDS counters);
//   2. one workgroup turns the histograms into per-block absolute bases,
//      expert offsets and the list of active experts (scans);
//   3. per block, one wavefront walks its tokens in order and scatters.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int TB = 64;  // tokens per block

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t *__restrict__ ids, int T,
                                                         int k, int E, int32_t *__restrict__ blk) {
  __shared__ int hist[1024];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t0 = b * TB;
  const int npairs = min(TB, T - t0) * k;
  for (int i = threadIdx.x; i < npairs; i += 256) {
    const int e = ids[(long long)t0 * k + i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);  // ids outside [0, E) are dropped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk[(long long)b * E + e] = hist[e];
}

// exclusive scan over 1024 threads (one value each); returns the prefix, total in *tot
__device__ int block_excl_scan(int x, int *wave_tot, int *tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int v = wave_tot[w];
    if (w < wave) before += v;
    all += v;
  }
  __syncthreads();
  *tot = all;
  return before + inc - x;
}

// Thread e owns expert e's column of block counts.  The column is read in
// batches of SB independent loads (all in flight at once), summed, and after
// the scan over experts rewritten as absolute bases: offsets[e] plus the
// counts of the blocks before.
constexpr int SB = 32;
__global__ __launch_bounds__(1024) void perm_scan_kernel(int nblk, int E, int P,
                                                         int32_t *__restrict__ blk,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ active) {
  __shared__ int wave_tot[16];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nblk; b0 += SB) {
      int c[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) c[i] = b0 + i < nblk ? blk[(long long)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < SB; ++i) cnt += c[i];
    }
  }
  int total;
  const int off = block_excl_scan(e < E ? cnt : 0, wave_tot, &total);
  if (e < E) {
    offsets[e] = off;
    int run = off;
    for (int b0 = 0; b0 < nblk; b0 += SB) {
      int c[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) c[i] = b0 + i < nblk ? blk[(long long)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (b0 + i < nblk) blk[(long long)(b0 + i) * E + e] = run;
        run += c[i];
      }
    }
  }
  if (e == 0) offsets[E] = P;
  const int flag = (e < E && cnt > 0) ? 1 : 0;
  int nact;
  const int pos = block_excl_scan(flag, wave_tot, &nact);
  if (active != nullptr) {
    if (flag) active[1 + pos] = e;
    if (e == 0) active[0] = nact;
  }
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t *__restrict__ ids, int T,
                                                          int k, int E,
                                                          const int32_t *__restrict__ blk,
                                                          int32_t *__restrict__ sorted_pair,
                                                          int32_t *__restrict__ pair_pos) {
  __shared__ int cur[1024];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cur[e] = blk[(long long)b * E + e];
  __syncthreads();
  const int t0 = b * TB;
  const int t1 = min(T, t0 + TB);
  for (int t = t0; t < t1; ++t) {
    if (lane < k) {
      const int p = t * k + lane;
      const int e = ids[p];
      if ((unsigned)e >= (unsigned)E) continue;
      const int pos = cur[e];
      cur[e] = pos + 1;  // a token holds each expert at most once
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
    // one wavefront: its LDS accesses complete in program order, so the next
    // token sees this token's increments
  }
}

// All three passes in one workgroup for a single block of tokens (T <= 64):
// histogram in LDS, the two scans, then wavefront 0 scatters the tokens in
// order.  Same results as the three kernels, one launch instead of three.
__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t *__restrict__ ids, int T, int k,
                                                          int E, int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ sorted_pair,
                                                          int32_t *__restrict__ pair_pos,
                                                          int32_t *__restrict__ active) {
  __shared__ int cur[1024];
  __shared__ int wave_tot[16];
  __shared__ int ids_lds[TB * 32];  // the block's ids, so the in-order scatter reads LDS only
  const int e = threadIdx.x;
  if (e < E) cur[e] = 0;
  __syncthreads();
  const int P = T * k;
  for (int i = threadIdx.x; i < P; i += 1024) {
    const int x = ids[i];
    ids_lds[i] = x;
    if ((unsigned)x < (unsigned)E) atomicAdd(&cur[x], 1);  // ids outside [0, E) are dropped
  }
  __syncthreads();
  const int cnt = e < E ? cur[e] : 0;
  int total;
  const int off = block_excl_scan(cnt, wave_tot, &total);
  if (e < E) {
    offsets[e] = off;
    cur[e] = off;  // this thread's own counter: the scan's barriers ordered every read of it
  }
  if (e == 0) offsets[E] = P;
  const int flag = (e < E && cnt > 0) ? 1 : 0;
  int nact;
  const int pos = block_excl_scan(flag, wave_tot, &nact);
  if (active != nullptr) {
    if (flag) active[1 + pos] = e;
    if (e == 0) active[0] = nact;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  for (int t = 0; t < T; ++t) {
    if (lane < k) {
      const int p = t * k + lane;
      const int x = ids_lds[p];
      if ((unsigned)x >= (unsigned)E) continue;
      const int q = cur[x];
      cur[x] = q + 1;  // a token holds each expert at most once
      sorted_pair[q] = p;
      pair_pos[p] = q;
    }
  }
}

}  // namespace

int permute_blocks(int T) { return (T + TB - 1) / TB; }

hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *blk, int32_t *offsets,
                          int32_t *sorted_pair, int32_t *pair_pos, int32_t *active,
                          hipStream_t st) {
  const int nblk = permute_blocks(T);
  if (nblk == 1) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), 0, st, ids, T, k, E, offsets, sorted_pair,
                       pair_pos, active);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_count_kernel, dim3(nblk), dim3(256), 0, st, ids, T, k, E, blk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, nblk, E, T * k, blk, offsets,
                     active);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nblk), dim3(64), 0, st, ids, T, k, E, blk,
                     sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
