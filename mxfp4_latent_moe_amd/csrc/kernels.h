// Kernel argument blocks and host-side launch helpers shared by the HIP
// sources and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// weight formats, activation formats
// W_AFF2: affine 2-bit codes [E][N][K/4] (element 4b + i in bits 2i..2i+1 of
// byte b), bf16 scales and biases [E][N][K/64]: w = scale * q + bias
enum { W_BF16 = 0, W_MXFP4 = 1, W_AFF2 = 2 };
enum { A_BF16 = 0, A_F32_SPLIT = 1, A_F32_ROUND = 2, A_MX8X3 = 3, A_MX6X3 = 4 };

// Weight-stationary GEMM: C[row, n] (+)= sum_k A[row, k] * W[n, k] over a
// list of row chunks, optionally with two weight matrices combined by
// SiTU-GLU.  Work item = (row chunk, block of weight rows, K split).
struct GemmArgs {
  const void *A;          // activations [rows, K], bf16 or fp32
  long long lda;          // elements per activation row
  const int32_t *a_map;   // chunk row p reads A row a_map[p] / a_div (NULL: row p)
  int a_div;
  long long a_rows;       // rows of A (grouped calls; gathered reads stay below it)
  const void *W0, *W1;    // weights [E][N][K] bf16 or packed [E][N][K/2]; W1 for SiTU pairs
  const uint8_t *S0, *S1; // e8m0 scales [E][N][K/32] (MXFP4), bf16 scales [E][N][K/64] (W_AFF2)
  const uint16_t *B0, *B1; // bf16 biases [E][N][K/64] (W_AFF2)
  const float *asum;      // W_AFF2 on the plane kernel: 64-element group sums of A's rows [rows][K/64]
  int asum_sorted;        // asum rows follow the sorted rows (a_map not applied to them)
  // dense tiled kernel, SiTU pairs with whole K: the result as bf16 planes
  // c_hi = bf16(v), c_lo = bf16(v - c_hi) ([rows][ldc] each; c_lo NULL: the
  // rounded plane only) instead of fp32 C
  uint16_t *c_hi, *c_lo;
  long long w_estride;    // per-expert stride of W (elements for bf16, bytes for packed)
  long long s_estride;    // per-expert stride of S in bytes
  int N, K;
  float *C;
  long long ldc;
  int accumulate;
  const float *rscale;    // optional row scale rscale[rscale_map[row]]
  const int32_t *rscale_map;
  const int32_t *chunks;  // grouped: int4 {expert, row0, nrows, 0} per chunk (NULL: dense)
  const int32_t *chunk_count;
  int dense_rows;         // dense: number of rows, chunked by the tile height
  int n_blocks, splits, grid_logical;
  float *partial;         // split-K partial sums [splits][partial_rows][ncols]
  int partial_rows;
  float beta, beta_lin;
  // MX activations (A_MX8X3, A_MX6X3): three e4m3 or packed e2m3 term planes
  // [3][mx_rows][K] and their e8m0 block scales [3][mx_rows][K/32]; A is
  // unused then
  const uint8_t *mxq, *mxs;
  long long mx_rows;
  // dense tiled kernel: the lo plane of split activations (A holds the hi
  // plane, both bf16 [rows][lda]) and the number of 256-row token tiles
  const void *A2;
  int dense_rows_tiles;
};

struct FinalizeArgs {
  const float *partial;
  int splits, rows, N;
  int pair;               // partial holds [G | U] (2N columns) to combine by SiTU-GLU
  float *C;
  long long ldc;
  int accumulate;
  const float *rscale;    // optional row scale rscale[rscale_map[row]]
  const int32_t *rscale_map;
  float beta, beta_lin;
};

// K steps (of 128) one streaming workgroup keeps in LDS; K is split so that
// no split exceeds it.
constexpr int STREAM_KSMAX = 8;
// Streaming expert GEMMs: rows per chunk and the K steps one workgroup holds
// (the whole K of the K3 expert matrices: 3584 / 128 = 28).
constexpr int STREAM_GROUPED_ROWS = 2;
constexpr int STREAM_GROUPED_KSMAX = 32;
// persistent grouped kernel: rows per chunk (decode segments rarely exceed 4)
constexpr int PERSIST_ROWS = 4;
// the same kernel over chunks of up to 8 rows: the small experts of a batch
// whose other experts run on the tiled kernel
constexpr int PERSIST_ROWS_WIDE = 8;
// tiled prefill kernel: 16-token tiles per chunk, 16-row weight tiles per wave
// and matrix, waves per work-group
constexpr int PREFILL_NT = 6;
constexpr int PREFILL_MX_NW = 4;  // MX-scaled variant: one wave per SIMD
constexpr int PREFILL_MX_MT_PAIR = 4;
constexpr int PREFILL_MX_MT_SINGLE = 8;

// kernel variant selection (host side)
struct GemmPlan {
  int variant;   // 0: tiled (LDS-staged K steps), 1: streaming (<= 16-row chunks),
                 // 2: persistent streaming over expert row chunks, 3: tiled prefill,
                 // 4: dense 256 x 256 tiles (bf16 activation planes)
  int nt;        // 16-token tiles per chunk (1 or 8)
  int mt;        // 16-row weight tiles per wave and matrix
  int chunk_rows;
  int n_blocks;
  int splits;
  int max_chunks;
  long long grid_logical;
  size_t partial_bytes;
};

GemmPlan plan_dense(int rows, int N, int K, bool pair);
GemmPlan plan_grouped(int P, int E, int N, int K, bool pair);

int stream_rows_per_wg(int wfmt, bool pair);
int grouped_stream_rows_per_wg(bool pair, int rows = PERSIST_ROWS);
bool grouped_stream_fits(int K);
// rows: chunk rows the kernel stages (PERSIST_ROWS, or PERSIST_ROWS_WIDE for MXFP4)
hipError_t launch_grouped_stream(int wfmt, int afmt, bool pair, const GemmArgs &a, hipStream_t st,
                                 int rows = PERSIST_ROWS);
int prefill_mx_rows_per_wg(bool pair);
// tiled prefill kernel over bf16 activation planes ([rows][npl][K]: hi then lo,
// or the rounded row), MXFP4 or affine 2-bit weights (affine: a.asum holds the
// activation rows' 64-element group sums); the fp32 -> planes split (with the
// group sums when sums != nullptr; out == nullptr: sums only) and the group
// sums of bf16 rows
int prefill_pl_rows_per_wg(bool pair, int wfmt);
hipError_t launch_prefill_planes(int wfmt, int npl, bool pair, const GemmArgs &a, long long grid, hipStream_t st);
size_t split_rows_bytes(long long rows, int K, int npl);
size_t row_sums_bytes(long long rows, int K);
// map != nullptr: output row r is activation row map[r] / div
hipError_t launch_split_rows(int npl, const float *A, long long lda, long long rows, int K, const int32_t *map,
                             int div, uint16_t *out, float *sums, hipStream_t st);
hipError_t launch_row_sums(const uint16_t *A, long long lda, long long rows, int K, const int32_t *map, int div,
                           float *sums, hipStream_t st);
// the MX-scaled tiled kernel (A_MX8X3 / A_MX6X3 activations, MXFP4 weights)
hipError_t launch_prefill_gemm(int wfmt, int afmt, bool pair, const GemmArgs &a, long long grid,
                               hipStream_t st);
size_t mx8_split_bytes(long long rows, int K);
// map != nullptr: term row r is activation row map[r] / div
hipError_t launch_mx_split(bool fp6, const float *A, long long lda, int rows, int K, const int32_t *map, int div,
                           uint8_t *ws, hipStream_t st);
hipError_t launch_stream_gemm(int wfmt, int afmt, bool pair, const GemmArgs &a, long long grid,
                              hipStream_t st);
int dense_tile_cols(bool pair);
int dense_tile_rows();
hipError_t launch_dense_tile(int nplanes, bool pair, const GemmArgs &a, hipStream_t st);
hipError_t launch_split_planes(const float *A, long long lda, int rows, int K, uint16_t *hi, uint16_t *lo,
                               hipStream_t st);

hipError_t launch_gemm(const GemmPlan &pl, int wfmt, int afmt, bool pair, const GemmArgs &a,
                       hipStream_t st);
hipError_t launch_finalize(const FinalizeArgs &f, hipStream_t st);
// experts with fewer than min_rows or more than max_rows rows get no chunks
hipError_t launch_plan_chunks(const int32_t *offsets, int E, int chunk_rows, int32_t *chunks,
                              int32_t *count, hipStream_t st, int min_rows = 1, int max_rows = 1 << 30);

// partial != nullptr: logits are the sum of `splits` split-K partials [splits][T][E]
// (logits unused); promoted == nullptr: no cap
hipError_t launch_topk(const float *logits, const float *partial, int splits, const float *bias, int T, int E,
                       int k, int32_t *ids, float *w, float *gap, const uint8_t *promoted, int k_hi,
                       hipStream_t st);

// permutation: workspace holds blk_counts [nblk][E] int32
int permute_blocks(int T);
hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *blk, int32_t *offsets,
                          int32_t *sorted_pair, int32_t *pair_pos, int32_t *active,
                          hipStream_t st);

hipError_t launch_reap(const float *Y, int P, int L, const float *pair_weight, const int32_t *sorted_pair,
                       const int32_t *offsets, int E, double *sal_sum, long long *counts, int accumulate,
                       float *contrib, hipStream_t st);

// contrib != nullptr: also g * ||Y row||_2 per sorted row (L <= 4096)
hipError_t launch_combine_norm(const float *Y, const int32_t *pair_pos, const float *w,
                               const uint16_t *gamma, int T, int k, int L, float eps, float *yn,
                               float *contrib, hipStream_t st);
// the combine writing y_n as bf16 planes hi = bf16(y_n), lo = bf16(y_n - hi) ([T][L] each; lo NULL:
// the rounded plane only), for L <= 4096
hipError_t launch_combine_norm_planes(const float *Y, const int32_t *pair_pos, const float *w,
                                      const uint16_t *gamma, int T, int k, int L, float eps, uint16_t *hi,
                                      uint16_t *lo, hipStream_t st);
// the per-expert pass of launch_reap alone, over contributions already made
hipError_t launch_reap_experts(const float *contrib, const int32_t *offsets, int E, double *sal_sum,
                               long long *counts, int accumulate, hipStream_t st);

}  // namespace moe
