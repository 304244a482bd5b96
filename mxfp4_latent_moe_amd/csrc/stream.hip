// Streaming variants of the weight-stationary GEMM for chunks of at most 16
// token rows (decode-sized work): the weights are the whole cost, so the
// kernels are built to keep many weight bytes in flight.
//
// stream_gemm_kernel (one item per work-group) serves the grouped MXFP4
// products the persistent kernel does not take; the dense bf16 products run
// on stream_persist_kernel below (the one-item kernel remains their fallback).
//
//  * A workgroup's token rows (R rows per chunk) for its K slice sit in LDS
//    for the whole main loop: one barrier per workgroup, none per K step.
//    Expert GEMMs use R = 2 rows and the whole K range; dense products use
//    R = 16 and split K so the slice fits.
//  * Each wave streams its own weight rows through a D-deep ring of
//    registers: the load for K step q+D is issued right after step q is
//    consumed, with every load unconditional (indices clamped) so the
//    in-order memory counter lets D-1 steps stay in flight.
//  * MXFP4 weights are dequantised in registers (scaled fp4->bf16 convert);
//    MFMA 16x16x32 bf16 with weight rows as M and tokens as N.
//  * Partial sums of the K splits go to a workspace; a finalize pass adds the
//    splits in fixed order and applies the epilogue (SiTU-GLU or plain).
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;
#ifndef STREAM_USE_PERSIST
#define STREAM_USE_PERSIST 1
#endif
constexpr bool USE_PERSIST = STREAM_USE_PERSIST;

template <int WF, int AF, bool PAIR, int MT, int D, int R, int KSMAX, int NW>
__global__ __launch_bounds__(64 * NW) void stream_gemm_kernel(GemmArgs g) {
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int NTHR = 64 * NW;
  constexpr int ROWS_WG = 16 * NW * MT;
  constexpr int WREG = (WF == W_MXFP4) ? 1 : 4;
  // bf16 weights: a lane's four 16-byte loads of a K step sit 64 bytes apart, so
  // each instruction reads 64 contiguous bytes of every row (K octet 4 j + kg
  // for lane group kg in sub-step j); with 16-byte neighbours instead (octet
  // 4 kg + j) every instruction touched both lines of the row's 256 bytes and
  // the layer-0 FFN at T = 16 streamed 5% slower
  constexpr bool CONTIG = WF != W_MXFP4;
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;
  constexpr int STEP = 16 * R * 8;  // bf16 elements per K step per plane: [octet 16][row R][8]
  constexpr int NGRP = (R * KSMAX * 16 + NTHR - 1) / NTHR;  // 8-element groups staged per thread
  __shared__ __attribute__((aligned(16))) __bf16 lds[NPL][KSMAX * STEP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;

  const int per_chunk = g.n_blocks * g.splits;
  const int total = g.chunks ? min(*g.chunk_count * per_chunk, g.grid_logical) : g.grid_logical;
  const int logical = xcd_logical(total);
  if (logical < 0) return;
  const int chunk = logical / per_chunk;
  const int rem = logical - chunk * per_chunk;
  const int nb = rem / g.splits;
  const int split = rem - nb * g.splits;

  int expert, row0, nrows;
  if (g.chunks != nullptr) {
    const int4 c = reinterpret_cast<const int4 *>(g.chunks)[chunk];
    expert = c.x;
    row0 = c.y;
    nrows = c.z;
  } else {
    expert = 0;
    row0 = chunk * R;
    nrows = min(R, g.dense_rows - row0);
    if (nrows <= 0) return;
  }
  const int N = g.N, K = g.K;
  const int ksteps = K / KSTEP;
  const int ks0 = (split * ksteps) / g.splits;
  const int nks = ((split + 1) * ksteps) / g.splits - ks0;  // <= KSMAX (host guarantees)

  // ---- weight rows of this wave, read through buffer resources (base in
  // SGPRs, one 32-bit row offset per tile); the first D K steps are requested
  // before anything else
  const int wrow_base = nb * ROWS_WG + wave * 16 * MT;
  constexpr uint32_t STEP_BYTES = (WF == W_MXFP4) ? KSTEP / 2 : KSTEP * 2;
  const uint32_t row_bytes = (WF == W_MXFP4) ? K / 2 : K * 2;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const char *W = static_cast<const char *>(mat ? g.W1 : g.W0) +
                    expert * g.w_estride * ((WF == W_MXFP4) ? 1 : 2);
    wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
    if constexpr (WF == W_MXFP4) {
      const uint8_t *S = (mat ? g.S1 : g.S0) + expert * g.s_estride;
      sr[mat] = make_rsrc(S, (uint32_t)N * (K / 32));
    }
  }
  uint32_t woff[NTILE], soff[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int n = min(wrow_base + (t % MT) * 16 + r16, N - 1);
    woff[t] = (uint32_t)n * row_bytes + (uint32_t)ks0 * STEP_BYTES + kg * ((WF == W_MXFP4 || CONTIG) ? 16 : 64);
    soff[t] = (uint32_t)n * (K / 32) + ks0 * 4;
  }
  u32x4_t wq[D][NTILE][WREG];
  uint32_t wsc[D][NTILE];
  auto load_w = [&](int d, int q) {
    q = min(q, nks - 1);  // clamped: tail requests re-read the last step, always in bounds
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const int mat = t / MT;
#pragma unroll
      for (int j = 0; j < WREG; ++j) wq[d][t][j] = buf_load16(wr[mat], woff[t] + (CONTIG ? 64 : 16) * j, q * STEP_BYTES);
      if constexpr (WF == W_MXFP4) wsc[d][t] = buf_load4(sr[mat], soff[t], q * 4);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(d, d);

  // ---- the chunk's token rows for this K slice -> LDS (bf16, or bf16 hi + lo),
  // in passes of SG groups per thread to keep few registers live
  {
    constexpr int SG = 2;
    const int esz = (AF == A_BF16) ? 2 : 4;
    const int ngrp = R * nks * 16;
#pragma unroll 1
    for (int i0 = 0; i0 < NGRP; i0 += SG) {
      u32x4_t araw[SG][(AF == A_BF16) ? 1 : 2];
      int aoff[SG];
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        const int gi = tid + NTHR * (i0 + ii);  // group -> (K step q, octet, row r)
        const int r = gi % R;
        const int oct = (gi / R) & 15;
        const int q = gi / (16 * R);
        aoff[ii] = (gi < ngrp) ? q * STEP + (oct * R + r) * 8 : -1;
        araw[ii][0] = u32x4_t{0, 0, 0, 0};
        if constexpr (AF != A_BF16) araw[ii][1] = u32x4_t{0, 0, 0, 0};
        if (gi < ngrp && r < nrows) {
          const int p = row0 + r;
          const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
          const char *src = static_cast<const char *>(g.A) +
                            (arow * g.lda + (long long)(ks0 + q) * KSTEP + oct * 8) * esz;
          if constexpr (AF == A_BF16) {
            araw[ii][0] = *reinterpret_cast<const u32x4_t *>(src);
          } else {
            araw[ii][0] = reinterpret_cast<const u32x4_t *>(src)[0];
            araw[ii][1] = reinterpret_cast<const u32x4_t *>(src)[1];
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        if (aoff[ii] < 0) continue;
        if constexpr (AF == A_BF16) {
          *reinterpret_cast<u32x4_t *>(&lds[0][aoff[ii]]) = araw[ii][0];
        } else {
          bf16x8_t hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = __uint_as_float(e < 4 ? araw[ii][0][e] : araw[ii][1][e - 4]);
            if constexpr (AF == A_F32_SPLIT) {
              __bf16 h, l;
              split_bf16(f, h, l);
              hi[e] = h;
              lo[e] = l;
            } else {
              hi[e] = to_bf16(f);
            }
          }
          *reinterpret_cast<bf16x8_t *>(&lds[0][aoff[ii]]) = hi;
          if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(&lds[NPL - 1][aoff[ii]]) = lo;
        }
      }
    }
  }
  __syncthreads();
  // The staging above already waited for every load it issued (the newest
  // ones); saying so explicitly lets the waitcnt pass enter the main loop with
  // no pending writes, instead of merging them into a full wait at the loop
  // head on every iteration.
  __builtin_amdgcn_s_waitcnt(0);

  // hi and lo products accumulate separately so consecutive MFMAs never wait
  // on each other's result; they are added once at the end
  f32x4_t acc[NTILE], accl[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accl[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Lanes whose token column is >= R read row (r16 % R): those MFMA output
  // columns are never stored, so their B values need no zeroing.
  const int brow = r16 % R;
  auto compute = [&](int d, int q) {
    bf16x8_t bh[4], bl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = q * STEP + ((CONTIG ? 4 * j + kg : 4 * kg + j) * R + brow) * 8;
      bh[j] = *reinterpret_cast<const bf16x8_t *>(&lds[0][off]);
      if constexpr (NPL == 2) bl[j] = *reinterpret_cast<const bf16x8_t *>(&lds[1][off]);
    }
    float sc[NTILE];
    if constexpr (WF == W_MXFP4) {
#pragma unroll
      for (int t = 0; t < NTILE; ++t) sc[t] = e8m0_to_float((wsc[d][t] >> (8 * kg)) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t wa[NTILE];
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        if constexpr (WF == W_MXFP4) {
          wa[t] = fp4x8_to_bf16(wq[d][t][0][j], sc[t]);
        } else {
          wa[t] = __builtin_bit_cast(bf16x8_t, wq[d][t][j]);
        }
      }
#pragma unroll
      for (int t = 0; t < NTILE; ++t) acc[t] = mfma_16x16x32(wa[t], bh[j], acc[t]);
      if constexpr (NPL == 2) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) accl[t] = mfma_16x16x32(wa[t], bl[j], accl[t]);
      }
    }
  };

  // main loop: whole rings of D steps, every load unconditional
  const int nfull = nks - nks % D;
  for (int q0 = 0; q0 < nfull; q0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d, q0 + d);
      load_w(d, q0 + d + D);
    }
  }
  // remaining nks % D steps: their weights are already in the ring
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (nfull + d < nks) compute(d, nfull + d);

  if constexpr (NPL == 2) {
#pragma unroll
    for (int t = 0; t < NTILE; ++t) acc[t] += accl[t];
  }

  // ---- epilogue: lane holds token r16, weight rows 4*kg + 0..3 of each tile
  const int tok = r16;
  if (tok >= nrows) return;
  const long long orow = row0 + tok;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int col0 = wrow_base + m * 16 + 4 * kg;
    if (g.splits > 1) {
      const int ncols = PAIR ? 2 * N : N;
      float *pp = g.partial + ((long long)split * g.partial_rows + orow) * ncols;
      if (col0 + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<f32x4_t *>(pp + col0) = acc[m];
        if constexpr (PAIR) *reinterpret_cast<f32x4_t *>(pp + N + col0) = acc[m + MT];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (col0 + r < N) {
            pp[col0 + r] = acc[m][r];
            if constexpr (PAIR) pp[N + col0 + r] = acc[m + MT][r];
          }
        }
      }
      continue;
    }
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (PAIR) {
        v[r] = situ_glu(acc[m][r], acc[m + MT][r], g.beta, g.beta_lin);
      } else {
        v[r] = acc[m][r];
      }
    }
    if (g.rscale != nullptr) {
      const float rs = g.rscale[g.rscale_map ? g.rscale_map[orow] : orow];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] *= rs;
    }
    float *cp = g.C + orow * g.ldc + col0;
    if (col0 + 3 < N && (g.ldc & 3) == 0) {
      f32x4_t o = {v[0], v[1], v[2], v[3]};
      if (g.accumulate) o += *reinterpret_cast<const f32x4_t *>(cp);
      *reinterpret_cast<f32x4_t *>(cp) = o;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (col0 + r < N) cp[r] = g.accumulate ? cp[r] + v[r] : v[r];
    }
  }
}


// Persistent form for bf16 weights (the dense products of at most 64 token
// rows): one resident wave of work-groups, each taking a contiguous range of
// (K split, 16-row chunk, weight block) items in that order, so consecutive
// items share the staged token slice, and the weight ring runs on across item
// boundaries: the next item's first K steps are requested while the current
// one finishes.  A work-group pays the staging and the ring's fill once per
// slice instead of once per item.  Per K step a wave requests 256 contiguous
// bytes of each of its 16 weight rows per matrix (four 64-byte loads, K octet
// 4 j + kg in sub-step j); the arithmetic, the split-K partials and the
// epilogue are those of stream_gemm_kernel.
template <int AF, bool PAIR, int AHEAD, int NW>
__global__ __launch_bounds__(64 * NW) void stream_persist_kernel(GemmArgs g) {
  constexpr int R = 16;
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTHR = 64 * NW;
  constexpr int ROWS_WG = 16 * NW;
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;
  constexpr int STEP = 16 * R * 8;  // bf16 elements per K step per plane: [octet 16][row R][8]
  constexpr int KS = STREAM_KSMAX;
  constexpr uint32_t STEP_BYTES = KSTEP * 2;
  __shared__ __attribute__((aligned(16))) __bf16 lds[NPL][KS * STEP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int ksteps = K / KSTEP;
  const int n_chunks = (g.dense_rows + R - 1) / R;
  const int per_split = n_chunks * g.n_blocks;
  const int n_items = g.splits * per_split;
  const int G = gridDim.x;
  const int i_begin = (int)((long long)blockIdx.x * n_items / G);
  const int i_end = (int)((long long)(blockIdx.x + 1) * n_items / G);
  if (i_begin >= i_end) return;
  const uint32_t row_bytes = (uint32_t)K * 2;
  __amdgpu_buffer_rsrc_t wr[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) wr[mat] = make_rsrc(mat ? g.W1 : g.W0, (uint32_t)N * row_bytes);

  // ---- load cursor: item and K step of the next weight request
  int l_item = i_begin, l_q = 0, l_nks = 0;
  uint32_t woff[NMAT];
  auto set_load_item = [&](int it) {
    const int split = it / per_split;
    const int nb = (it - split * per_split) % g.n_blocks;
    const int ks0 = split * ksteps / g.splits;
    l_nks = (split + 1) * ksteps / g.splits - ks0;
    const int n = min(nb * ROWS_WG + wave * 16 + r16, N - 1);
#pragma unroll
    for (int t = 0; t < NMAT; ++t) woff[t] = (uint32_t)n * row_bytes + (uint32_t)ks0 * STEP_BYTES + kg * 16;
  };
  set_load_item(i_begin);
  // wq[0]: the step being computed; [1..AHEAD]: steps requested ahead.  Past
  // the last item the requests stay (the memory counter pattern is fixed) but
  // every lane reads the first 16 bytes.
  u32x4_t wq[AHEAD + 1][NMAT][4];
  auto load_step = [&](int bi) {
    const bool live = l_item < i_end;
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wq[bi][t][j] = buf_load16(wr[t], live ? woff[t] + 64 * j : 0u, live ? (uint32_t)l_q * STEP_BYTES : 0u);
    if (++l_q == l_nks) {
      l_q = 0;
      if (++l_item < i_end) set_load_item(l_item);
    }
  };

  // ---- compute cursor
  int staged = -1;  // split * n_chunks + chunk of the slice in LDS
  int c_split = 0, c_nb = 0, c_nks = 0, row0 = 0, nrows = 0;
  auto stage = [&](int ks0, int nks) {
    constexpr int SG = 2;
    constexpr int NGRP = (R * KS * 16 + NTHR - 1) / NTHR;  // 8-element groups per thread
    const int esz = (AF == A_BF16) ? 2 : 4;
    const int ngrp = R * nks * 16;
#pragma unroll 1
    for (int i0 = 0; i0 < NGRP; i0 += SG) {
      u32x4_t araw[SG][(AF == A_BF16) ? 1 : 2];
      int aoff[SG];
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        const int gi = tid + NTHR * (i0 + ii);  // group -> (K step q, octet, row r)
        const int r = gi % R;
        const int oct = (gi / R) & 15;
        const int q = gi / (16 * R);
        aoff[ii] = (gi < ngrp) ? q * STEP + (oct * R + r) * 8 : -1;
        araw[ii][0] = u32x4_t{0, 0, 0, 0};
        if constexpr (AF != A_BF16) araw[ii][1] = u32x4_t{0, 0, 0, 0};
        if (gi < ngrp && r < nrows) {
          const int p = row0 + r;
          const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
          const char *src = static_cast<const char *>(g.A) +
                            (arow * g.lda + (long long)(ks0 + q) * KSTEP + oct * 8) * esz;
          if constexpr (AF == A_BF16) {
            araw[ii][0] = *reinterpret_cast<const u32x4_t *>(src);
          } else {
            araw[ii][0] = reinterpret_cast<const u32x4_t *>(src)[0];
            araw[ii][1] = reinterpret_cast<const u32x4_t *>(src)[1];
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        if (aoff[ii] < 0) continue;
        if constexpr (AF == A_BF16) {
          *reinterpret_cast<u32x4_t *>(&lds[0][aoff[ii]]) = araw[ii][0];
        } else {
          bf16x8_t hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = __uint_as_float(e < 4 ? araw[ii][0][e] : araw[ii][1][e - 4]);
            if constexpr (AF == A_F32_SPLIT) {
              __bf16 h, l;
              split_bf16(f, h, l);
              hi[e] = h;
              lo[e] = l;
            } else {
              hi[e] = to_bf16(f);
            }
          }
          *reinterpret_cast<bf16x8_t *>(&lds[0][aoff[ii]]) = hi;
          if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(&lds[NPL - 1][aoff[ii]]) = lo;
        }
      }
    }
  };

  f32x4_t acc[NMAT], accl[NMAT];
  auto begin_item = [&](int it) {
    c_split = it / per_split;
    const int rem = it - c_split * per_split;
    const int chunk = rem / g.n_blocks;
    c_nb = rem - chunk * g.n_blocks;
    const int ks0 = c_split * ksteps / g.splits;
    c_nks = (c_split + 1) * ksteps / g.splits - ks0;
    row0 = chunk * R;
    nrows = min(R, g.dense_rows - row0);
    const int key = c_split * n_chunks + chunk;
    if (key != staged) {
      __syncthreads();  // every wave is done with the previous slice
      stage(ks0, c_nks);
      __syncthreads();
      staged = key;
    }
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
      acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accl[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // one K step from ring slot 0
  auto compute = [&](int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = q * STEP + ((4 * j + kg) * R + r16) * 8;
      const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&lds[0][off]);
      bf16x8_t bl;
      if constexpr (NPL == 2) bl = *reinterpret_cast<const bf16x8_t *>(&lds[1][off]);
#pragma unroll
      for (int t = 0; t < NMAT; ++t) {
        const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, wq[0][t][j]);
        acc[t] = mfma_16x16x32(wa, bh, acc[t]);
        if constexpr (NPL == 2) accl[t] = mfma_16x16x32(wa, bl, accl[t]);
      }
    }
  };

  // lane: token r16, weight rows 4 kg + 0..3 of its tile
  auto finish_item = [&]() {
    if constexpr (NPL == 2) {
#pragma unroll
      for (int t = 0; t < NMAT; ++t) acc[t] += accl[t];
    }
    const int tok = r16;
    if (tok >= nrows) return;
    const long long orow = row0 + tok;
    const int col0 = c_nb * ROWS_WG + wave * 16 + 4 * kg;
    if (g.splits > 1) {
      const int ncols = PAIR ? 2 * N : N;
      float *pp = g.partial + ((long long)c_split * g.partial_rows + orow) * ncols;
      if (col0 + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<f32x4_t *>(pp + col0) = acc[0];
        if constexpr (PAIR) *reinterpret_cast<f32x4_t *>(pp + N + col0) = acc[1];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (col0 + r < N) {
            pp[col0 + r] = acc[0][r];
            if constexpr (PAIR) pp[N + col0 + r] = acc[1][r];
          }
        }
      }
      return;
    }
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (PAIR) {
        v[r] = situ_glu(acc[0][r], acc[1][r], g.beta, g.beta_lin);
      } else {
        v[r] = acc[0][r];
      }
    }
    if (g.rscale != nullptr) {
      const float rs = g.rscale[g.rscale_map ? g.rscale_map[orow] : orow];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] *= rs;
    }
    float *cp = g.C + orow * g.ldc + col0;
    if (col0 + 3 < N && (g.ldc & 3) == 0) {
      f32x4_t o = {v[0], v[1], v[2], v[3]};
      if (g.accumulate) o += *reinterpret_cast<const f32x4_t *>(cp);
      *reinterpret_cast<f32x4_t *>(cp) = o;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (col0 + r < N) cp[r] = g.accumulate ? cp[r] + v[r] : v[r];
    }
  };

#pragma unroll
  for (int i = 1; i <= AHEAD; ++i) load_step(i);
  for (int it = i_begin; it < i_end; ++it) {
    begin_item(it);
    for (int q = 0; q < c_nks; ++q) {
      // the oldest requested step becomes the computed one (static indices)
#pragma unroll
      for (int i = 0; i < AHEAD; ++i)
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) wq[i][t][j] = wq[i + 1][t][j];
      load_step(AHEAD);
      compute(q);
    }
    finish_item();
  }
}

#ifndef STREAM_PERSIST_AHEAD
#define STREAM_PERSIST_AHEAD 2
#endif
constexpr int SP_AHEAD = STREAM_PERSIST_AHEAD;
constexpr int SP_WAVES = 4;

template <int AF, bool PAIR>
hipError_t launch_persist(const GemmArgs &a, hipStream_t st) {
  // every split owns at least one K step (the kernel walks each item's steps)
  // and at most the STREAM_KSMAX steps of the slice the kernel stages
  const int ksteps = a.K / KSTEP;
  if (a.K % KSTEP || a.splits < 1 || a.splits > ksteps || (ksteps + a.splits - 1) / a.splits > STREAM_KSMAX ||
      a.n_blocks < 1)
    return hipErrorInvalidValue;
  void *fn = reinterpret_cast<void *>(&stream_persist_kernel<AF, PAIR, SP_AHEAD, SP_WAVES>);
  // one resident wave of work-groups (occupancy queried once per kernel and device)
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int per_cu = cache[dev].load();
  if (per_cu == 0) {
    int blocks = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, 64 * SP_WAVES, 0);
    if (e != hipSuccess) return e;
    per_cu = blocks > 0 ? blocks : 1;
    cache[dev].store(per_cu);
  }
  static std::atomic<int> cus[64];
  int ncu = cus[dev].load();
  if (ncu == 0) {
    hipError_t e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus[dev].store(ncu);
  }
  const long long n_items = (long long)a.splits * ((a.dense_rows + 15) / 16) * a.n_blocks;
  long long grid = (long long)ncu * per_cu;
  if (grid > n_items) grid = n_items;
  if (grid < 1) grid = 1;
  GemmArgs args = a;
  void *params[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * SP_WAVES), params, 0, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <int WF, int AF, bool PAIR>
hipError_t launch_cfg(const GemmArgs &a, long long grid, hipStream_t st) {
  if constexpr (WF == W_MXFP4) {
    hipLaunchKernelGGL((stream_gemm_kernel<WF, AF, PAIR, 2, 4, STREAM_GROUPED_ROWS,
                                           STREAM_GROUPED_KSMAX, 4>),
                       dim3((unsigned)grid), dim3(256), 0, st, a);
  } else if (USE_PERSIST && a.chunks == nullptr && a.dense_rows > 0 && a.splits <= a.K / KSTEP) {
    return launch_persist<AF, PAIR>(a, st);
  } else {
    hipLaunchKernelGGL((stream_gemm_kernel<WF, AF, PAIR, 1, 3, 16, STREAM_KSMAX, 4>),
                       dim3((unsigned)grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int WF, int AF>
hipError_t launch_pair(bool pair, const GemmArgs &a, long long grid, hipStream_t st) {
  return pair ? launch_cfg<WF, AF, true>(a, grid, st) : launch_cfg<WF, AF, false>(a, grid, st);
}

template <int WF>
hipError_t launch_af(int afmt, bool pair, const GemmArgs &a, long long grid, hipStream_t st) {
  switch (afmt) {
    case A_BF16: return launch_pair<WF, A_BF16>(pair, a, grid, st);
    case A_F32_SPLIT: return launch_pair<WF, A_F32_SPLIT>(pair, a, grid, st);
    default: return launch_pair<WF, A_F32_ROUND>(pair, a, grid, st);
  }
}

}  // namespace

int stream_rows_per_wg(int wfmt, bool pair) {
  (void)pair;
  const int mt = (wfmt == W_MXFP4) ? 2 : 1;
  return 64 * mt;
}

hipError_t launch_stream_gemm(int wfmt, int afmt, bool pair, const GemmArgs &a, long long grid,
                              hipStream_t st) {
  if (wfmt == W_MXFP4) return launch_af<W_MXFP4>(afmt, pair, a, grid, st);
  return launch_af<W_BF16>(afmt, pair, a, grid, st);
}

}  // namespace moe
