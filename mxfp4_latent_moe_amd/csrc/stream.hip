// Streaming variant of the weight-stationary GEMM for chunks of at most 16
// token rows (decode-sized work): the weights are the whole cost, so the
// kernel is built to keep many weight bytes in flight.
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
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;

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

template <int WF, int AF, bool PAIR>
hipError_t launch_cfg(const GemmArgs &a, long long grid, hipStream_t st) {
  if constexpr (WF == W_MXFP4) {
    hipLaunchKernelGGL((stream_gemm_kernel<WF, AF, PAIR, 2, 4, STREAM_GROUPED_ROWS,
                                           STREAM_GROUPED_KSMAX, 4>),
                       dim3((unsigned)grid), dim3(256), 0, st, a);
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
