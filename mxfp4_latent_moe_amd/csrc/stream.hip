// Streaming variant of the weight-stationary GEMM for chunks of at most 16
// token rows (decode-sized work): the weights are the whole cost, so the
// kernel is built to keep many weight bytes in flight.
//
//  * K is split across workgroups so that one workgroup's slice of the token
//    rows (<= 16 rows x KSMAX*128 K values, bf16 or bf16 hi+lo) sits in LDS
//    for the whole main loop: one barrier per workgroup, none per K step.
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

template <int WF, int AF, bool PAIR, int MT, int D, int KSMAX>
__global__ __launch_bounds__(256) void stream_gemm_kernel(GemmArgs g) {
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int ROWS_WG = 64 * MT;
  constexpr int WREG = (WF == W_MXFP4) ? 1 : 4;
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;
  constexpr int STEP = 16 * KSTEP;  // bf16 elements per K step per plane: [octet][token][8]
  __shared__ __attribute__((aligned(16))) __bf16 lds[NPL][KSMAX * STEP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;

  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int logical = (b & 7) * (G >> 3) + (b >> 3);
  if (logical >= g.grid_logical) return;
  const int per_chunk = g.n_blocks * g.splits;
  const int chunk = logical / per_chunk;
  const int rem = logical - chunk * per_chunk;
  const int nb = rem / g.splits;
  const int split = rem - nb * g.splits;

  int expert, row0, nrows;
  if (g.chunks != nullptr) {
    if (chunk >= *g.chunk_count) return;
    const int4 c = reinterpret_cast<const int4 *>(g.chunks)[chunk];
    expert = c.x;
    row0 = c.y;
    nrows = c.z;
  } else {
    expert = 0;
    row0 = chunk * 16;
    nrows = min(16, g.dense_rows - row0);
    if (nrows <= 0) return;
  }
  const int N = g.N, K = g.K;
  const int ksteps = K / KSTEP;
  const int ks0 = (split * ksteps) / g.splits;
  const int nks = ((split + 1) * ksteps) / g.splits - ks0;  // <= KSMAX (host guarantees)

  // ---- activation rows of the chunk for this K slice: thread = (token tid/16, octet tid%16)
  {
    const int r = tid >> 4;
    const int oct = tid & 15;
    const int esz = (AF == A_BF16) ? 2 : 4;
    const char *src = nullptr;
    if (r < nrows) {
      const int p = row0 + r;
      const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
      src = static_cast<const char *>(g.A) + (arow * g.lda + (long long)ks0 * KSTEP + oct * 8) * esz;
    }
    u32x4_t araw[KSMAX][(AF == A_BF16) ? 1 : 2];
#pragma unroll
    for (int q = 0; q < KSMAX; ++q) {
      if (q < nks && src != nullptr) {
        if constexpr (AF == A_BF16) {
          araw[q][0] = *reinterpret_cast<const u32x4_t *>(src + (long long)q * KSTEP * 2);
        } else {
          const u32x4_t *p4 = reinterpret_cast<const u32x4_t *>(src + (long long)q * KSTEP * 4);
          araw[q][0] = p4[0];
          araw[q][1] = p4[1];
        }
      } else {
        araw[q][0] = u32x4_t{0, 0, 0, 0};
        if constexpr (AF != A_BF16) araw[q][1] = u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int q = 0; q < KSMAX; ++q) {
      if (q < nks) {
        const int off = q * STEP + (oct * 16 + r) * 8;
        if constexpr (AF == A_BF16) {
          *reinterpret_cast<u32x4_t *>(&lds[0][off]) = araw[q][0];
        } else {
          bf16x8_t hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = __uint_as_float(e < 4 ? araw[q][0][e] : araw[q][1][e - 4]);
            if constexpr (AF == A_F32_SPLIT) {
              __bf16 h, l;
              split_bf16(f, h, l);
              hi[e] = h;
              lo[e] = l;
            } else {
              hi[e] = to_bf16(f);
            }
          }
          *reinterpret_cast<bf16x8_t *>(&lds[0][off]) = hi;
          if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(&lds[NPL - 1][off]) = lo;
        }
      }
    }
  }

  // ---- weight rows of this wave
  const int wrow_base = nb * ROWS_WG + wave * 16 * MT;
  const uint8_t *wptr8[NTILE];
  const uint8_t *sptr[NTILE];
  const __bf16 *wptr16[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int m = t % MT;
    const int mat = t / MT;
    const int n = min(wrow_base + m * 16 + r16, N - 1);
    if constexpr (WF == W_MXFP4) {
      const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0);
      const uint8_t *S = mat ? g.S1 : g.S0;
      wptr8[t] = W + expert * g.w_estride + (long long)n * (K / 2) + (long long)ks0 * 64 + kg * 16;
      sptr[t] = S + expert * g.s_estride + (long long)n * (K / 32) + ks0 * 4;
      wptr16[t] = nullptr;
    } else {
      const __bf16 *W = static_cast<const __bf16 *>(mat ? g.W1 : g.W0);
      wptr16[t] = W + expert * g.w_estride + (long long)n * K + (long long)ks0 * KSTEP + kg * 32;
      wptr8[t] = nullptr;
      sptr[t] = nullptr;
    }
  }

  u32x4_t wq[D][NTILE][WREG];
  uint32_t wsc[D][NTILE];
  auto load_w = [&](int d, int q) {
    q = min(q, nks - 1);  // clamped: tail loads re-read the last step, always in bounds
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      if constexpr (WF == W_MXFP4) {
        wq[d][t][0] = *reinterpret_cast<const u32x4_t *>(wptr8[t] + (long long)q * 64);
        wsc[d][t] = *reinterpret_cast<const uint32_t *>(sptr[t] + q * 4);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wq[d][t][j] = *reinterpret_cast<const u32x4_t *>(wptr16[t] + (long long)q * KSTEP + 8 * j);
      }
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(d, d);

  __syncthreads();

  f32x4_t acc[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int q0 = 0; q0 < nks; q0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int q = q0 + d;
      if (q < nks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int off = q * STEP + ((4 * kg + j) * 16 + r16) * 8;
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&lds[0][off]);
          bf16x8_t bl;
          if constexpr (NPL == 2) bl = *reinterpret_cast<const bf16x8_t *>(&lds[1][off]);
#pragma unroll
          for (int t = 0; t < NTILE; ++t) {
            bf16x8_t wa;
            if constexpr (WF == W_MXFP4) {
              wa = fp4x8_to_bf16(wq[d][t][0][j], e8m0_to_float((wsc[d][t] >> (8 * kg)) & 0xFFu));
            } else {
              wa = __builtin_bit_cast(bf16x8_t, wq[d][t][j]);
            }
            acc[t] = mfma_16x16x32(wa, bh, acc[t]);
            if constexpr (NPL == 2) acc[t] = mfma_16x16x32(wa, bl, acc[t]);
          }
        }
        load_w(d, q + D);
      }
    }
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
      if (col0 + 3 < N) {
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
    if (col0 + 3 < N) {
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
    hipLaunchKernelGGL((stream_gemm_kernel<WF, AF, PAIR, PAIR ? 2 : 4, 4, STREAM_KSMAX>),
                       dim3((unsigned)grid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((stream_gemm_kernel<WF, AF, PAIR, PAIR ? 1 : 2, 2, STREAM_KSMAX>),
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
  const int mt = (wfmt == W_MXFP4) ? (pair ? 2 : 4) : (pair ? 1 : 2);
  return 64 * mt;
}

hipError_t launch_stream_gemm(int wfmt, int afmt, bool pair, const GemmArgs &a, long long grid,
                              hipStream_t st) {
  if (wfmt == W_MXFP4) return launch_af<W_MXFP4>(afmt, pair, a, grid, st);
  return launch_af<W_BF16>(afmt, pair, a, grid, st);
}

}  // namespace moe
