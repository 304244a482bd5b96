// Weight-stationary MFMA GEMM for gfx950, shared by the MXFP4 grouped expert
// GEMMs and the bf16 dense products of the layer.
//
// Orientation: weight rows are the MFMA's M side, tokens its N side.  Each
// wave owns 16*MT weight rows (per matrix) and streams them straight from HBM
// into registers -- for MXFP4 a lane's 16-byte load is one full 32-element
// scale group of one row, dequantised in registers with the hardware
// fp4->bf16 scaled convert; the e8m0 byte is used as the scale exponent as-is.
// The chunk's token rows (activations) are staged through LDS once per
// 128-wide K step and shared by the four waves.  fp32 activations are split
// into bf16 hi + lo planes (two MFMAs per product) or rounded once, as asked.
//
// K ordering inside a 128-wide K step: lane group g = lane/16 owns K offsets
// 32g .. 32g+31 (one scale group); MFMA sub-step j uses offsets 32g+8j .. +7.
// The activation tile in LDS is stored as [octet 0..15][token][8], octet =
// K offset / 8, so that sixteen lanes of one group read 256 contiguous bytes.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int KSTEP = 128;

template <int WF, int AF, bool PAIR, int NT, int MT>
__global__ __launch_bounds__(256) void ws_gemm_kernel(GemmArgs g) {
  constexpr int C = 16 * NT;                       // chunk height (tokens)
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1; // LDS planes (hi, lo)
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;                 // weight tiles per wave
  constexpr int ROWS_WG = 64 * MT;                 // weight rows per matrix per workgroup
  constexpr int PLANE = C * KSTEP;                 // bf16 elements per plane per stage
  constexpr int WREG = (WF == W_MXFP4) ? 1 : 4;    // 16-byte loads per tile per K step
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][NPL][PLANE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;

  // XCD-aware remap over the real work items (one chunk's weight blocks share an L2)
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
    row0 = chunk * C;
    nrows = min(C, g.dense_rows - row0);
    if (nrows <= 0) return;
  }
  const int nt_active = (nrows + 15) >> 4;
  const int N = g.N, K = g.K;
  const int ksteps = K / KSTEP;
  const int ks0 = (split * ksteps) / g.splits;
  const int ks1 = ((split + 1) * ksteps) / g.splits;

  // ---- weight row pointers (rows clamped to N-1 for loads, masked at store)
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
      wptr8[t] = W + expert * g.w_estride + (long long)n * (K / 2) + kg * 16;
      sptr[t] = S + expert * g.s_estride + (long long)n * (K / 32);
      wptr16[t] = nullptr;
    } else {
      const __bf16 *W = static_cast<const __bf16 *>(mat ? g.W1 : g.W0);
      wptr16[t] = W + expert * g.w_estride + (long long)n * K + kg * 32;
      wptr8[t] = nullptr;
      sptr[t] = nullptr;
    }
  }

  // ---- activation rows staged by this thread: rows (tid/16) + 16 i, octet tid%16
  const int a_oct = tid & 15;
  const char *a_src[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int r = (tid >> 4) + 16 * i;
    a_src[i] = nullptr;
    if (r < nrows) {
      const int p = row0 + r;
      const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
      const int esz = (AF == A_BF16) ? 2 : 4;
      a_src[i] = static_cast<const char *>(g.A) + (arow * g.lda + a_oct * 8) * esz;
    }
  }

  u32x4_t wq[NTILE][WREG];
  uint32_t wsc[NTILE];
  u32x4_t aq[NT][(AF == A_BF16) ? 1 : 2];

  auto load_w = [&](int s) {
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      if constexpr (WF == W_MXFP4) {
        wq[t][0] = *reinterpret_cast<const u32x4_t *>(wptr8[t] + (long long)s * 64);
        const uint32_t sv = *reinterpret_cast<const uint32_t *>(sptr[t] + s * 4);
        wsc[t] = (sv >> (8 * kg)) & 0xFFu;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wq[t][j] = *reinterpret_cast<const u32x4_t *>(wptr16[t] + (long long)s * KSTEP + 8 * j);
      }
    }
  };
  auto load_a = [&](int s) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (a_src[i] != nullptr) {
        if constexpr (AF == A_BF16) {
          aq[i][0] = *reinterpret_cast<const u32x4_t *>(a_src[i] + (long long)s * KSTEP * 2);
        } else {
          const u32x4_t *p = reinterpret_cast<const u32x4_t *>(a_src[i] + (long long)s * KSTEP * 4);
          aq[i][0] = p[0];
          aq[i][1] = p[1];
        }
      } else {
        aq[i][0] = u32x4_t{0, 0, 0, 0};
        if constexpr (AF != A_BF16) aq[i][1] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int r = (tid >> 4) + 16 * i;
      const int off = (a_oct * C + r) * 8;
      if constexpr (AF == A_BF16) {
        *reinterpret_cast<u32x4_t *>(&lds[buf][0][off]) = aq[i][0];
      } else {
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = __uint_as_float(aq[i][0][e]);
          f[4 + e] = __uint_as_float(aq[i][1][e]);
        }
        bf16x8_t hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (AF == A_F32_SPLIT) {
            __bf16 h, l;
            split_bf16(f[e], h, l);
            hi[e] = h;
            lo[e] = l;
          } else {
            hi[e] = to_bf16(f[e]);
          }
        }
        *reinterpret_cast<bf16x8_t *>(&lds[buf][0][off]) = hi;
        if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(&lds[buf][NPL - 1][off]) = lo;
      }
    }
  };

  f32x4_t acc[NTILE][NT];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ks0 < ks1) {
    load_w(ks0);
    load_a(ks0);
    store_a(0);
  }
  __syncthreads();

  for (int s = ks0; s < ks1; ++s) {
    const int buf = (s - ks0) & 1;
    u32x4_t wcur[NTILE][WREG];
    uint32_t sccur[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      sccur[t] = wsc[t];
#pragma unroll
      for (int j = 0; j < WREG; ++j) wcur[t][j] = wq[t][j];
    }
    const bool more = (s + 1 < ks1);
    if (more) {
      load_w(s + 1);
      load_a(s + 1);
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t wa[NTILE];
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        if constexpr (WF == W_MXFP4) {
          wa[t] = fp4x8_to_bf16(wcur[t][0][j], e8m0_to_float(sccur[t]));
        } else {
          wa[t] = __builtin_bit_cast(bf16x8_t, wcur[t][j]);
        }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n < nt_active) {
          const int off = ((4 * kg + j) * C + 16 * n + r16) * 8;
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&lds[buf][0][off]);
#pragma unroll
          for (int t = 0; t < NTILE; ++t) acc[t][n] = mfma_16x16x32(wa[t], bh, acc[t][n]);
          if constexpr (NPL == 2) {
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&lds[buf][1][off]);
#pragma unroll
            for (int t = 0; t < NTILE; ++t) acc[t][n] = mfma_16x16x32(wa[t], bl, acc[t][n]);
          }
        }
      }
    }
    if (more) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds token (16n + r16), weight rows 4*kg + 0..3 of each tile
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int col0 = wrow_base + m * 16 + 4 * kg;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int tok = 16 * n + r16;
      if (n >= nt_active || tok >= nrows) continue;
      const long long orow = row0 + tok;
      if (g.splits > 1) {
        const int ncols = PAIR ? 2 * N : N;
        float *pp = g.partial + ((long long)split * g.partial_rows + orow) * ncols;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (col0 + r < N) {
            pp[col0 + r] = acc[m][n][r];
            if constexpr (PAIR) pp[N + col0 + r] = acc[m + MT][n][r];
          }
        }
        continue;
      }
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (PAIR) {
          v[r] = situ_glu(acc[m][n][r], acc[m + MT][n][r], g.beta, g.beta_lin);
        } else {
          v[r] = acc[m][n][r];
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
}

__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs f) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)f.rows * f.N;
  if (i >= total) return;
  const long long row = i / f.N;
  const int col = (int)(i - row * f.N);
  const int ncols = f.pair ? 2 * f.N : f.N;
  float a = 0.f, u = 0.f;
  for (int s = 0; s < f.splits; ++s) {
    const float *p = f.partial + ((long long)s * f.rows + row) * ncols;
    a += p[col];
    if (f.pair) u += p[f.N + col];
  }
  float v = f.pair ? situ_glu(a, u, f.beta, f.beta_lin) : a;
  if (f.rscale != nullptr) v *= f.rscale[f.rscale_map ? f.rscale_map[row] : row];
  float *c = f.C + row * f.ldc + col;
  *c = f.accumulate ? *c + v : v;
}

// One workgroup: chunk list {expert, row0, nrows, 0} in expert order from the
// expert offsets, chunks of at most `chunk_rows` rows, for the experts whose
// row count lies in [min_rows, max_rows].
__global__ __launch_bounds__(1024) void plan_chunks_kernel(const int32_t *offsets, int E,
                                                           int chunk_rows, int32_t *chunks,
                                                           int32_t *count, int min_rows, int max_rows) {
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tid;
  int ne = 0, nch = 0;
  if (e < E) {
    ne = offsets[e + 1] - offsets[e];
    nch = (ne < min_rows || ne > max_rows) ? 0 : (ne + chunk_rows - 1) / chunk_rows;
  }
  // inclusive wave scan
  int x = nch;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const int base = before + x - nch;
  for (int i = 0; i < nch; ++i) {
    int4 c;
    c.x = e;
    c.y = offsets[e] + i * chunk_rows;
    c.z = min(chunk_rows, ne - i * chunk_rows);
    c.w = 0;
    reinterpret_cast<int4 *>(chunks)[base + i] = c;
  }
  if (tid == 1023) {
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += wave_tot[w];
    *count = tot;
  }
}

template <int WF, int AF, bool PAIR, int NT, int MT>
hipError_t launch_variant(const GemmArgs &a, long long grid, hipStream_t st) {
  hipLaunchKernelGGL((ws_gemm_kernel<WF, AF, PAIR, NT, MT>), dim3((unsigned)grid), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

template <int WF, int AF, bool PAIR>
hipError_t launch_nt(const GemmPlan &pl, const GemmArgs &a, long long grid, hipStream_t st) {
  (void)pl;
  return launch_variant<WF, AF, PAIR, 8, 2>(a, grid, st);
}

template <int WF, int AF>
hipError_t launch_pair(const GemmPlan &pl, bool pair, const GemmArgs &a, long long grid,
                       hipStream_t st) {
  return pair ? launch_nt<WF, AF, true>(pl, a, grid, st) : launch_nt<WF, AF, false>(pl, a, grid, st);
}

template <int WF>
hipError_t launch_af(const GemmPlan &pl, int afmt, bool pair, const GemmArgs &a, long long grid,
                     hipStream_t st) {
  switch (afmt) {
    case A_BF16: return launch_pair<WF, A_BF16>(pl, pair, a, grid, st);
    case A_F32_SPLIT: return launch_pair<WF, A_F32_SPLIT>(pl, pair, a, grid, st);
    default: return launch_pair<WF, A_F32_ROUND>(pl, pair, a, grid, st);
  }
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

GemmPlan plan_dense(int rows, int N, int K, bool pair) {
  GemmPlan p{};
  const int ksteps = K / KSTEP;
  if (rows <= 64) {
    // streaming variant: 16-row chunks, K split so each split fits in LDS and
    // the grid fills the chip
    p.variant = 1;
    p.nt = 1;
    p.chunk_rows = 16;
    p.mt = stream_rows_per_wg(W_BF16, pair) / 64;
    p.n_blocks = ceil_div(N, stream_rows_per_wg(W_BF16, pair));
    p.max_chunks = ceil_div(rows, 16);
    const long long items = (long long)p.max_chunks * p.n_blocks;
    int splits = ceil_div(ksteps, STREAM_KSMAX);
    // a split below 8 K steps only pays while the grid would not cover the
    // CUs: each work-group stages its token slice before streaming, and short
    // streams spend more of their time in that ramp (measured on the shared
    // experts at T = 16: 124 us with 2048 items, 86 us with 256)
    while (items * splits < 256 && ceil_div(ksteps, splits * 2) >= 2) splits *= 2;
    p.splits = splits;
    p.grid_logical = items * splits;
  } else if (rows >= 128 && (long long)rows * K * 2 < (1LL << 31) && (long long)N * K * 2 < (1LL << 31)) {
    // 256 x 256 tiles; K is split while the tiles alone leave CUs idle.  From
    // 128 rows on: at batched-decode sizes (T = 256) the mid-size kernel took
    // the latent projection 122 us plus a 65 us finalize of 16 partials; on
    // these tiles (K split 8 ways) the batched-decode step went from 3.52 to
    // 3.06 ms
    p.variant = 4;
    p.nt = 16;
    p.chunk_rows = dense_tile_rows();
    p.mt = 0;
    p.n_blocks = ceil_div(N, dense_tile_cols(pair));
    p.max_chunks = ceil_div(rows, p.chunk_rows);
    const long long items = (long long)p.max_chunks * p.n_blocks;
    // K is split only while the tiles leave CUs idle, and a split is taken
    // only where it halves the time of the rounds of work over the 256 CUs
    // (one tile per CU): 224 whole tiles take one round, as long as 448 half
    // tiles take in two, and the split would add partials and a finalize pass
    // for nothing
    int splits = 1;
    if (items < 256) {
      long long best = 256;  // rounds x 256 / s (in 1/256 of a whole tile); s = 1: one round
      for (int s2 = 2; s2 <= 8 && K % (128 * s2) == 0; s2 *= 2) {
        const long long rounds = (items * s2 + 255) / 256;
        const long long cost = rounds * 256 / s2;
        if (2 * cost <= best) {
          best = cost;
          splits = s2;
        }
      }
    }
    p.splits = splits;
    p.grid_logical = items * splits;
  } else {
    p.variant = 0;
    p.nt = 8;
    p.mt = 2;
    p.chunk_rows = 128;
    p.n_blocks = ceil_div(N, 64 * p.mt);
    p.max_chunks = ceil_div(rows, p.chunk_rows);
    const long long items = (long long)p.max_chunks * p.n_blocks;
    int splits = 1;
    while (items * splits < 1024 && splits * 2 <= ksteps && splits < 16) splits *= 2;
    p.splits = splits;
    p.grid_logical = items * splits;
  }
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * rows * (pair ? 2 : 1) * N * sizeof(float) : 0;
  return p;
}

GemmPlan plan_grouped(int P, int E, int N, int K, bool pair) {
  GemmPlan p{};
  const int ksteps = K / KSTEP;
  // average rows per expert decides between the streaming and the tiled variant
  const double avg = (double)P / (double)E;
  if (avg < 2.0 && grouped_stream_fits(K)) {
    p.variant = 2;
    p.nt = 1;
    p.chunk_rows = PERSIST_ROWS;
    p.mt = 1;
    p.n_blocks = ceil_div(N, grouped_stream_rows_per_wg(pair));
    p.splits = 1;
  } else if (avg < 2.0) {
    p.variant = 1;
    p.nt = 1;
    p.chunk_rows = STREAM_GROUPED_ROWS;
    p.mt = stream_rows_per_wg(W_MXFP4, pair) / 64;
    p.n_blocks = ceil_div(N, stream_rows_per_wg(W_MXFP4, pair));
    p.splits = ceil_div(ksteps, STREAM_GROUPED_KSMAX);
  } else {
    // the prefill kernel addresses sorted rows from each chunk's first row, so
    // any P fits its 32-bit buffer offsets (gathered rows are bounded at the ABI)
    p.variant = 3;
    p.nt = PREFILL_NT;
    p.chunk_rows = 16 * PREFILL_NT;
    p.mt = prefill_pl_rows_per_wg(pair, W_MXFP4) / 64;
    p.n_blocks = ceil_div(N, prefill_pl_rows_per_wg(pair, W_MXFP4));
    p.splits = 1;
  }
  p.max_chunks = P / p.chunk_rows + (E < P ? E : P);
  p.grid_logical = (long long)p.max_chunks * p.n_blocks * p.splits;
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * P * (pair ? 2 : 1) * N * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemm(const GemmPlan &pl, int wfmt, int afmt, bool pair, const GemmArgs &a,
                       hipStream_t st) {
  const long long grid = (pl.grid_logical + 7) / 8 * 8;
  if (pl.variant == 2) return launch_grouped_stream(wfmt, afmt, pair, a, st);
  if (pl.variant == 3) return launch_prefill_gemm(wfmt, afmt, pair, a, grid, st);
  if (pl.variant == 4) {
    // activations arrive as bf16 planes (the caller splits fp32 ones)
    if (wfmt != W_BF16) return hipErrorInvalidValue;
    return launch_dense_tile(afmt == A_F32_SPLIT ? 2 : 1, pair, a, st);
  }
  if (pl.variant == 1) return launch_stream_gemm(wfmt, afmt, pair, a, grid, st);
  // the tiled variant 0 serves the mid-size dense products only (grouped
  // MXFP4 segments run on the stream, persistent or prefill kernels)
  if (wfmt == W_MXFP4) return hipErrorInvalidValue;
  return launch_af<W_BF16>(pl, afmt, pair, a, grid, st);
}

hipError_t launch_finalize(const FinalizeArgs &f, hipStream_t st) {
  const long long total = (long long)f.rows * f.N;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, f);
  return hipGetLastError();
}

hipError_t launch_plan_chunks(const int32_t *offsets, int E, int chunk_rows, int32_t *chunks,
                              int32_t *count, hipStream_t st, int min_rows, int max_rows) {
  hipLaunchKernelGGL(plan_chunks_kernel, dim3(1), dim3(1024), 0, st, offsets, E, chunk_rows, chunks,
                     count, min_rows, max_rows);
  return hipGetLastError();
}

}  // namespace moe
