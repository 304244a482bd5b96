// Tiled MXFP4 grouped GEMM for prefill-sized expert segments.
//
// Work item = (chunk of <= 16*NT expert-sorted token rows of one expert,
// block of 64*MT weight rows).  Weight rows are the MFMA's M side, tokens its
// N side (v_mfma_f32_16x16x32_bf16), so each wave dequantises only its own
// weight rows and every dequantised fragment feeds NT (x2 for hi + lo) MFMAs.
//
// Per 128-wide K step:
//  * weights: one 16-byte buffer load per lane per 16-row tile (32 e2m1 codes
//    = one scale group of one row), issued a full step before use, converted
//    in registers by the scaled fp4 -> bf16 instruction;
//  * activations: the chunk's rows are loaded one step ahead into registers,
//    split into bf16 hi + lo (or rounded), and written to a double-buffered
//    LDS tile [octet][token ^ octet][8] -- the XOR swizzle keeps both the
//    octet-wise writes and the token-wise fragment reads free of bank
//    conflicts;
//  * one barrier per step.
// Token tiles past the chunk's last row are skipped (wave-uniform branch).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;

template <int AF, bool PAIR, int NT, int MT>
__global__ __launch_bounds__(256, 1) void prefill_kernel(GemmArgs g) {
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;  // LDS planes (hi, lo)
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;                  // 16-row weight tiles per wave
  constexpr int CT = 16 * NT;                       // tokens per chunk
  constexpr int ROWS_WG = 64 * MT;                  // weight rows per matrix per work-group
  constexpr int PLANE = CT * KSTEP;                 // bf16 elements per plane per stage
  constexpr int AW = (AF == A_BF16) ? 1 : 2;        // 16-byte loads per staged octet
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][NPL][PLANE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;

  // ---- work item (XCD-aware over the items that exist on the device)
  const int total = min(*g.chunk_count * g.n_blocks, g.grid_logical);
  const int logical = xcd_logical(total);
  if (logical < 0) return;
  const int chunk = logical / g.n_blocks;
  const int nb = logical - chunk * g.n_blocks;
  const int4 cinfo = reinterpret_cast<const int4 *>(g.chunks)[chunk];
  const int expert = cinfo.x, row0 = cinfo.y, nrows = cinfo.z;
  const int nta = (nrows + 15) >> 4;  // active token tiles
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;

  // ---- weight rows of this wave: buffer resources per matrix, offsets per tile
  const uint32_t row_bytes = K / 2, srow_bytes = K / 32;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0) + expert * g.w_estride;
    const uint8_t *S = (mat ? g.S1 : g.S0) + expert * g.s_estride;
    wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
    sr[mat] = make_rsrc(S, (uint32_t)N * srow_bytes);
  }
  const int wrow_base = nb * ROWS_WG + wave * 16 * MT;
  uint32_t woff[NTILE], soff[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int n = min(wrow_base + (t % MT) * 16 + r16, N - 1);
    woff[t] = (uint32_t)n * row_bytes + kg * 16;
    soff[t] = (uint32_t)n * srow_bytes;
  }

  // ---- activation rows this thread stages: token (tid >> 4) + 16 i, octet tid & 15
  const int a_oct = tid & 15;
  const int esz = (AF == A_BF16) ? 2 : 4;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(g.A, 0x7FFFFFF0u);
  uint32_t aoff[NT];
  bool alive[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int r = (tid >> 4) + 16 * i;
    alive[i] = r < nrows;
    const int p = row0 + min(r, nrows - 1);
    const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
    aoff[i] = (uint32_t)((arow * g.lda + a_oct * 8) * esz);
  }

  u32x4_t wq[2][NTILE];
  uint32_t wsc[2][NTILE];
  u32x4_t aq[NT][AW];

  auto load_w = [&](int b, int s) {
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      wq[b][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)s * 64u);
      wsc[b][t] = buf_load4(sr[t / MT], soff[t], (uint32_t)s * 4u);
    }
  };
  auto load_a = [&](int s) {
    const uint32_t so = (uint32_t)s * KSTEP * esz;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int h = 0; h < AW; ++h) aq[i][h] = buf_load16(ar, aoff[i] + 16 * h, so);
    }
  };
  // swizzled LDS slot of (octet, token): octet-major, token XOR octet
  auto slot = [](int oct, int tok) { return (oct * CT + (tok ^ oct)) * 8; };
  auto store_a = [&](int b) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int r = (tid >> 4) + 16 * i;
      const int off = slot(a_oct, r);
      if constexpr (AF == A_BF16) {
        const u32x4_t v = alive[i] ? aq[i][0] : u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t *>(&lds[b][0][off]) = v;
      } else {
        bf16x8_t hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = alive[i] ? __uint_as_float(aq[i][e >> 2][e & 3]) : 0.f;
          if constexpr (AF == A_F32_SPLIT) {
            __bf16 h, l;
            split_bf16(f, h, l);
            hi[e] = h;
            lo[e] = l;
          } else {
            hi[e] = to_bf16(f);
          }
        }
        *reinterpret_cast<bf16x8_t *>(&lds[b][0][off]) = hi;
        if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(&lds[b][NPL - 1][off]) = lo;
      }
    }
  };

  f32x4_t acc[NTILE][NT];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int b) {
    float scl[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) scl[t] = e8m0_to_float((wsc[b][t] >> (8 * kg)) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int oct = 4 * kg + j;
      bf16x8_t wa[NTILE];
#pragma unroll
      for (int t = 0; t < NTILE; ++t) wa[t] = fp4x8_to_bf16(wq[b][t][j], scl[t]);
#pragma unroll
      for (int p = 0; p < NPL; ++p) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (n < nta) {
            const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(&lds[b][p][slot(oct, 16 * n + r16)]);
#pragma unroll
            for (int t = 0; t < NTILE; ++t) acc[t][n] = mfma_16x16x32(wa[t], bv, acc[t][n]);
          }
        }
      }
    }
  };

  // ---- pipeline: step s computes from LDS stage s&1 and weight buffer s&1;
  // activations of step s+1 and weights of step s+2 are in flight meanwhile.
  load_w(0, 0);
  load_a(0);
  if (nks > 1) load_w(1, 1);
  store_a(0);
  __syncthreads();
  for (int s = 0; s < nks; s += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ss = s + h;
      if (ss < nks) {
        if (ss + 1 < nks) load_a(ss + 1);
        compute(h);
        if (ss + 2 < nks) load_w(h, ss + 2);
        if (ss + 1 < nks) store_a(h ^ 1);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: SiTU-GLU of the gate/up pair (or the plain product), row scale, store
  const int col_base = wrow_base + 4 * kg;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int tok = 16 * n + r16;
    if (n < nta && tok < nrows) {
      const long long orow = row0 + tok;
      float rs = 1.f;
      if (g.rscale != nullptr) rs = g.rscale[g.rscale_map ? g.rscale_map[orow] : orow];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int col0 = col_base + m * 16;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (PAIR) v[r] = situ_glu(acc[m][n][r], acc[m + MT][n][r], g.beta, g.beta_lin) * rs;
          else v[r] = acc[m][n][r] * rs;
        }
        float *cp = g.C + orow * g.ldc + col0;
        if (col0 + 3 < N) {
          *reinterpret_cast<f32x4_t *>(cp) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col0 + r < N) cp[r] = v[r];
        }
      }
    }
  }
}

template <int AF, bool PAIR>
hipError_t launch_pf(const GemmArgs &a, long long grid, hipStream_t st) {
  constexpr int MT = PAIR ? PREFILL_MT_PAIR : PREFILL_MT_SINGLE;
  hipLaunchKernelGGL((prefill_kernel<AF, PAIR, PREFILL_NT, MT>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_wg(bool pair) { return 64 * (pair ? PREFILL_MT_PAIR : PREFILL_MT_SINGLE); }

hipError_t launch_prefill_gemm(int afmt, bool pair, const GemmArgs &a, long long grid, hipStream_t st) {
  switch (afmt) {
    case A_BF16: return pair ? launch_pf<A_BF16, true>(a, grid, st) : launch_pf<A_BF16, false>(a, grid, st);
    case A_F32_SPLIT:
      return pair ? launch_pf<A_F32_SPLIT, true>(a, grid, st) : launch_pf<A_F32_SPLIT, false>(a, grid, st);
    default:
      return pair ? launch_pf<A_F32_ROUND, true>(a, grid, st) : launch_pf<A_F32_ROUND, false>(a, grid, st);
  }
}

}  // namespace moe
