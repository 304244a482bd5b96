// Tiled GEMM for prefill-sized work: MXFP4 expert segments (grouped) and the
// bf16 dense products of the layer.
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
// The item body is specialised on the number of active 16-token tiles, so the
// K loop is straight-line code and token tiles past the chunk's last row cost
// nothing.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;

// One work item with NTA active 16-token tiles (the K loop has no branches).
template <int WF, int AF, bool PAIR, int NTA, int MT, int NW>
__device__ __forceinline__ void pf_item(const GemmArgs &g, __bf16 *lds_base, int expert, int row0,
                                        int nrows, int nb) {
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;  // LDS planes (hi, lo)
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;                  // 16-row weight tiles per wave
  constexpr int CT = 16 * NTA;                      // staged tokens
  constexpr int ROWS_WG = 16 * NW * MT;             // weight rows per matrix per work-group
  constexpr int PLANE = CT * KSTEP;                 // bf16 elements per plane per stage
  constexpr int AW = (AF == A_BF16) ? 1 : 2;        // 16-byte loads per staged octet
  constexpr int RPP = 4 * NW;                       // token rows staged per pass (16 threads a row)
  constexpr int NPASS = (CT + RPP - 1) / RPP;       // staging passes per K step
  auto lds = [&](int b, int p) { return lds_base + (b * NPL + p) * PLANE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;

  // ---- weight rows of this wave: buffer resources per matrix, offsets per tile.
  // MXFP4: lane group kg's 16 bytes of a 128-wide K step are its 32 codes (one
  // scale group); bf16: its 64 bytes (32 values), one 16-byte load per sub-step.
  constexpr bool FP4 = WF == W_MXFP4;
  const uint32_t row_bytes = FP4 ? K / 2 : K * 2, srow_bytes = FP4 ? K / 32 : 0;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0) + expert * g.w_estride;
    wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
    if constexpr (FP4) sr[mat] = make_rsrc((mat ? g.S1 : g.S0) + expert * g.s_estride, (uint32_t)N * srow_bytes);
  }
  const int wrow_base = nb * ROWS_WG + wave * 16 * MT;
  uint32_t woff[NTILE], soff[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int n = min(wrow_base + (t % MT) * 16 + r16, N - 1);
    woff[t] = (uint32_t)n * row_bytes + kg * (FP4 ? 16 : 64);
    soff[t] = (uint32_t)n * srow_bytes;
  }

  // ---- activation rows this thread stages: token (tid >> 4) + RPP i, octet tid & 15
  const int a_oct = tid & 15;
  const int esz = (AF == A_BF16) ? 2 : 4;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(g.A, 0x7FFFFFF0u);
  uint32_t aoff[NPASS];
  bool alive[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    const int r = (tid >> 4) + RPP * i;
    alive[i] = r < nrows;
    const int p = row0 + min(r, nrows - 1);
    const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
    aoff[i] = (uint32_t)((arow * g.lda + a_oct * 8) * esz);
  }

  u32x4_t wq[2][NTILE];    // MXFP4: codes of one K step per stage
  uint32_t wsc[2][NTILE];
  u32x4_t wb[4][NTILE];    // bf16: ring of sub-steps, two ahead of use
  u32x4_t aq[NPASS][AW];

  // loads past the last K step re-read the last one (never past the rows)
  auto load_w = [&](int b, int s) {
    if constexpr (!FP4) return;
    s = min(s, nks - 1);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      wq[b][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)s * 64u);
      wsc[b][t] = buf_load4(sr[t / MT], soff[t], (uint32_t)s * 4u);
    }
  };
  // bf16 sub-step j of step s into ring slot j (sub-steps past the last step re-read it)
  auto load_wj = [&](int s, int j) {
    if constexpr (FP4) return;
    s = min(s, nks - 1);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) wb[j][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)s * 256u + 16u * j);
  };
  auto load_a = [&](int s) {
    s = min(s, nks - 1);
    const uint32_t so = (uint32_t)s * KSTEP * esz;
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
#pragma unroll
      for (int h = 0; h < AW; ++h) aq[i][h] = buf_load16(ar, aoff[i] + 16 * h, so);
    }
  };
  // swizzled LDS slot of (octet, token): octet-major, token XOR octet
  auto slot = [](int oct, int tok) { return (oct * CT + (tok ^ oct)) * 8; };
  auto store_a = [&](int b) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int r = (tid >> 4) + RPP * i;
      if (CT % RPP != 0 && r >= CT) continue;
      const int off = slot(a_oct, r);
      if constexpr (AF == A_BF16) {
        const u32x4_t v = alive[i] ? aq[i][0] : u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t *>(lds(b, 0) + off) = v;
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
        *reinterpret_cast<bf16x8_t *>(lds(b, 0) + off) = hi;
        if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(lds(b, NPL - 1) + off) = lo;
      }
    }
  };

  f32x4_t acc[NTILE][NTA];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragments f = (sub-step j, plane p, token tile n) in order; each B fragment
  // is read from LDS two fragments ahead of its MFMAs, and the weights of
  // sub-step j+1 are converted while sub-step j's MFMAs run.
  auto compute = [&](int b, int s) {
    float scl[NTILE];
    if constexpr (FP4) {
#pragma unroll
      for (int t = 0; t < NTILE; ++t) scl[t] = e8m0_to_float((wsc[b][t] >> (8 * kg)) & 0xFFu);
    }
    constexpr int FJ = NPL * NTA;  // fragments per sub-step
    constexpr int F = 4 * FJ;      // fragments per K step
    constexpr int D = 2;           // read-ahead distance
    auto rd = [&](int f) {
      const int j = f / FJ, p = (f / NTA) % NPL, n = f % NTA;
      return *reinterpret_cast<const bf16x8_t *>(lds(b, p) + slot(4 * kg + j, 16 * n + r16));
    };
    auto wfrag = [&](int j, int t) {
      if constexpr (FP4) return fp4x8_to_bf16(wq[b][t][j], scl[t]);
      else return __builtin_bit_cast(bf16x8_t, wb[j][t]);
    };
    bf16x8_t bq[D + 1];
#pragma unroll
    for (int f = 0; f < D; ++f) bq[f] = rd(f);
    bf16x8_t wa[2][NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) wa[0][t] = wfrag(0, t);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int j = f / FJ, n = f % NTA;
      if (f + D < F) bq[(f + D) % (D + 1)] = rd(f + D);
      if (f % FJ == 0) {
        if (j + 1 < 4) {
#pragma unroll
          for (int t = 0; t < NTILE; ++t) wa[(j + 1) & 1][t] = wfrag(j + 1, t);
        }
        // bf16: sub-step j+2 (of this step or the next) into its ring slot,
        // whose previous sub-step was converted before sub-step j began
        load_wj(j + 2 < 4 ? s : s + 1, (j + 2) & 3);
      }
#pragma unroll
      for (int t = 0; t < NTILE; ++t) acc[t][n] = mfma_16x16x32(wa[j & 1][t], bq[f % (D + 1)], acc[t][n]);
    }
    // let the scheduler interleave the LDS reads with the MFMAs of this region
    __builtin_amdgcn_iglp_opt(0);
  };
  // one K step: activations of s+1 and weights of s+2 are requested while s computes
  auto step = [&](int h, int s) {
    load_a(s + 1);
    compute(h, s);
    load_w(h, s + 2);
    store_a(h ^ 1);
    __syncthreads();
  };

  load_w(0, 0);
  load_wj(0, 0);
  load_wj(0, 1);
  load_a(0);
  load_w(1, 1);
  store_a(0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < nks; s += 2) {
    step(0, s);
    step(1, s + 1);
  }
  if (s < nks) step(0, s);

  // ---- epilogue: SiTU-GLU of the gate/up pair (or the plain product), row scale, store
  const int col_base = wrow_base + 4 * kg;
#pragma unroll
  for (int n = 0; n < NTA; ++n) {
    const int tok = 16 * n + r16;
    if (tok < nrows) {
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
          f32x4_t o = f32x4_t{v[0], v[1], v[2], v[3]};
          if (g.accumulate) o += *reinterpret_cast<const f32x4_t *>(cp);
          *reinterpret_cast<f32x4_t *>(cp) = o;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col0 + r < N) cp[r] = g.accumulate ? cp[r] + v[r] : v[r];
        }
        // one output group at a time: interleaving all of them costs registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <int WF, int AF, bool PAIR, int NT, int MT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_kernel(GemmArgs g) {
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * NPL * 16 * NT * KSTEP];
  static_assert(NT >= 1 && NT <= 6, "the item dispatch covers 1..6 active token tiles");

  // ---- work item (XCD-aware over the items that exist on the device).
  // Expert chunks come from the chunk list, chunk-major (the weight blocks of
  // one chunk share its activations); dense rows are cut into chunks of 16*NT
  // here, block-major (the chunks of one weight block share its weights).
  int expert, row0, nrows, nb;
  if (g.chunks != nullptr) {
    const int total = min(*g.chunk_count * g.n_blocks, g.grid_logical);
    const int logical = xcd_logical(total);
    if (logical < 0) return;
    const int chunk = logical / g.n_blocks;
    nb = logical - chunk * g.n_blocks;
    const int4 c = reinterpret_cast<const int4 *>(g.chunks)[chunk];
    expert = c.x;
    row0 = c.y;
    nrows = c.z;
  } else {
    const int nch = (g.dense_rows + 16 * NT - 1) / (16 * NT);
    const int logical = xcd_logical(min(nch * g.n_blocks, g.grid_logical));
    if (logical < 0) return;
    nb = logical / nch;
    const int chunk = logical - nb * nch;
    expert = 0;
    row0 = chunk * 16 * NT;
    nrows = min(16 * NT, g.dense_rows - row0);
  }
  const int nta = min((nrows + 15) >> 4, NT);  // active 16-token tiles
  if (nta == NT) {
    pf_item<WF, AF, PAIR, NT, MT, NW>(g, lds, expert, row0, nrows, nb);
    return;
  }
  switch (nta) {
    case 1: if constexpr (NT > 1) pf_item<WF, AF, PAIR, 1, MT, NW>(g, lds, expert, row0, nrows, nb); break;
    case 2: if constexpr (NT > 2) pf_item<WF, AF, PAIR, 2, MT, NW>(g, lds, expert, row0, nrows, nb); break;
    case 3: if constexpr (NT > 3) pf_item<WF, AF, PAIR, 3, MT, NW>(g, lds, expert, row0, nrows, nb); break;
    case 4: if constexpr (NT > 4) pf_item<WF, AF, PAIR, 4, MT, NW>(g, lds, expert, row0, nrows, nb); break;
    default: if constexpr (NT > 5) pf_item<WF, AF, PAIR, 5, MT, NW>(g, lds, expert, row0, nrows, nb); break;
  }
}


// ---------------------------------------------------------------------------
// MX-scaled variant for MXFP4 weights and activations given as three e4m3
// terms with e8m0 block scales.  v_mfma_scale_f32_16x16x128_f8f6f4 takes
// each lane's raw 16 weight bytes (32 e2m1 codes = its row's K block
// 32*(lane/16) .. +31 of the 128-wide step) with that block's e8m0 scale, and
// 32 activation bytes per lane: token lane%16, K 16*(lane/16) .. +15 and
// 64 + 16*(lane/16) .. +15, with the scale of block lane/16 of that token.
// One MFMA per weight tile, token tile and term covers the whole K step.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// The fp4 operand occupies four registers; the upper half of the builtin's
// eight-register argument is left undefined so no registers are spent on it.
MOE_DEV f32x4_t mfma_mx_fp4_fp8(u32x4_t w, i32x8_t b, f32x4_t c, int sa, int sb) {
  const i32x4_t w4 = __builtin_bit_cast(i32x4_t, w);
  const i32x8_t a = __builtin_shufflevector(w4, w4, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}

template <bool PAIR, int NTA, int MT, int NW>
__device__ __forceinline__ void pfmx_item(const GemmArgs &g, uint8_t *lds_base, int expert, int row0, int nrows,
                                          int nb) {
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int CT = 16 * NTA;
  constexpr int ROWS_WG = 16 * NW * MT;
  constexpr int NTHR = 64 * NW;
  constexpr int TERMS = 3;
  constexpr int QBYTES = TERMS * 8 * CT * 16;  // per stage: [term][K group][token][32]
  constexpr int SBYTES = TERMS * CT * 4;       // per stage: [term][token] dword of 4 block scales
  auto qlds = [&](int b) { return lds_base + b * (QBYTES + SBYTES); };
  auto slds = [&](int b) { return reinterpret_cast<uint32_t *>(lds_base + b * (QBYTES + SBYTES) + QBYTES); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;

  // ---- weights: as in the bf16-dequantising path
  const uint32_t row_bytes = K / 2, srow_bytes = K / 32;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0) + expert * g.w_estride;
    wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
    sr[mat] = make_rsrc((mat ? g.S1 : g.S0) + expert * g.s_estride, (uint32_t)N * srow_bytes);
  }
  const int wrow_base = nb * ROWS_WG + wave * 16 * MT;
  uint32_t woff[NTILE], soff[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int n = min(wrow_base + (t % MT) * 16 + r16, N - 1);
    woff[t] = (uint32_t)n * row_bytes + kg * 16;
    soff[t] = (uint32_t)n * srow_bytes;
  }
  u32x4_t wq[2][NTILE];
  uint32_t wsc[2][NTILE];
  auto load_w = [&](int b, int s) {
    s = min(s, nks - 1);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      wq[b][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)s * 64u);
      wsc[b][t] = buf_load4(sr[t / MT], soff[t], (uint32_t)s * 4u);
    }
  };

  // ---- activation terms: each thread stages 16-byte chunk (tid & 7) of tokens
  // (tid >> 3) + TPP*j of every term; rows past the chunk read past the buffer
  // (zeros), stores past the staged tokens go to a per-thread trash slot
  constexpr int TPP = NTHR / 8;                 // tokens per pass
  constexpr int NP = (CT + TPP - 1) / TPP;      // passes per term
  const uint32_t plane = (uint32_t)(g.mx_rows * K), splane = (uint32_t)(g.mx_rows * (K / 32));
  __amdgpu_buffer_rsrc_t qr[TERMS], sr8[TERMS];
#pragma unroll
  for (int term = 0; term < TERMS; ++term) {
    qr[term] = make_rsrc(g.mxq + (size_t)term * plane, plane);
    sr8[term] = make_rsrc(g.mxs + (size_t)term * splane, splane);
  }
  const int cidx = tid & 7;
  uint32_t aoff[NP];
  int aslot[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int tok = (tid >> 3) + TPP * j;
    aoff[j] = 0xFFFFFF00u;
    if (tok < nrows && tok < CT) {
      const int p = row0 + tok;
      const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
      aoff[j] = (uint32_t)(arow * K + cidx * 16);
    }
    aslot[j] = tok < CT ? ((cidx & 3) * CT + (tok ^ (cidx & 3))) * 32 + (cidx >> 2) * 16 : QBYTES + SBYTES + tid * 16;
  }
  // block scales: thread (term, token) for tid < 3 * CT loads the token's 4 scale bytes of the step
  const int sterm = tid / CT, stok = tid - (tid / CT) * CT;
  uint32_t soff8 = 0xFFFFFF00u;
  if (tid < TERMS * CT && stok < nrows) {
    const int p = row0 + stok;
    const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
    soff8 = (uint32_t)(arow * (K / 32));
  }
  u32x4_t aq[TERMS][NP];
  uint32_t asc = 0;
  auto load_a = [&](int s) {
    s = min(s, nks - 1);
#pragma unroll
    for (int term = 0; term < TERMS; ++term)
#pragma unroll
      for (int j = 0; j < NP; ++j) aq[term][j] = buf_load16(qr[term], aoff[j], (uint32_t)s * 128u);
    if (tid < TERMS * CT) {
      __amdgpu_buffer_rsrc_t r = sterm == 0 ? sr8[0] : (sterm == 1 ? sr8[1] : sr8[2]);
      asc = buf_load4(r, soff8, (uint32_t)s * 4u);
    }
  };
  auto store_a = [&](int b) {
#pragma unroll
    for (int term = 0; term < TERMS; ++term)
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        // trash slots lie past both stages; a real slot is offset by its stage and term
        const int off = aslot[j] < QBYTES + SBYTES ? b * (QBYTES + SBYTES) + term * 8 * CT * 16 + aslot[j]
                                                   : 2 * (QBYTES + SBYTES) + tid * 16;
        *reinterpret_cast<u32x4_t *>(lds_base + off) = aq[term][j];
      }
    if (tid < TERMS * CT) slds(b)[tid] = stok < nrows ? asc : 0x7F7F7F7Fu;  // [term][token]
  };

  f32x4_t acc[NTILE][NTA];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int b) {
    int sa[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) sa[t] = (int)((wsc[b][t] >> (8 * kg)) & 0xFFu);
    constexpr int F = TERMS * NTA;  // fragments (term, token tile) per step
    constexpr int D = 2;
    // lane (token r16 of tile n, group kg): 32 contiguous bytes = K 16kg..+15 and 64+16kg..+15
    auto rd = [&](int f, int &sb) {
      const int term = f / NTA, n = f % NTA;
      const int tok = 16 * n + r16;
      sb = (int)((slds(b)[term * CT + tok] >> (8 * kg)) & 0xFFu);
      return *reinterpret_cast<const i32x8_t *>(qlds(b) + ((term * 4 + kg) * CT + (tok ^ kg)) * 32);
    };
    i32x8_t bq[D + 1];
    int sbq[D + 1];
#pragma unroll
    for (int f = 0; f < D; ++f) bq[f] = rd(f, sbq[f]);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int n = f % NTA;
      if (f + D < F) bq[(f + D) % (D + 1)] = rd(f + D, sbq[(f + D) % (D + 1)]);
#pragma unroll
      for (int t = 0; t < NTILE; ++t)
        acc[t][n] = mfma_mx_fp4_fp8(wq[b][t], bq[f % (D + 1)], acc[t][n], sa[t], sbq[f % (D + 1)]);
      // keep the read-ahead distance as written: no LDS read moves across fragments
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](int h, int s) {
    load_a(s + 1);
    compute(h);
    load_w(h, s + 2);
    store_a(h ^ 1);
    __syncthreads();
  };

  load_w(0, 0);
  load_a(0);
  load_w(1, 1);
  store_a(0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < nks; s += 2) {
    step(0, s);
    step(1, s + 1);
  }
  if (s < nks) step(0, s);

  const int col_base = wrow_base + 4 * kg;
#pragma unroll
  for (int n = 0; n < NTA; ++n) {
    const int tok = 16 * n + r16;
    if (tok < nrows) {
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
          f32x4_t o = f32x4_t{v[0], v[1], v[2], v[3]};
          if (g.accumulate) o += *reinterpret_cast<const f32x4_t *>(cp);
          *reinterpret_cast<f32x4_t *>(cp) = o;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col0 + r < N) cp[r] = g.accumulate ? cp[r] + v[r] : v[r];
        }
        // one output group at a time: interleaving all of them costs registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <bool PAIR, int NT, int MT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_mx_kernel(GemmArgs g) {
  // two stages of [term][chunk][token][16] bytes + [term][token] scale dwords, then a trash slot per thread
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (3 * 8 * 16 * NT * 16 + 3 * 16 * NT * 4) + 64 * NW * 16];
  static_assert(NT >= 1 && NT <= 6, "the item dispatch covers 1..6 active token tiles");
  const int total = min(*g.chunk_count * g.n_blocks, g.grid_logical);
  const int logical = xcd_logical(total);
  if (logical < 0) return;
  const int chunk = logical / g.n_blocks;
  const int nb = logical - chunk * g.n_blocks;
  const int4 c = reinterpret_cast<const int4 *>(g.chunks)[chunk];
  const int nta = min((c.z + 15) >> 4, NT);
  if (nta == NT) {
    pfmx_item<PAIR, NT, MT, NW>(g, lds, c.x, c.y, c.z, nb);
    return;
  }
  switch (nta) {
    case 1: if constexpr (NT > 1) pfmx_item<PAIR, 1, MT, NW>(g, lds, c.x, c.y, c.z, nb); break;
    case 2: if constexpr (NT > 2) pfmx_item<PAIR, 2, MT, NW>(g, lds, c.x, c.y, c.z, nb); break;
    case 3: if constexpr (NT > 3) pfmx_item<PAIR, 3, MT, NW>(g, lds, c.x, c.y, c.z, nb); break;
    case 4: if constexpr (NT > 4) pfmx_item<PAIR, 4, MT, NW>(g, lds, c.x, c.y, c.z, nb); break;
    default: if constexpr (NT > 5) pfmx_item<PAIR, 5, MT, NW>(g, lds, c.x, c.y, c.z, nb); break;
  }
}

template <int WF, int AF, bool PAIR>
hipError_t launch_pf(const GemmArgs &a, long long grid, hipStream_t st) {
  constexpr int MT = PAIR ? PREFILL_MT_PAIR : PREFILL_MT_SINGLE;
  hipLaunchKernelGGL((prefill_kernel<WF, AF, PAIR, PREFILL_NT, MT, PREFILL_NW>), dim3((unsigned)grid),
                     dim3(64 * PREFILL_NW), 0, st, a);
  return hipGetLastError();
}

template <int WF>
hipError_t launch_wf(int afmt, bool pair, const GemmArgs &a, long long grid, hipStream_t st) {
  switch (afmt) {
    case A_BF16: return pair ? launch_pf<WF, A_BF16, true>(a, grid, st) : launch_pf<WF, A_BF16, false>(a, grid, st);
    case A_F32_SPLIT:
      return pair ? launch_pf<WF, A_F32_SPLIT, true>(a, grid, st) : launch_pf<WF, A_F32_SPLIT, false>(a, grid, st);
    default:
      return pair ? launch_pf<WF, A_F32_ROUND, true>(a, grid, st) : launch_pf<WF, A_F32_ROUND, false>(a, grid, st);
  }
}

}  // namespace

int prefill_rows_per_wg(bool pair) { return 16 * PREFILL_NW * (pair ? PREFILL_MT_PAIR : PREFILL_MT_SINGLE); }

hipError_t launch_prefill_gemm(int wfmt, int afmt, bool pair, const GemmArgs &a, long long grid,
                               hipStream_t st) {
  if (afmt == A_MX8X3) {
    if (wfmt != W_MXFP4) return hipErrorInvalidValue;
    if (pair)
      hipLaunchKernelGGL((prefill_mx_kernel<true, PREFILL_NT, PREFILL_MT_PAIR, PREFILL_NW>), dim3((unsigned)grid),
                         dim3(64 * PREFILL_NW), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_mx_kernel<false, PREFILL_NT, PREFILL_MT_SINGLE, PREFILL_NW>), dim3((unsigned)grid),
                         dim3(64 * PREFILL_NW), 0, st, a);
    return hipGetLastError();
  }
  return wfmt == W_MXFP4 ? launch_wf<W_MXFP4>(afmt, pair, a, grid, st) : launch_wf<W_BF16>(afmt, pair, a, grid, st);
}

}  // namespace moe
