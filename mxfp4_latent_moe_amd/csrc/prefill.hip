// MX-scaled tiled GEMM for prefill-sized MXFP4 expert segments (the MX8X3
// and MX6X3 operand modes); bf16 and fp32 activations run on the plane kernel
// of prefill_pl.hip, the dense bf16 products of the layer on dense.hip's
// tiles.
//
// Work item = (chunk of <= 16*NT expert-sorted token rows of one expert,
// block of 16*NW*MT weight rows).  Weight rows are the MFMA's M side, tokens
// its N side, so each wave holds only its own weight rows.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;

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

// fp4 weights x e2m3 activations (format code 2): the fp6 operand is six
// registers, 32 codes of K 32*(lane/16) .. +31 packed LSB first (checked on
// the GPU against random operands); the instruction runs at the fp4 rate.
MOE_DEV f32x4_t mfma_mx_fp4_fp6(u32x4_t w, u32x4_t blo, u32x2_t bhi, f32x4_t c, int sa, int sb) {
  const i32x4_t w4 = __builtin_bit_cast(i32x4_t, w);
  const i32x8_t a = __builtin_shufflevector(w4, w4, 0, 1, 2, 3, -1, -1, -1, -1);
  const u32x4_t h4 = __builtin_shufflevector(bhi, bhi, 0, 1, -1, -1);
  const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(blo, h4, 0, 1, 2, 3, 4, 5, -1, -1));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, sa, 0, sb);
}

// LDS bytes of one activation stage with NT token tiles: term bytes
// [term][token][slot][16] and block scales [term][token] (dwords, padded to
// whole wave loads).  A token's 128 bytes of one K step are eight 16-byte
// parts; part p sits in slot p ^ (token & 7).  fp8: part g + 4h is K 16g +
// 64h .. +15; fp6: parts 2g and 2g + 1 are the 32-byte slot of block g (24
// code bytes, then padding that is loaded but never read).  Eight lanes load
// one token's whole 128-byte line, and the eight tokens a fragment read
// serves at a time hit eight different slots, so the reads are free of bank
// conflicts.
constexpr int mx_q_bytes(int nt) { return 3 * 4 * 16 * nt * 32; }
// Scale groups: the e8m0 scales of four consecutive K steps (16 bytes of a
// row) are loaded once per group, a 16-byte load per row, into one of two
// group buffers: activation scales [term][token][16] (padded to whole 1 KB
// wave loads), then weight scales [matrix][row][16] of the work-group's rows.
constexpr int mx_gsa_bytes(int nt) { return (3 * 16 * nt * 16 + 1023) / 1024 * 1024; }
constexpr int MX_GSW_BYTES = 2 * 16 * PREFILL_MX_NW * PREFILL_MX_MT_PAIR * 16;
static_assert(MX_GSW_BYTES == 16 * PREFILL_MX_NW * PREFILL_MX_MT_SINGLE * 16, "one scale area for both shapes");
constexpr int mx_group_bytes(int nt) { return mx_gsa_bytes(nt) + MX_GSW_BYTES; }
constexpr int MX_DUMMY_BYTES = 8 * 1024;  // target of the padding loads

// 16 activation bytes at ql + QO, 16 more at qh + QO and a scale dword at
// sa + SO, issued without waiting
template <int QO, int SO>
MOE_DEV void lds_read_frag(uint32_t ql, uint32_t qh, uint32_t sa, u32x4_t &lo, u32x4_t &hi, uint32_t &sc) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:%6\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b32 %2, %5 offset:%7"
      : "=&v"(lo), "=&v"(hi), "=&v"(sc)
      : "v"(ql), "v"(qh), "v"(sa), "n"(QO), "n"(SO)
      : "memory");
}

// wait until at most N LDS reads are outstanding; the operands tie the wait
// to the registers it protects, so their users stay behind it
template <int N>
MOE_DEV void lds_wait_frag(u32x4_t &lo, u32x4_t &hi, uint32_t &sc) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(lo), "+v"(hi), "+v"(sc) : "n"(N) : "memory");
}

// a weight-scale dword at wa + WO (the four lanes of a row read the same
// dword), issued without waiting
template <int WO>
MOE_DEV void lds_read_wscale(uint32_t wa, uint32_t &w) {
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=&v"(w) : "v"(wa), "n"(WO) : "memory");
}

// fp6 fragment: the 24 code bytes of a lane's block (16 at ql + QO, 8 at qh + QO)
template <int QO, int SO>
MOE_DEV void lds_read_frag6(uint32_t ql, uint32_t qh, uint32_t sa, u32x4_t &lo, u32x2_t &hi, uint32_t &sc) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:%6\n\t"
      "ds_read_b64 %1, %4 offset:%6\n\t"
      "ds_read_b32 %2, %5 offset:%7"
      : "=&v"(lo), "=&v"(hi), "=&v"(sc)
      : "v"(ql), "v"(qh), "v"(sa), "n"(QO), "n"(SO)
      : "memory");
}
template <int N>
MOE_DEV void lds_wait_frag6(u32x4_t &lo, u32x2_t &hi, uint32_t &sc) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(lo), "+v"(hi), "+v"(sc) : "n"(N) : "memory");
}

template <bool FP6, bool PAIR, int NTA, int MT, int NW>
__device__ __forceinline__ void pfmx_item(const GemmArgs &g, uint8_t *st0, uint8_t *st1, uint8_t *st2,
                                          uint8_t *grp0, uint8_t *dummy, int expert, int row0, int nrows,
                                          int nb) {
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int CT = 16 * NTA;
  constexpr int ROWS_WG = 16 * NW * MT;
  constexpr int TERMS = 3;
  constexpr int QB = mx_q_bytes(NTA);
  constexpr int QI = QB / 1024;                   // 1 KB wave loads per stage for the terms
  constexpr int KQ = (QI + NW - 1) / NW;          // per wave, equal for all waves
  constexpr int GAI = mx_gsa_bytes(NTA) / 1024;    // 1 KB wave loads per group, activation scales
  constexpr int KGA = (GAI + NW - 1) / NW;
  constexpr int GSA = mx_gsa_bytes(PREFILL_NT);    // weight scales in a group buffer
  constexpr int GB = mx_group_bytes(PREFILL_NT);   // bytes of a group buffer
  constexpr int GWI = NMAT * ROWS_WG * 16 / 1024;  // 1 KB wave loads per group, weight scales
  constexpr int KGW = GWI / NW;
  static_assert(NMAT * ROWS_WG * 16 == MX_GSW_BYTES && GWI % NW == 0 && ROWS_WG % 64 == 0, "weight-scale loads");
  static_assert((KQ * NW - QI) * 1024 <= MX_DUMMY_BYTES / 2 && (KGA * NW - GAI) * 1024 <= MX_DUMMY_BYTES / 2,
                "dummy area");
  uint8_t *stage[3] = {st0, st1, st2};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;

  // ---- weights: a three-deep register ring, two steps ahead.  Their scales
  // go through the LDS scale groups.
  const uint32_t row_bytes = K / 2, srow_bytes = K / 32;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0) + expert * g.w_estride;
    wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
    sr[mat] = make_rsrc((mat ? g.S1 : g.S0) + expert * g.s_estride, (uint32_t)N * srow_bytes);
  }
  const int wrow_base = nb * ROWS_WG + wave * 16 * MT;
  uint32_t woff[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int n = min(wrow_base + (t % MT) * 16 + r16, N - 1);
    woff[t] = (uint32_t)n * row_bytes + kg * 16;
  }
  u32x4_t wq[3][NTILE];
  auto load_w_tile = [&](int b, int t, int s) { wq[b][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)s * 64u); };
  // weight-scale group load k of this wave: rows [64 (wave + NW k), +64) of [matrix][row]
  uint32_t wsoff[KGW];
#pragma unroll
  for (int k = 0; k < KGW; ++k) {
    const int q = 64 * (wave + NW * k) + lane;
    const int n = min(nb * ROWS_WG + q % ROWS_WG, N - 1);
    wsoff[k] = (uint32_t)n * srow_bytes;
  }
  auto load_gw = [&](uint8_t *grp, uint32_t oob, int k, int gi) {
    const int ii = wave + NW * k;  // uniform: the whole load is in one matrix
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr[(ii * 64) / ROWS_WG], (lds_void *)(grp + GSA + ii * 1024), 16,
                                             wsoff[k] | oob, (uint32_t)gi * 16u, 0, 0);
  };

  // ---- activation terms, loaded straight into LDS: wave load k of this wave
  // covers 16-byte slots [64 (wave + NW k), +64); slot q of a stage is (term,
  // token, slot); eight consecutive lanes fetch one token's 128-byte line.
  // Rows past the chunk repeat its first row (their columns are never stored).
  const uint32_t plane = (uint32_t)(g.mx_rows * K), splane = (uint32_t)(g.mx_rows * (K / 32));
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(g.mxq, 3u * plane);
  const __amdgpu_buffer_rsrc_t sr8 = make_rsrc(g.mxs, 3u * splane);
  auto arow_of = [&](int tok) -> long long {
    const int p = row0 + (tok < nrows ? tok : 0);
    return g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
  };
  uint32_t qoff[KQ];
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const int q = 64 * (wave + NW * k) + lane;
    const int term = q / (8 * CT), rem = q - term * 8 * CT;
    const int tok = rem >> 3, part = (rem & 7) ^ (tok & 7);  // 16-byte part of the token's 128-wide step
    qoff[k] = q < QB / 16 ? (uint32_t)(term * (long long)plane + arow_of(tok) * K + part * 16) : 0u;
  }
  uint32_t soffs[KGA];
#pragma unroll
  for (int k = 0; k < KGA; ++k) {
    const int q = 64 * (wave + NW * k) + lane;
    const int term = q / CT, tok = q - term * CT;
    soffs[k] = q < TERMS * CT ? (uint32_t)(term * (long long)splane + arow_of(tok) * (K / 32)) : 0u;
  }
  auto load_q = [&](int b, int k, int s) {
    const int ii = wave + NW * k;
    uint8_t *dst = ii < QI ? stage[b] + ii * 1024 : dummy + (ii - QI) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void *)dst, 16, qoff[k], (uint32_t)s * 128u, 0, 0);
  };
  auto load_ga = [&](uint8_t *grp, uint32_t oob, int k, int gi) {
    const int ii = wave + NW * k;
    uint8_t *dst = ii < GAI ? grp + ii * 1024 : dummy + MX_DUMMY_BYTES / 2 + (ii - GAI) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr8, (lds_void *)dst, 16, soffs[k] | oob, (uint32_t)gi * 16u, 0, 0);
  };
  // the memory operations that fill ring slot b with step s: KQ loads into LDS
  // and NTILE weight tiles, after NG scale-group loads.  Those fetch group
  // s / 4 into group buffer (s / 4) % 2 on the first step of a group; on the
  // other steps their offsets lie past the end of the buffers, so they read
  // nothing (out-of-range buffer loads return zero) and they write the zeros
  // to the dummy area.  The same instruction count on every step keeps the
  // unrolled steps free of branches.
  constexpr int NOPS = KQ + NTILE;
  constexpr int NG = KGA + KGW;
  auto issue_op = [&](int o, int b, int s) {
    if (o < KQ) load_q(b, o, s);
    else load_w_tile(b, o - KQ, s);
  };
  auto load_group = [&](int s) {
    const bool real = (s & 3) == 0 && s < nks;
    const int gi = min(s, nks - 1) >> 2;
    uint8_t *grp = real ? grp0 + (gi & 1) * GB : dummy;
    const uint32_t oob = real ? 0u : 0x80000000u;
#pragma unroll
    for (int k = 0; k < KGA; ++k) load_ga(grp, oob, k, gi);
#pragma unroll
    for (int k = 0; k < KGW; ++k) load_gw(real ? grp : dummy - GSA, oob, k, gi);
  };
  auto load_all = [&](int b, int s) {
    load_group(s);
    s = min(s, nks - 1);
#pragma unroll
    for (int o = 0; o < NOPS; ++o) issue_op(o, b, s);
  };

  f32x4_t acc[NTILE][NTA];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LDS reads of the activation fragments are written as inline assembly with
  // explicit lgkmcnt waits: the compiler would otherwise wait for every load
  // into LDS still in flight (it cannot tell the stages apart) before each read.
  // Fragment f = (term, token tile n); lane (token r16, group kg) reads the two
  // 16-byte parts of its token and group and its token's scale dword.
  const int plo = FP6 ? 2 * kg : kg, phi = FP6 ? 2 * kg + 1 : kg + 4;
  uint32_t qlo[3], qhi[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    qlo[b] = lds_addr(stage[b]) + (uint32_t)(r16 * 128 + ((plo ^ (r16 & 7)) << 4));
    qhi[b] = lds_addr(stage[b]) + (uint32_t)(r16 * 128 + ((phi ^ (r16 & 7)) << 4));
  }
  // scale dword of (token r16, step) and (weight row of this lane, step) in group buffer 0
  const uint32_t sbase = lds_addr(grp0) + (uint32_t)(r16 * 16);
  const uint32_t wbase = lds_addr(grp0) + (uint32_t)(GSA + (wave * 16 * MT + r16) * 16);
  // compute step s from slot b; after each fragment's products a share of the
  // loads of step s + 2 (into slot b2) goes out, so that no wave stalls on a
  // burst of memory instructions
  auto compute = [&](int b, int b2, int s) {
    const int s2 = min(s + 2, nks - 1);
    const uint32_t gsel = (uint32_t)(((s >> 2) & 1) * GB + (s & 3) * 4);
    const uint32_t slane = sbase + gsel, wlane = wbase + gsel;
    // the scales of step s + 2's group go out before this step's reads
    load_group(s + 2);
    // weight scales first: the wait for the first fragment covers them
    uint32_t wsv[NTILE];
    static_for<NTILE>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      lds_read_wscale<((t / MT) * ROWS_WG + (t % MT) * 16) * 16>(wlane, wsv[t]);
    });
    int sa[NTILE];
    constexpr int F = TERMS * NTA;
    constexpr int D = 2;
    u32x4_t lo[D + 1], hi[D + 1];
    u32x2_t hi6[D + 1];
    uint32_t sc[D + 1];
    auto issue = [&](auto fc) {
      constexpr int f = decltype(fc)::value;
      constexpr int term = f / NTA, n = f % NTA;
      constexpr int QO = (term * CT + 16 * n) * 128, SO = (term * CT + 16 * n) * 16;
      if constexpr (FP6)
        lds_read_frag6<QO, SO>(qlo[b], qhi[b], slane, lo[f % (D + 1)], hi6[f % (D + 1)], sc[f % (D + 1)]);
      else
        lds_read_frag<QO, SO>(qlo[b], qhi[b], slane, lo[f % (D + 1)], hi[f % (D + 1)], sc[f % (D + 1)]);
    };
    static_for<D>([&](auto fc) { issue(fc); });
    static_for<F>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      constexpr int n = f % NTA;
      if constexpr (f + D < F) issue(std::integral_constant<int, f + D>{});
      constexpr int behind = (f + D < F) ? D : F - 1 - f;  // fragments issued after f
      auto scales_ready = [&]() {
        if constexpr (f == 0) {
#pragma unroll
          for (int t = 0; t < NTILE; ++t) {
            asm volatile("" : "+v"(wsv[t]));  // after the first fragment's wait
            sa[t] = (int)((wsv[t] >> (8 * kg)) & 0xFFu);
          }
        }
      };
      if constexpr (FP6) {
        lds_wait_frag6<3 * behind>(lo[f % (D + 1)], hi6[f % (D + 1)], sc[f % (D + 1)]);
        scales_ready();
        const int sb = (int)((sc[f % (D + 1)] >> (8 * kg)) & 0xFFu);
#pragma unroll
        for (int t = 0; t < NTILE; ++t)
          acc[t][n] = mfma_mx_fp4_fp6(wq[b][t], lo[f % (D + 1)], hi6[f % (D + 1)], acc[t][n], sa[t], sb);
      } else {
        lds_wait_frag<3 * behind>(lo[f % (D + 1)], hi[f % (D + 1)], sc[f % (D + 1)]);
        scales_ready();
        const int sb = (int)((sc[f % (D + 1)] >> (8 * kg)) & 0xFFu);
        const i32x8_t bq = __builtin_bit_cast(
            i32x8_t, __builtin_shufflevector(lo[f % (D + 1)], hi[f % (D + 1)], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[t][n] = mfma_mx_fp4_fp8(wq[b][t], bq, acc[t][n], sa[t], sb);
      }
      constexpr int J = (NOPS + F - 1) / F;
#pragma unroll
      for (int o = f * J; o < (f + 1) * J && o < NOPS; ++o) issue_op(o, b2, s2);
    });
  };
  // step s (ring slot b = s % 3): stage s+2's loads and weights of s+2 go out
  // while s computes; then stage s+1 (requested a step earlier) must be in LDS
  // for every wave before the barrier
  auto step = [&](int b, int s) {
    compute(b, (b + 2) % 3, s);
    // a bare barrier: a workgroup fence here would also wait for stage s+2
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NOPS + NG));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);  // keep the next step's register work behind the wait
  };

  load_all(0, 0);
  load_all(1, 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(NOPS + NG));  // stage 0, scale group 0 and weights 0 are here
  __builtin_amdgcn_s_barrier();
  int s = 0;
  for (; s + 2 < nks; s += 3) {
    step(0, s);
    step(1, s + 1);
    step(2, s + 2);
  }
  if (s < nks) step(0, s);
  if (s + 1 < nks) step(1, s + 1);
  // drain the loads past the last step before the LDS is reused
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

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
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <bool FP6, bool PAIR, int NT, int MT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_mx_kernel(GemmArgs g) {
  // three activation stages (separate objects, so waits on one stage's loads
  // do not cover the others) and the padding loads' target
  __shared__ __attribute__((aligned(1024))) uint8_t st0[mx_q_bytes(NT)];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[mx_q_bytes(NT)];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[mx_q_bytes(NT)];
  __shared__ __attribute__((aligned(1024))) uint8_t grp[2 * mx_group_bytes(NT)];
  __shared__ __attribute__((aligned(1024))) uint8_t dummy[MX_DUMMY_BYTES];
  static_assert(NT == PREFILL_NT, "group buffer layout assumes the compiled tile count");
  static_assert(NT >= 1 && NT <= 6, "the item dispatch covers 1..6 active token tiles");
  const int total = min(*g.chunk_count * g.n_blocks, g.grid_logical);
  const int logical = xcd_logical(total);
  if (logical < 0) return;
  const int chunk = logical / g.n_blocks;
  const int nb = logical - chunk * g.n_blocks;
  const int4 c = reinterpret_cast<const int4 *>(g.chunks)[chunk];
  const int nta = min((c.z + 15) >> 4, NT);
  if (nta == NT) {
    pfmx_item<FP6, PAIR, NT, MT, NW>(g, st0, st1, st2, grp, dummy, c.x, c.y, c.z, nb);
    return;
  }
  switch (nta) {
    case 1: if constexpr (NT > 1) pfmx_item<FP6, PAIR, 1, MT, NW>(g, st0, st1, st2, grp, dummy, c.x, c.y, c.z, nb); break;
    case 2: if constexpr (NT > 2) pfmx_item<FP6, PAIR, 2, MT, NW>(g, st0, st1, st2, grp, dummy, c.x, c.y, c.z, nb); break;
    case 3: if constexpr (NT > 3) pfmx_item<FP6, PAIR, 3, MT, NW>(g, st0, st1, st2, grp, dummy, c.x, c.y, c.z, nb); break;
    case 4: if constexpr (NT > 4) pfmx_item<FP6, PAIR, 4, MT, NW>(g, st0, st1, st2, grp, dummy, c.x, c.y, c.z, nb); break;
    default: if constexpr (NT > 5) pfmx_item<FP6, PAIR, 5, MT, NW>(g, st0, st1, st2, grp, dummy, c.x, c.y, c.z, nb); break;
  }
}

}  // namespace

int prefill_mx_rows_per_wg(bool pair) { return 16 * PREFILL_MX_NW * (pair ? PREFILL_MX_MT_PAIR : PREFILL_MX_MT_SINGLE); }

hipError_t launch_prefill_gemm(int wfmt, int afmt, bool pair, const GemmArgs &a, long long grid,
                               hipStream_t st) {
  if (afmt == A_MX8X3 || afmt == A_MX6X3) {
    if (wfmt != W_MXFP4) return hipErrorInvalidValue;
    // one wave per SIMD: the MX operands need the larger register budget
    const dim3 gr((unsigned)grid), blk(64 * PREFILL_MX_NW);
    if (afmt == A_MX6X3) {
      if (pair) hipLaunchKernelGGL((prefill_mx_kernel<true, true, PREFILL_NT, PREFILL_MX_MT_PAIR, PREFILL_MX_NW>), gr, blk, 0, st, a);
      else hipLaunchKernelGGL((prefill_mx_kernel<true, false, PREFILL_NT, PREFILL_MX_MT_SINGLE, PREFILL_MX_NW>), gr, blk, 0, st, a);
    } else {
      if (pair) hipLaunchKernelGGL((prefill_mx_kernel<false, true, PREFILL_NT, PREFILL_MX_MT_PAIR, PREFILL_MX_NW>), gr, blk, 0, st, a);
      else hipLaunchKernelGGL((prefill_mx_kernel<false, false, PREFILL_NT, PREFILL_MX_MT_SINGLE, PREFILL_MX_NW>), gr, blk, 0, st, a);
    }
    return hipGetLastError();
  }
  // bf16 or fp32 activations run on the plane kernel (launch_prefill_planes)
  return hipErrorInvalidValue;
}

}  // namespace moe
