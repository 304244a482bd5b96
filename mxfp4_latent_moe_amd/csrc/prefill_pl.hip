// Tiled prefill GEMM for MXFP4 expert segments over activations given as bf16
// planes: row r of the activations is [NPL][K] bf16, hi = bf16(a) then
// lo = bf16(a - hi) (NPL = 2), or the rounded row alone (NPL = 1).
//
// kimi-k3-mlx README, Architecture table and the MXFP4 format of the
// checkpoint (weight_packed e2m1 nibbles, weight_scale e8m0 per 32): each
// weight code is dequantised to bf16 by the scaled fp4 convert and fed to the
// bf16 MFMA with fp32 accumulation; a = hi + lo makes two products into the
// same accumulator.
//
// Work item = (chunk of <= 16 NT expert-sorted rows of one expert, block of
// 16 NW MT weight rows per matrix), as for the fp32-staging kernel.  Here the
// activations need no register work on their way to LDS: each K step's planes
// are loaded straight into an LDS ring (three stages, two for items of one or
// two token tiles).  Eight waves, two per SIMD, each hold 4 weight tiles of
// 16 rows (gate and up of a SiTU pair: 2 + 2), so the accumulators and
// operands fit the 256 registers of a wave without spilling, and each SIMD
// interleaves two instruction streams.  The weights go to registers through a
// ring of 3 steps, or 4 for items of one or two token tiles, whose steps are
// too short to cover a memory trip.
//
// Affine 2-bit weights (w = scale * q + bias per 64-element group; the
// second bank of kimi-k3-mlx README, Tiers section) run the same loop with
// the codes entering the MFMA as exact integers q: each instruction stays
// inside one 64-element group, the two instructions of a group sum into a
// temporary that is added times the group's scale of each output row, and
// the bias part sum_g bias_g * sum_{k in g} a_k is one more product per item,
// against the activation rows' group sums written beside the planes.
//
// LDS stage: [plane][token][16 cells of 16 bytes]; cell c of token t holds
// octet c ^ pl_swz(t) of the token's 128-wide K step.  A wave load of 64 cells
// covers 4 tokens, 16 lanes reading one token's 256 contiguous bytes.  A
// fragment read takes one octet of 16 tokens (one 256-byte row each); with
// pl_swz(t) = t mod 16 such reads cost two LDS passes instead of one on
// gfx950 (bank-conflict counter, measured by a probe), with the swizzle
// below they cost one.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;
constexpr int pl_stage_bytes(int npl, int nt) { return npl * 16 * nt * 256; }
// a bijection of 0..15: the even cells for tokens 0..7, the odd ones for 8..15
MOE_DEV constexpr int pl_swz(int t) { return ((t << 1) & 15) ^ ((t >> 3) & 1); }

// 16 bytes of LDS at addr + OFF, issued without waiting
template <int OFF>
MOE_DEV void lds_read16(uint32_t addr, u32x4_t &v) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(v) : "v"(addr), "n"(OFF) : "memory");
}
// wait until at most N LDS reads are outstanding; the operand ties the wait to
// the register it protects, so its users stay behind it
template <int N>
MOE_DEV void lds_wait16(u32x4_t &v) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N) : "memory");
}

constexpr int pl_gcd(int a, int b) { return b == 0 ? a : pl_gcd(b, a % b); }

// Weights issued in pairs of K steps: every even step issues the codes of
// steps s + L and s + L + 1 (the two halves of each row's 128-byte line,
// back to back) and their scales, odd steps no weights.  Memory operations
// a wave issues in step i: kq LDS loads, plus wp weight operations when i is
// even.  After step s (of parity sp), LDS stage s + 1 (issued first in step
// s + 2 - S) and weight step s + 1 (issued last in the even step e whose pair
// holds s + 1) must have landed; returns how many operations issued after the
// later of the two may stay in flight.
constexpr int pl_pair_ops(int i, int kq, int wp) { return kq + ((i & 1) == 0 ? wp : 0); }
constexpr int pl_pair_vm_left(int sp, int S, int L, int kq, int wp) {
  const int s = 64 + sp;  // any step of this parity far from the start
  const int e = ((s + 1 - L) & 1) == 0 ? s + 1 - L : s - L;
  int left_w = 0;
  for (int i = e + 1; i <= s; ++i) left_w += pl_pair_ops(i, kq, wp);
  const int a = s + 2 - S;
  int left_a = (a & 1) == 0 ? wp : 0;
  for (int i = a + 1; i <= s; ++i) left_a += pl_pair_ops(i, kq, wp);
  return left_w < left_a ? left_w : left_a;
}

// Eight affine 2-bit codes (a 16-bit run, code i in bits 2i .. 2i+1) as
// exact bf16 integers in element order: the codes are spread one per nibble
// (the low two bits of nibble i), where code q reads as the e2m1 value q / 2,
// and the convert's scale 2 (a power of two: the convert takes only the
// exponent of its scale) gives q.
MOE_DEV bf16x8_t aff2x8_ordered(uint32_t x) {
  x = (x | (x << 8)) & 0x00FF00FFu;  // codes 0-3 in byte 0, 4-7 in byte 2
  x = (x | (x << 4)) & 0x0F0F0F0Fu;  // two codes per byte
  x = (x | (x << 2)) & 0x33333333u;  // one code per nibble
  return fp4x8_to_bf16(x, 2.0f);
}

// WF: MXFP4 or affine 2-bit weights; RW weight-ring slots, S LDS stages, LDS
// reads D fragments ahead; PW = 2: MXFP4 weights issued in pairs of K steps
// (pl_pair_vm_left), RW - 2 steps ahead of the even step of a pair
template <int WF, bool PAIR, int NPL, int NTA, int MT, int NW, int RW, int S, int D, int PW>
__device__ __forceinline__ void pfpl_item(const GemmArgs &g, uint8_t *lds, int expert, int row0, int nrows,
                                          int nb) {
  constexpr bool AFF = WF == W_AFF2;
  static_assert(WF == W_MXFP4 || AFF, "MXFP4 or affine 2-bit weights");
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int CT = 16 * NTA;          // staged tokens
  constexpr int ROWS_WG = 16 * NW * MT;
  constexpr int PLB = CT * 256;         // bytes of one plane in a stage
  constexpr int QI = 4 * NPL * NTA;     // 1 KB wave loads per stage
  constexpr int KQ = (QI + NW - 1) / NW;  // per wave (the last round may leave waves idle)
  static_assert(pl_stage_bytes(NPL, NTA) == QI * 1024, "whole wave loads");
  static_assert(RW >= 2 && RW <= 8 && S >= 2 && S <= 4, "ring shapes");
  static_assert(PW == 1 || (PW == 2 && !AFF && RW % 2 == 0 && RW >= 4), "paired weights: MXFP4, even ring");
  constexpr int L = RW - 2;  // paired weights: the even step s issues steps s + L, s + L + 1
  // stage b of the LDS ring
  auto stage = [&](int b) { return lds + b * pl_stage_bytes(NPL, NTA); };
  constexpr int U = RW * S / pl_gcd(RW, S);  // steps per unrolled round: slot and stage repeat

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;

  // ---- weights into a register ring of RW slots, RW - 1 steps ahead.
  // MXFP4: lane group kg's 16 bytes of a K step are its row's 32 codes of
  // scale group kg, with the row's four scale bytes of the step.  Affine: the
  // lane loads dwords kg and 4 + kg of the step's 32 code bytes (16 codes of
  // each of the step's two groups), with the row's two bf16 scales of the step.
  // Both formats keep K / 32 scale bytes per row.
  const uint32_t row_bytes = AFF ? K / 4 : K / 2, srow_bytes = K / 32;
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
    woff[t] = (uint32_t)n * row_bytes + kg * (AFF ? 4 : 16);
  }
  typename std::conditional<AFF, u32x2_t, u32x4_t>::type wq[RW][NTILE];
  uint32_t wsc[RW][NTILE];
  auto scale_row = [&](int t) { return AFF ? (woff[t] - kg * 4) >> 3 : (woff[t] - kg * 16) >> 4; };

  // ---- activation planes straight into LDS: wave load k of this wave fills
  // cells [64 (wave + NW k), +64) of a stage.  Gathered rows index A from its
  // start; rows in sorted order from the chunk's first row.  Rows past the
  // chunk repeat its first row (their columns are never stored).
  const long long lda = g.lda;  // bf16 elements per activation row
  const char *abase = static_cast<const char *>(g.A) + (g.a_map ? 0LL : (long long)row0 * lda * 2);
  const long long abytes = (g.a_map ? g.a_rows : (long long)nrows) * lda * 2;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(abase, (uint32_t)min(abytes, 0x7FFFFFF0LL));
  uint32_t qoff[KQ];
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const int q = min(64 * (wave + NW * k), 64 * (QI - 1)) + lane;
    const int p = q / (16 * CT), rem = q - p * 16 * CT;
    const int tok = rem >> 4, oct = (rem & 15) ^ pl_swz(tok & 15);
    const int tt = tok < nrows ? tok : 0;
    const long long arow = g.a_map ? (long long)(g.a_map[row0 + tt] / g.a_div) : (long long)tt;
    qoff[k] = (uint32_t)((arow * lda + (long long)p * K) * 2 + oct * 16);
  }
  // the memory operations of one step: KQ loads into LDS stage sb (a wave
  // past the stage's last load skips it: KQ_MIN of them are issued by every
  // wave), then the codes and scales of each weight tile into ring slot wb
  // (WI memory instructions).  The LDS loads go first: they feed the next
  // step, and loads complete in the order they are issued.
  constexpr int NOPS = KQ + 2 * NTILE;
  constexpr int KQ_MIN = QI / NW;
  constexpr int WI = (AFF ? 3 : 2) * NTILE;
  constexpr uint32_t STEP_BYTES = AFF ? 32u : 64u;
  // paired weights: an even step's operations are [KQ LDS loads][codes of
  // step sw0 into slot wb0][codes of step sw1 into slot wb1][the two steps'
  // scale dwords, one 8-byte load per tile]; an odd step's the LDS loads
  constexpr int NOPS_E = KQ + 3 * NTILE, NOPS_O = KQ;
  auto issue_pair_op = [&](int o, int sb, int wb0, int wb1, int sa, int sw0, int sw1) {
    if (o < KQ) {
      const int ii = wave + NW * o;  // uniform
      if (ii < QI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)(stage(sb) + ii * 1024), 16, qoff[o],
                                                 (uint32_t)sa * 256u, 0, 0);
    } else if (o < KQ + NTILE) {
      const int t = o - KQ;
      if constexpr (!AFF) wq[wb0][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)sw0 * STEP_BYTES);
    } else if (o < KQ + 2 * NTILE) {
      const int t = o - KQ - NTILE;
      if constexpr (!AFF) wq[wb1][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)sw1 * STEP_BYTES);
    } else {
      // scales of steps sw0 and sw0 + 1 (past the row's last step the second
      // dword belongs to no computed step)
      const int t = o - KQ - 2 * NTILE;
      const u32x2_t v = buf_load8(sr[t / MT], scale_row(t), (uint32_t)sw0 * 4u);
      wsc[wb0][t] = v[0];
      wsc[wb1][t] = v[1];
    }
  };
  auto issue_op = [&](int o, int sb, int wb, int sa, int sw) {
    if (o < KQ) {
      const int ii = wave + NW * o;  // uniform
      if (ii < QI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)(stage(sb) + ii * 1024), 16, qoff[o],
                                                 (uint32_t)sa * 256u, 0, 0);
    } else if (o < KQ + NTILE) {
      const int t = o - KQ;
      if constexpr (AFF)
        wq[wb][t] = u32x2_t{buf_load4(wr[t / MT], woff[t], (uint32_t)sw * STEP_BYTES),
                            buf_load4(wr[t / MT], woff[t] + 16u, (uint32_t)sw * STEP_BYTES)};
      else
        wq[wb][t] = buf_load16(wr[t / MT], woff[t], (uint32_t)sw * STEP_BYTES);
    } else {
      const int t = o - KQ - NTILE;
      wsc[wb][t] = buf_load4(sr[t / MT], scale_row(t), (uint32_t)sw * 4u);
    }
  };

  f32x4_t acc[NTILE][NTA];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment reads: in sub-step j (K 32 wide) lane (token r16, group kg) takes
  // one octet of its token: MXFP4, octet 4 kg + j, the K positions of its
  // weight codes 8j .. 8j+7; affine, octet aff2_octet(j / 2, kg, j % 2), so
  // that sub-steps 2h and 2h + 1 cover 64-element group h of the step
  auto octet = [&](int j) { return AFF ? aff2_octet(j >> 1, kg, j & 1) : 4 * kg + j; };
  uint32_t la[S][4];
#pragma unroll
  for (int b = 0; b < S; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) la[b][j] = lds_addr(stage(b)) + (uint32_t)(r16 * 256 + ((octet(j) ^ pl_swz(r16)) << 4));

  // step s from LDS stage SB and weight slot WB; its fragments f = (sub-step
  // j, plane p, token tile n) are read from LDS D ahead of their MFMAs; the
  // weights of sub-step j + 1 are converted tile by tile over sub-step j's
  // fragments; over the first half of the step go out the loads of LDS stage
  // s + S - 1 (stage SN, which held step s - 1) and then of weight step
  // s + RW - 1 (slot WN, which held step s - 1).  Step indices past the last
  // step reload the last one; before the first (the prologue) they load step 0.
  auto compute = [&](auto sbc, auto wbc, int s) {
    constexpr int SB = decltype(sbc)::value, WB = decltype(wbc)::value;
    constexpr int WN = (WB + RW - 1) % RW, SN = (SB + S - 1) % S;
    const int sa = min(s + S - 1, nks - 1), sw = min(s + RW - 1, nks - 1);
    // paired weights (WB = s mod RW, RW even, so WB has the parity of s)
    constexpr bool EVEN = (WB & 1) == 0;
    constexpr int WP0 = (WB + L) % RW, WP1 = (WB + L + 1) % RW;
    const int sw0 = min(s + L, nks - 1), sw1 = min(s + L + 1, nks - 1);
    constexpr int NOPS_S = PW == 1 ? NOPS : EVEN ? NOPS_E : NOPS_O;
    constexpr int FJ = NPL * NTA;  // fragments per sub-step
    constexpr int F = 4 * FJ;
    constexpr int J = (NOPS_S + F / 2 - 1) / (F / 2);  // loads issued per fragment
    u32x4_t bq[D + 1];
    // converted weights: sub-step j + 1 is converted over sub-step j's
    // fragments into the other buffer; items of five or six token tiles with
    // paired weights (whose ring takes the registers) convert each sub-step's
    // tiles at its start into one buffer
    constexpr int WAB = (PW == 2 && NTA >= 5) ? 1 : 2;
    bf16x8_t wa[WAB][NTILE];
    // MXFP4: the scale of the lane's scale group; affine: the two groups'
    // scales of the lane's four output rows 4 kg + r (from the lanes that
    // loaded those rows), with a temporary sum per group
    float scl[NTILE];
    uint32_t sc[AFF ? NTILE : 1][4];  // bf16 pairs: group 0 low, group 1 high
    f32x4_t tmp[AFF ? NTILE : 1][AFF ? NTA : 1];
    if constexpr (AFF) {
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[t][r] = (uint32_t)__shfl((int)wsc[WB][t], 4 * kg + r, 64);
#pragma unroll
        for (int n = 0; n < NTA; ++n) tmp[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    } else {
#pragma unroll
      for (int t = 0; t < NTILE; ++t) scl[t] = e8m0_to_float((wsc[WB][t] >> (8 * kg)) & 0xFFu);
    }
    // sub-step j of tile t: MXFP4 dword j; affine, half j % 2 of dword j / 2
    auto convert = [&](int j, int t) -> bf16x8_t {
      if constexpr (AFF) return aff2x8_ordered((wq[WB][t][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      else return fp4x8_to_bf16(wq[WB][t][j], scl[t]);
    };
    auto issue = [&](auto fc) {
      constexpr int f = decltype(fc)::value;
      constexpr int j = f / FJ, p = (f / NTA) % NPL, n = f % NTA;
      lds_read16<p * PLB + n * 16 * 256>(la[SB][j], bq[f % (D + 1)]);
    };
    static_for<(D < F ? D : F)>([&](auto fc) { issue(fc); });
#pragma unroll
    for (int t = 0; t < NTILE; ++t) wa[0][t] = convert(0, t);
    static_for<F>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      constexpr int j = f / FJ, i = f % FJ, n = f % NTA;
      if constexpr (f + D < F) issue(std::integral_constant<int, f + D>{});
      if constexpr (WAB == 2 && j + 1 < 4) {
        // tiles [i NTILE / FJ, (i + 1) NTILE / FJ) of sub-step j + 1
#pragma unroll
        for (int t = (i * NTILE) / FJ; t < ((i + 1) * NTILE) / FJ; ++t) wa[(j + 1) & 1][t] = convert(j + 1, t);
      }
      if constexpr (WAB == 1 && i == 0 && j > 0) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) wa[0][t] = convert(j, t);
      }
      constexpr int behind = (f + D < F) ? D : F - 1 - f;  // reads issued after f
      lds_wait16<behind>(bq[f % (D + 1)]);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bq[f % (D + 1)]);
      if constexpr (AFF) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) tmp[t][n] = mfma_16x16x32(wa[(j & 1) % WAB][t], bv, tmp[t][n]);
        if constexpr ((f + 1) % (2 * FJ) == 0) {
          // group h of the step is complete: add it times its scales
          constexpr int h = f / (2 * FJ);
#pragma unroll
          for (int t = 0; t < NTILE; ++t)
#pragma unroll
            for (int m = 0; m < NTA; ++m) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[t][m][r] = fmaf(h ? __uint_as_float(sc[t][r] & 0xFFFF0000u) : bf16_lo_to_float(sc[t][r]),
                                    tmp[t][m][r], acc[t][m][r]);
              tmp[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
      } else {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[t][n] = mfma_16x16x32(wa[(j & 1) % WAB][t], bv, acc[t][n]);
      }
#pragma unroll
      for (int o = f * J; o < (f + 1) * J && o < NOPS_S; ++o) {
        if constexpr (PW == 1) issue_op(o, SN, WN, sa, sw);
        else issue_pair_op(o, SN, WP0, WP1, sa, sw0, sw1);
      }
    });
  };
  // After step s, stage s + 1 must be in LDS for every wave and weight step
  // s + 1 in registers.  Every step issues [LDS loads][weight loads]; stage
  // s + 1 went out in step s + 2 - S, weight step s + 1 in step s + 2 - RW, and
  // the loads issued after the later of the two may stay in flight.
  constexpr int PER_STEP = KQ_MIN + WI;
  constexpr int AFTER_A = WI + (S - 2) * PER_STEP, AFTER_W = (RW - 2) * PER_STEP;
  constexpr int VM_LEFT = AFTER_A < AFTER_W ? AFTER_A : AFTER_W;
  // paired weights: by the parity of the step just computed
  constexpr int VM_LEFT_E = pl_pair_vm_left(0, S, L, KQ_MIN, 3 * NTILE);
  constexpr int VM_LEFT_O = pl_pair_vm_left(1, S, L, KQ_MIN, 3 * NTILE);
  static_assert(VM_LEFT < 64 && VM_LEFT_E < 64 && VM_LEFT_O < 64, "vmcnt range");
  auto wait_and_sync = [&](auto oddc) {
    constexpr int V = PW == 1 ? VM_LEFT : decltype(oddc)::value ? VM_LEFT_O : VM_LEFT_E;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(V));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);  // keep the next step's register work behind the wait
  };
  static_assert(PW == 1 || U % 2 == 0, "paired weights: rounds of whole pairs");
  auto step = [&](auto ic, int s) {
    constexpr int I = decltype(ic)::value;
    compute(std::integral_constant<int, I % S>{}, std::integral_constant<int, I % RW>{}, s);
    wait_and_sync(std::integral_constant<bool, (I & 1) == 1>{});
  };

  // prologue: the loads of steps -M .. -1, in the same pattern as every step
  // (paired weights: M covers the pairs of steps 0 .. L - 1 and no earlier pair)
  constexpr int M = PW == 1 ? (RW > S ? RW : S) - 1 : (L > S - 1 ? L : S - 1);
  static_assert(PW == 1 || M < L + 2, "no pair before step 0");
  static_for<M>([&](auto ic) {
    constexpr int r = decltype(ic)::value - M;  // -M .. -1
    constexpr int SN = ((r + S - 1) % S + S) % S, WN = ((r + RW - 1) % RW + RW) % RW;
    const int sa = max(min(r + S - 1, nks - 1), 0), sw = max(min(r + RW - 1, nks - 1), 0);
    if constexpr (PW == 1) {
#pragma unroll
      for (int o = 0; o < NOPS; ++o) issue_op(o, SN, WN, sa, sw);
    } else {
      constexpr bool EVEN = (r & 1) == 0;
      constexpr int WP0 = ((r + L) % RW + RW) % RW, WP1 = ((r + L + 1) % RW + RW) % RW;
      const int sw0 = max(min(r + L, nks - 1), 0), sw1 = max(min(r + L + 1, nks - 1), 0);
#pragma unroll
      for (int o = 0; o < (EVEN ? NOPS_E : NOPS_O); ++o) issue_pair_op(o, SN, WP0, WP1, sa, sw0, sw1);
    }
  });
  wait_and_sync(std::true_type{});  // the virtual step -1 is odd
  int s = 0;
  for (; s + U - 1 < nks; s += U) static_for<U>([&](auto ic) { step(ic, s + decltype(ic)::value); });
  // tail: s is a multiple of U, so step i keeps stage i % S and slot i % RW
  static_for<U - 1>([&](auto ic) {
    if (s + decltype(ic)::value < nks) step(ic, s + decltype(ic)::value);
  });
  // drain the loads past the last step before the LDS is reused
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  if constexpr (AFF) {
    // the bias part sum_g b_g sum_{k in g} a_k: the biases of the lane's row,
    // eight groups per 32-group slice (M side), against the token rows' group
    // sums in hi + lo (N side); groups past the row's end contribute zero
    const int ngroups = K / 64;
    bf16x8_t bw[NTILE][2];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const __amdgpu_buffer_rsrc_t br =
          make_rsrc((t / MT ? g.B1 : g.B0) + expert * (g.s_estride / 2), (uint32_t)N * srow_bytes);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int g0 = 8 * kg + 32 * i;
        const u32x4_t v = g0 < ngroups ? buf_load16(br, scale_row(t) + 2 * g0, 0) : u32x4_t{0, 0, 0, 0};
        bw[t][i] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
#pragma unroll
    for (int n = 0; n < NTA; ++n) {
      const int tok = 16 * n + r16;
      const int tt = tok < nrows ? tok : 0;
      const long long arow = (g.a_map && !g.asum_sorted) ? (long long)(g.a_map[row0 + tt] / g.a_div)
                                                          : (long long)(row0 + tt);
      const float *srow = g.asum + arow * ngroups;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int g0 = 8 * kg + 32 * i;
        f32x4_t v0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (g0 < ngroups) {
          v0 = reinterpret_cast<const f32x4_t *>(srow + g0)[0];
          v1 = reinterpret_cast<const f32x4_t *>(srow + g0)[1];
        }
        bf16x8_t sh, sl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 h, l;
          split_bf16(e < 4 ? v0[e] : v1[e - 4], h, l);
          sh[e] = h;
          sl[e] = l;
        }
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
          acc[t][n] = mfma_16x16x32(bw[t][i], sh, acc[t][n]);
          acc[t][n] = mfma_16x16x32(bw[t][i], sl, acc[t][n]);
        }
      }
    }
  }

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
        if (g.c_hi != nullptr) {
          // bf16 planes: hi = bf16(v), lo = bf16(v - hi), rows of ldc elements
          bf16x4_t h, l;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            __bf16 hr, lr;
            split_bf16(v[r], hr, lr);
            h[r] = hr;
            l[r] = lr;
          }
          const long long o = orow * g.ldc + col0;
          if (col0 + 3 < N) {
            *reinterpret_cast<bf16x4_t *>(g.c_hi + o) = h;
            *reinterpret_cast<bf16x4_t *>(g.c_lo + o) = l;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (col0 + r < N) {
                g.c_hi[o + r] = __builtin_bit_cast(uint16_t, h[r]);
                g.c_lo[o + r] = __builtin_bit_cast(uint16_t, l[r]);
              }
          }
        } else {
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
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Weight-ring slots and LDS stages.  Items with one or two token tiles have
// steps too short to cover a memory trip: their weights go three steps ahead
// and their activation stages (small, so four fit) three steps ahead too.
// Larger items: three and three; affine weights (more registers per tile),
// two and two.
// MXFP4 weights are issued in pairs of K steps (both halves of each row's
// 128-byte line back to back: one step apart, most second halves missed the
// L2 and the weight lines crossed the memory bus about 1.75 times); their ring
// holds the step pair computed and one pair in flight (two for items of one
// or two token tiles, whose steps are short).  Items of six token
// tiles keep single steps and a ring of three: the accumulators leave no
// registers for a fourth slot.
constexpr int pl_pw(int wf, int nta) { return wf == W_AFF2 || nta == 6 ? 1 : 2; }
constexpr int pl_ring(int wf, int nta) {
  return wf == W_AFF2 ? (nta <= 2 ? 4 : 2) : nta == 6 ? 3 : nta <= 2 ? 6 : 4;
}
constexpr int pl_stages(int wf, int nta) { return nta <= 2 ? 4 : wf == W_AFF2 ? 2 : 3; }
// fragment reads ahead of their MFMAs (affine weights: one, for registers)
constexpr int pl_d(int wf) { return wf == W_AFF2 ? 1 : 2; }
// LDS of the largest ring over the item shapes 1 .. nt
constexpr int pl_lds_bytes(int wf, int npl, int nt) {
  return nt == 0 ? 0
                 : (pl_stages(wf, nt) * pl_stage_bytes(npl, nt) > pl_lds_bytes(wf, npl, nt - 1)
                        ? pl_stages(wf, nt) * pl_stage_bytes(npl, nt)
                        : pl_lds_bytes(wf, npl, nt - 1));
}

template <int WF, bool PAIR, int NPL, int NT, int MT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_pl_kernel(GemmArgs g) {
  // the activation ring: stages of the item's shape, back to back (the LDS
  // reads wait on their own loads explicitly, so one object serves all stages)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[pl_lds_bytes(WF, NPL, NT)];
  static_assert(NT >= 1 && NT <= 6, "the item dispatch covers 1..6 active token tiles");
  const int total = min(*g.chunk_count * g.n_blocks, g.grid_logical);
  const int logical = xcd_logical(total);
  if (logical < 0) return;
  const int chunk = logical / g.n_blocks;
  const int nb = logical - chunk * g.n_blocks;
  const int4 c = reinterpret_cast<const int4 *>(g.chunks)[chunk];
  const int nta = min((c.z + 15) >> 4, NT);
#define MOE_PL_ITEM(A) \
  pfpl_item<WF, PAIR, NPL, A, MT, NW, pl_ring(WF, A), pl_stages(WF, A), pl_d(WF), pl_pw(WF, A)>(g, lds, c.x, c.y, c.z, nb)
  if (nta == NT) {
    MOE_PL_ITEM(NT);
    return;
  }
  switch (nta) {
    case 1: if constexpr (NT > 1) MOE_PL_ITEM(1); break;
    case 2: if constexpr (NT > 2) MOE_PL_ITEM(2); break;
    case 3: if constexpr (NT > 3) MOE_PL_ITEM(3); break;
    case 4: if constexpr (NT > 4) MOE_PL_ITEM(4); break;
    default: if constexpr (NT > 5) MOE_PL_ITEM(5); break;
  }
#undef MOE_PL_ITEM
}

// fp32 rows -> [rows][NPL][K] bf16 rows: hi = bf16(a) and lo = bf16(a - hi)
// (NPL 2), or the rounded row alone (NPL 1); output row r is activation row
// map[r] / div (map NULL: row r); 8 values per thread.  With sums given, also
// each row's 64-element group sums [rows][K / 64] (fp32, the eight threads of
// a group in one wavefront; bf16 input: the sums alone).
template <typename TIn, int NPL, bool SUMS>
__global__ __launch_bounds__(256) void split_rows_kernel(const TIn *__restrict__ A, long long lda, long long rows,
                                                         int K, const int32_t *__restrict__ map, int div,
                                                         __bf16 *__restrict__ out, float *__restrict__ sums) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = K / 8;
  if (i >= rows * per_row) return;  // whole groups of eight threads (K / 8 is a multiple of 8 with sums)
  const long long row = i / per_row;
  const int c = (int)(i - row * per_row);
  const long long src = map ? (long long)(map[row] / div) : row;
  float v[8];
  if constexpr (std::is_same<TIn, float>::value) {
    const f32x4_t *p = reinterpret_cast<const f32x4_t *>(A + src * lda + c * 8);
    const f32x4_t x0 = p[0], x1 = p[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < 4 ? x0[e] : x1[e - 4];
  } else {
    const bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(A + src * lda + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = from_bf16(x[e]);
  }
  if (out != nullptr) {
    bf16x8_t h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 vh, vl;
      split_bf16(v[e], vh, vl);
      h[e] = NPL == 2 ? vh : to_bf16(v[e]);
      l[e] = vl;
    }
    __bf16 *o = out + row * NPL * K + c * 8;
    *reinterpret_cast<bf16x8_t *>(o) = h;
    if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(o + K) = l;
  }
  if constexpr (SUMS) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += v[e];
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    if ((c & 7) == 0) sums[row * (K / 64) + (c >> 3)] = part;
  }
}

// Waves per work-group and 16-row weight tiles per wave and matrix: eight
// waves (two per SIMD); MXFP4, 4 tiles per wave (2 + 2 for a SiTU pair);
// affine weights keep a temporary sum per tile beside the result, so their
// waves hold 2 tiles.
constexpr int pl_nw(int wf) { return 8; }
constexpr int pl_mt(int wf, bool pair) { return (wf == W_AFF2 ? 1 : 2) * (pair ? 1 : 2); }

template <int WF>
hipError_t launch_pl(int npl, bool pair, const GemmArgs &a, long long grid, hipStream_t st) {
  constexpr int NW = pl_nw(WF);
  const dim3 gr((unsigned)grid), blk(64 * NW);
  if (npl == 2) {
    if (pair) hipLaunchKernelGGL((prefill_pl_kernel<WF, true, 2, PREFILL_NT, pl_mt(WF, true), NW>), gr, blk, 0, st, a);
    else hipLaunchKernelGGL((prefill_pl_kernel<WF, false, 2, PREFILL_NT, pl_mt(WF, false), NW>), gr, blk, 0, st, a);
  } else {
    if (pair) hipLaunchKernelGGL((prefill_pl_kernel<WF, true, 1, PREFILL_NT, pl_mt(WF, true), NW>), gr, blk, 0, st, a);
    else hipLaunchKernelGGL((prefill_pl_kernel<WF, false, 1, PREFILL_NT, pl_mt(WF, false), NW>), gr, blk, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

int prefill_pl_rows_per_wg(bool pair, int wfmt) {
  return 16 * (wfmt == W_AFF2 ? pl_nw(W_AFF2) : pl_nw(W_MXFP4)) * pl_mt(wfmt, pair);
}

hipError_t launch_prefill_planes(int wfmt, int npl, bool pair, const GemmArgs &a, long long grid, hipStream_t st) {
  if (a.chunks == nullptr || (npl != 1 && npl != 2) || a.K % KSTEP != 0) return hipErrorInvalidValue;
  if (wfmt == W_AFF2) {
    // whole 512-element runs of groups, at most 64 groups (two 32-group bias slices)
    if (a.asum == nullptr || a.B0 == nullptr || a.K % 512 != 0 || a.K > 4096) return hipErrorInvalidValue;
    return launch_pl<W_AFF2>(npl, pair, a, grid, st);
  }
  if (wfmt != W_MXFP4) return hipErrorInvalidValue;
  return launch_pl<W_MXFP4>(npl, pair, a, grid, st);
}

size_t split_rows_bytes(long long rows, int K, int npl) { return (size_t)rows * npl * K * 2; }
size_t row_sums_bytes(long long rows, int K) { return (size_t)rows * (K / 64) * 4; }

hipError_t launch_split_rows(int npl, const float *A, long long lda, long long rows, int K, const int32_t *map,
                             int div, uint16_t *out, float *sums, hipStream_t st) {
  if ((npl != 1 && npl != 2) || K % 8 != 0 || (sums && K % 512 != 0)) return hipErrorInvalidValue;
  const long long n = rows * (K / 8);
  const dim3 gr((unsigned)((n + 255) / 256)), blk(256);
  __bf16 *o = reinterpret_cast<__bf16 *>(out);
  if (sums) {
    if (npl == 2) hipLaunchKernelGGL((split_rows_kernel<float, 2, true>), gr, blk, 0, st, A, lda, rows, K, map, div, o, sums);
    else hipLaunchKernelGGL((split_rows_kernel<float, 1, true>), gr, blk, 0, st, A, lda, rows, K, map, div, o, sums);
  } else {
    if (npl == 2) hipLaunchKernelGGL((split_rows_kernel<float, 2, false>), gr, blk, 0, st, A, lda, rows, K, map, div, o, sums);
    else hipLaunchKernelGGL((split_rows_kernel<float, 1, false>), gr, blk, 0, st, A, lda, rows, K, map, div, o, sums);
  }
  return hipGetLastError();
}

hipError_t launch_row_sums(const uint16_t *A, long long lda, long long rows, int K, const int32_t *map, int div,
                           float *sums, hipStream_t st) {
  if (K % 512 != 0) return hipErrorInvalidValue;
  const long long n = rows * (K / 8);
  hipLaunchKernelGGL((split_rows_kernel<__bf16, 1, true>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const __bf16 *>(A), lda, rows, K, map, div, nullptr, sums);
  return hipGetLastError();
}

}  // namespace moe
