// Tiled bf16 GEMM for the dense products at prefill sizes (router, latent
// down projection, up projection, shared experts):
//   C[t, n] (+)= sum_k A[t, k] W[n, k]   or, for a SiTU-GLU pair,
//   C[t, n] = SiTU(sum_k A[t, k] W0[n, k], sum_k A[t, k] W1[n, k]).
//
// Work item: 256 tokens x 256 weight rows (a pair: 128 gate rows and the 128
// up rows of the same output columns), optionally one of `splits` K ranges.
// Eight waves, two per SIMD, each own 128 weight rows x 64 tokens as 4 x 2
// tiles of v_mfma_f32_32x32x16_bf16 (weights on the MFMA's M side, tokens
// on its N side; 128 accumulator registers).  With one wave per SIMD (4 x 4
// tiles each) the MFMA pipe idled through every step's barrier and LDS waits;
// the second wave of a SIMD fills them (the layer-0 FFN at T = 4096: 7.78 to
// 7.20 ms).
//
// Both operands reach LDS through direct-to-LDS buffer loads in which eight
// consecutive lanes fetch one 128-byte line, so every L1 request is a whole
// line.  A stage holds KS values of K for the 256 weight rows and for the 256
// tokens of each activation plane (one plane of bf16 activations, or the hi
// and lo planes of fp32 activations split beforehand), in a ring of three or
// four stages, so the loads run two or three K steps ahead.  Inside LDS, 16-byte
// chunk c of row r sits at line r / RPL, slot ((r % RPL) * CPR + c) ^ (line
// % 8): the eight lanes an MFMA operand read serves at a time hit eight
// different slots, so the reads are free of bank conflicts.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int DT = 256;  // tokens and weight rows per work-group
constexpr int DNW = 8;   // waves: two halves of the weight rows x DNW / 2 slices of the tokens
constexpr int DNB = DT / (DNW / 2) / 32;  // 32-token tiles per wave


MOE_DEV f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}


// 16 bytes of LDS at a + O, issued without waiting
template <int O>
MOE_DEV void dread(uint32_t a, u32x4_t &v) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(v) : "v"(a), "n"(O) : "memory");
}
template <int N>
MOE_DEV void dwait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
// ties a register to the preceding wait: its users stay behind it
MOE_DEV void dtie(u32x4_t &v) { asm volatile("" : "+v"(v)); }

template <int KS>
struct DLayout {
  static constexpr int CPR = KS / 8;          // 16-byte chunks per row
  static constexpr int RPL = 128 / (2 * KS);  // rows per 128-byte line
  static constexpr int ROW_BYTES = 2 * KS;
  static constexpr int REGION = DT * ROW_BYTES;  // bytes of 256 rows
  // slot swizzle of a line: the 8 rows (4 lines) one 128-byte read pass
  // serves and the 16 rows (8 lines) of a 256-byte pass both land on distinct
  // 16-byte bank groups; it repeats every 4 lines within a 16-line period and
  // is unchanged by a shift of 16 lines (32 rows, one MFMA tile)
  static MOE_DEV int swz(int line) { return (line + (line >> 2)) & 3; }
  static MOE_DEV int slot_offset(int r, int c) {
    const int line = r / RPL;
    return line * 128 + ((((r % RPL) * CPR) + c) ^ swz(line)) * 16;
  }
};

// global byte offset of the 16 bytes lane `lane` of wave load ii fetches
// (weights: region 0 of the stage, rows clamped to N; activations: regions
// 1, 2, rows clamped to the token count)
template <int KS, bool PAIR>
MOE_DEV uint32_t dense_voff(int ii, int lane, int n0, int t0, int N, int K, int rows, long long lda, int k0) {
  using Lay = DLayout<KS>;
  constexpr int REG = Lay::REGION;
  const int region = (ii * 1024) / REG;
  const int line = ((ii * 1024) % REG) / 128 + lane / 8;
  const int u = (lane % 8) ^ Lay::swz(line);
  const int r = line * Lay::RPL + u / Lay::CPR;
  const int c = u % Lay::CPR;
  if (region == 0) {
    int n = PAIR ? n0 + (r % (DT / 2)) : n0 + r;  // a pair: rows 0..127 gate, 128..255 up
    n = n < N ? n : N - 1;
    return (uint32_t)(((long long)n * K + k0) * 2 + c * 16);
  }
  const int t = t0 + r < rows ? t0 + r : rows - 1;
  return (uint32_t)(((long long)t * lda + k0) * 2 + c * 16);
}

// K per stage and LDS bytes of a stage for NPL activation planes
constexpr int dense_ks(int npl) { return 32; }  // two 64-byte rows per 128-byte line
constexpr int dense_stage_bytes(int npl) { return (1 + npl) * DT * 2 * dense_ks(npl); }
// stages in the LDS ring: loads run NST - 1 K steps ahead of the MFMAs
constexpr int dense_stages(int npl) { return npl == 1 ? 4 : 3; }

template <int NPL, bool PAIR>
MOE_DEV void dense_tile_body(const GemmArgs &g, uint8_t *ring) {
  constexpr int KS = dense_ks(NPL);
  using Lay = DLayout<KS>;
  constexpr int REG = Lay::REGION;
  constexpr int STAGE = (1 + NPL) * REG;
  static_assert(STAGE == dense_stage_bytes(NPL), "stage size");
  constexpr int NL = STAGE / 1024;        // 1 KB wave loads per stage
  constexpr int KL = NL / DNW;            // per wave
  constexpr int J = KS / 16;              // MFMA K steps per stage
  static_assert(NL % DNW == 0 && (REG / 1024) % (2 * DNW) == 0, "loads split evenly; regions and halves whole");
  static_assert(Lay::RPL == 2, "the swizzle is laid out for two rows per line");

  const int n_tiles = g.n_blocks;
  const int t_tiles = g.dense_rows_tiles;
  const int total = n_tiles * t_tiles * g.splits;
  const int logical = xcd_logical(total);
  if (logical < 0) return;
  // token tiles of one weight tile (and split) are consecutive: they share its rows in L2
  const int split = logical / (n_tiles * t_tiles);
  const int rem = logical - split * n_tiles * t_tiles;
  const int nt = rem / t_tiles;
  const int tt = rem - nt * t_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = g.N, K = g.K, rows = g.dense_rows;
  const int ksplit = K / g.splits;           // a multiple of 128 (host-checked)
  const int nks = ksplit / KS;
  const int k0 = split * ksplit;
  const int ncols = PAIR ? DT / 2 : DT;      // output columns of a weight tile
  const int n0 = nt * ncols;
  const int t0 = tt * DT;

  // ---- loads: wave load ii of a stage covers bytes [ii KB, +1 KB) of the
  // stage = lines 8 ii .. 8 ii + 7 of region ii / (REG / 1024) (weights, then
  // activation planes); lane -> (line, slot) -> (row, chunk)
  // descriptors: weights (gate / up of a pair), activation planes
  __amdgpu_buffer_rsrc_t rsrc[4];
  rsrc[0] = make_rsrc(g.W0, (uint32_t)((long long)N * K * 2));
  rsrc[1] = make_rsrc(PAIR ? g.W1 : g.W0, (uint32_t)((long long)N * K * 2));
  rsrc[2] = make_rsrc(g.A, (uint32_t)((long long)rows * g.lda * 2));
  rsrc[3] = make_rsrc(NPL == 2 ? g.A2 : g.A, (uint32_t)((long long)rows * g.lda * 2));
  // wave load k of this wave for stage buffer stg and K step s; region and
  // matrix half follow from k alone (regions and halves are whole multiples
  // of DNW loads), so the descriptor choice folds away.  The lane offsets do
  // not depend on s (the compiler keeps them out of the K loop).
  auto load_one = [&](uint8_t *stg, int k, int s) {
    const int ii = wave + DNW * k;  // uniform
    const int region = (DNW * k * 1024) / REG;
    const int upper = (PAIR && ((DNW * k * 1024) % REG) >= REG / 2) ? 1 : 0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc[region == 0 ? upper : 1 + region], (lds_void *)(stg + ii * 1024),
                                             16, dense_voff<KS, PAIR>(ii, lane, n0, t0, N, K, rows, g.lda, k0),
                                             (uint32_t)s * (uint32_t)(KS * 2), 0, 0);
  };
  auto load_stage = [&](uint8_t *stg, int s) {
#pragma unroll
    for (int k = 0; k < KL; ++k) load_one(stg, k, s);
  };

  // ---- operand reads: wave (wm, wn) = (wave % (DNW / 2), wave / (DNW / 2))
  // owns tokens 32 DNB wm .. + 32 DNB - 1 and weight rows 128 wn .. +127 of
  // the tile (a pair: gate rows 64 wn .. +63 and the up rows 128 + 64 wn ..
  // +63).  Lane l reads row l % 32 of each 32-row tile, chunk 2 j + l / 32 of
  // MFMA step j.
  const int wm = wave % (DNW / 2), wn = wave / (DNW / 2);
  const int l32 = lane & 31, lh = lane >> 5;
  // per-lane offsets within a region of row l32 (+32 a for tile a), chunk 2 j + lh;
  // 32 rows are a whole number of 8-line swizzle periods, so the tile offset is a constant
  uint32_t roff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) roff[j] = (uint32_t)Lay::slot_offset(l32, 2 * j + lh);
  constexpr int TILE_OFF = 32 * Lay::ROW_BYTES;  // bytes between 32-row tiles
  auto wrow_tile = [&](int a) -> int {  // first WG row of the wave's weight tile a (0..3)
    if constexpr (PAIR) return (a < 2 ? 64 * wn + 32 * a : DT / 2 + 64 * wn + 32 * (a - 2));
    else return 128 * wn + 32 * a;
  };
  constexpr int NST = dense_stages(NPL);
  const uint32_t ring_base = lds_addr(ring);
  // weight rows and token rows of the wave as region offsets
  const int wrow0 = wrow_tile(0);
  const int tokrow0 = 32 * DNB * wm;

  f32x16_t acc[4][DNB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < DNB; ++b) acc[a][b] = f32x16_t{};

  constexpr int R = 4 + DNB * NPL;  // fragment reads per MFMA step
  static_assert(J % 2 == 0, "fragment buffers alternate with the MFMA step");
  u32x4_t fw[2][4], ft[2][NPL][DNB];
  // reads of MFMA step j of the stage at `base` into fragment buffer j % 2
  auto issue = [&](uint32_t base, auto jc) {
    constexpr int j = decltype(jc)::value;
    const uint32_t aw = base + roff[j] + (uint32_t)(wrow0 / 32) * TILE_OFF;
    const uint32_t at = base + roff[j] + (uint32_t)(tokrow0 / 32) * TILE_OFF;
    if constexpr (PAIR) {
      dread<0>(aw, fw[j & 1][0]);
      dread<TILE_OFF>(aw, fw[j & 1][1]);
      dread<(DT / 2 / 32) * TILE_OFF>(aw, fw[j & 1][2]);
      dread<(DT / 2 / 32 + 1) * TILE_OFF>(aw, fw[j & 1][3]);
    } else {
      dread<0>(aw, fw[j & 1][0]);
      dread<TILE_OFF>(aw, fw[j & 1][1]);
      dread<2 * TILE_OFF>(aw, fw[j & 1][2]);
      dread<3 * TILE_OFF>(aw, fw[j & 1][3]);
    }
    static_for<NPL>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      static_for<DNB>([&](auto bc) {
        constexpr int b = decltype(bc)::value;
        dread<(1 + p) * REG + b * TILE_OFF>(at, ft[j & 1][p][b]);
      });
    });
  };
  auto tie = [&](int q) {
#pragma unroll
    for (int a = 0; a < 4; ++a) dtie(fw[q][a]);
#pragma unroll
    for (int p = 0; p < NPL; ++p)
#pragma unroll
      for (int b = 0; b < DNB; ++b) dtie(ft[q][p][b]);
  };
  auto mfmas = [&](int q) {
#pragma unroll
    for (int p = 0; p < NPL; ++p)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < DNB; ++b) acc[a][b] = mfma32(fw[q][a], ft[q][p][b], acc[a][b]);
  };
  auto slot_base = [&](int s) { return ring_base + (uint32_t)((s % NST) * STAGE); };

  // ring of NST stages, K step s in slot s % NST.  Step s first refills the
  // slot step s - 1 used (every wave has passed the barrier after it) with
  // step s + NST - 1, then computes; at its end step s + 1 must have landed,
  // so NST - 2 stages of loads may stay in flight.  Loads past the last step
  // re-read it into slots that are not read again.  The products of a step's
  // last MFMA step run after the barrier, behind the next step's first reads,
  // so no step starts on an exposed LDS latency.
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) load_stage(ring + s * STAGE, min(s, nks - 1));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(KL * (NST - 2)));
  __builtin_amdgcn_s_barrier();
  issue(slot_base(0), std::integral_constant<int, 0>{});
  for (int s = 0; s < nks; ++s) {
    const int fill = (s + NST - 1) % NST;
    load_stage(ring + fill * STAGE, min(s + NST - 1, nks - 1));
    const uint32_t base = slot_base(s);
    static_for<J>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j + 1 < J) {
        issue(base, std::integral_constant<int, j + 1>{});
        dwait<R>();
        tie(j & 1);
        mfmas(j & 1);
      } else {
        dwait<0>();  // this stage's reads are done before the barrier
        tie(j & 1);
      }
    });
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(KL * (NST - 2)));
    __builtin_amdgcn_s_barrier();
    // the next step's first fragments (past the last step: a read of a slot
    // that holds valid data, drained below), then the deferred products
    issue(slot_base(min(s + 1, nks - 1)), std::integral_constant<int, 0>{});
    mfmas((J - 1) & 1);
  }
  dwait<0>();
  tie(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // ---- epilogue: acc[a][b] register i of lane l is weight row 32 a + (i % 4)
  // + 8 (i / 4) + 4 (l / 32) and token 32 b + l % 32 of the wave's tiles
  float *C = g.splits > 1 ? g.partial + (long long)split * rows * (PAIR ? 2 * N : N) : g.C;
  const long long ldc = g.splits > 1 ? (PAIR ? 2 * N : N) : g.ldc;
  const bool acc_in = g.splits == 1 && g.accumulate;
  // 16-byte stores need every row to start 16-byte aligned
  const bool vec_ok = (ldc & 3) == 0;
#pragma unroll
  for (int b = 0; b < DNB; ++b) {
    const int t = t0 + tokrow0 + 32 * b + l32;
    if (t >= rows) continue;
    float *crow = C + (long long)t * ldc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // groups of four consecutive weight rows
      if constexpr (PAIR) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int col = n0 + 64 * wn + 32 * a + 8 * q + 4 * lh;
          if (col >= N) continue;
          f32x4_t v;
          if (g.splits > 1) {
            // partial sums of G and U, [G | U] per row, combined by the finalize pass
            f32x4_t gv, uv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              gv[r] = acc[a][b][4 * q + r];
              uv[r] = acc[a + 2][b][4 * q + r];
            }
            *reinterpret_cast<f32x4_t *>(crow + col) = gv;
            *reinterpret_cast<f32x4_t *>(crow + N + col) = uv;
            continue;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = situ_glu(acc[a][b][4 * q + r], acc[a + 2][b][4 * q + r], g.beta, g.beta_lin);
          if (g.c_hi != nullptr) {
            // bf16 planes for the next GEMM's operands (whole K, no accumulate: host-checked)
            const long long o = (long long)t * ldc + col;
            bf16x4_t h, l;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              __bf16 vh, vl;
              split_bf16(v[r], vh, vl);
              h[r] = vh;
              l[r] = vl;
            }
            *reinterpret_cast<bf16x4_t *>(g.c_hi + o) = h;
            if (g.c_lo != nullptr) *reinterpret_cast<bf16x4_t *>(g.c_lo + o) = l;
            continue;
          }
          if (acc_in) v += *reinterpret_cast<const f32x4_t *>(crow + col);
          *reinterpret_cast<f32x4_t *>(crow + col) = v;
        }
      } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = n0 + 128 * wn + 32 * a + 8 * q + 4 * lh;
          if (col >= N) continue;
          if (vec_ok && col + 3 < N) {
            f32x4_t v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[a][b][4 * q + r];
            if (acc_in) v += *reinterpret_cast<const f32x4_t *>(crow + col);
            *reinterpret_cast<f32x4_t *>(crow + col) = v;
          } else {
            // the last group of a row whose length is not a multiple of 4 (the
            // router at an expert count that is not), or rows not 16-byte aligned
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (col + r < N) crow[col + r] = acc_in ? crow[col + r] + acc[a][b][4 * q + r] : acc[a][b][4 * q + r];
          }
        }
      }
    }
  }
}

template <int NPL, bool PAIR>
__global__ __launch_bounds__(64 * DNW, 1) void dense_tile_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[dense_stages(NPL) * dense_stage_bytes(NPL)];
  dense_tile_body<NPL, PAIR>(g, ring);
}

// fp32 activations -> bf16 planes: hi = bf16(a) and lo = bf16(a - hi), or
// only the rounded plane; 8 values per thread
__global__ __launch_bounds__(256) void split_planes_kernel(const float *__restrict__ A, long long lda, int rows,
                                                           int K, __bf16 *__restrict__ hi, __bf16 *__restrict__ lo) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = K / 8;
  if (i >= (long long)rows * per_row) return;
  const long long row = i / per_row;
  const int c = (int)(i - row * per_row);
  const f32x4_t *src = reinterpret_cast<const f32x4_t *>(A + row * lda + c * 8);
  const f32x4_t x0 = src[0], x1 = src[1];
  bf16x8_t h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = e < 4 ? x0[e] : x1[e - 4];
    __bf16 vh, vl;
    split_bf16(v, vh, vl);
    h[e] = vh;
    l[e] = vl;
  }
  *reinterpret_cast<bf16x8_t *>(hi + row * K + c * 8) = h;
  if (lo != nullptr) *reinterpret_cast<bf16x8_t *>(lo + row * K + c * 8) = l;
}

}  // namespace

int dense_tile_cols(bool pair) { return pair ? DT / 2 : DT; }
int dense_tile_rows() { return DT; }

hipError_t launch_dense_tile(int nplanes, bool pair, const GemmArgs &a, hipStream_t st) {
  const long long grid = (long long)a.n_blocks * a.dense_rows_tiles * a.splits;
  const dim3 gr((unsigned)((grid + 7) & ~7LL)), blk(64 * DNW);
  if (nplanes == 2) {
    if (pair) hipLaunchKernelGGL((dense_tile_kernel<2, true>), gr, blk, 0, st, a);
    else hipLaunchKernelGGL((dense_tile_kernel<2, false>), gr, blk, 0, st, a);
  } else {
    if (pair) hipLaunchKernelGGL((dense_tile_kernel<1, true>), gr, blk, 0, st, a);
    else hipLaunchKernelGGL((dense_tile_kernel<1, false>), gr, blk, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_split_planes(const float *A, long long lda, int rows, int K, uint16_t *hi, uint16_t *lo,
                               hipStream_t st) {
  const long long n = (long long)rows * (K / 8);
  hipLaunchKernelGGL(split_planes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A, lda, rows, K,
                     reinterpret_cast<__bf16 *>(hi), reinterpret_cast<__bf16 *>(lo));
  return hipGetLastError();
}

}  // namespace moe
