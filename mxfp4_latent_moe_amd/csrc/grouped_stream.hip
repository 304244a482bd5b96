// Persistent streaming MXFP4 grouped GEMM for decode-sized expert segments.
//
// Work item = (row chunk of <= R sorted rows of one expert, block of weight
// rows); R = 4 at decode sizes, 8 for the small experts of a batch whose
// larger experts run on the tiled kernel.  The grid holds one resident wave of work-groups; work-group
// w takes the contiguous item range [w*n/G, (w+1)*n/G) of the n items that
// exist on the device (n is read from the chunk list, so nothing waits on the
// host).  Within a work-group the weight stream never stops: every wave walks
// the K steps of its rows item after item.  Weights are requested a group of
// four K steps at a time (256 contiguous bytes per row in one burst, which
// keeps DRAM pages open), two groups ahead of the MFMAs, across item
// boundaries.  The token rows of the current chunk (bf16, or bf16 hi + lo) sit
// in LDS; they are restaged only when the chunk changes.
//
// Per K step (128 K values) a lane holds one 16-byte slice of one weight row
// (32 e2m1 codes = one scale group), converted in registers with the scaled
// fp4 -> bf16 instruction and fed to MFMA 16x16x32 bf16 as the M side; the
// tokens are the N side.  Scales are read 16 bytes at a time (four K steps of
// one row); the kernel takes rows whose K steps come in groups of four.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KSTEP = 128;
constexpr int KSMAX = STREAM_GROUPED_KSMAX;

template <int AF, bool PAIR, int MT, int AHEAD, int NW, int R>
__global__ __launch_bounds__(64 * NW) void grouped_stream_kernel(GemmArgs g) {
  constexpr int D = 4;  // K steps per group: one 16-byte read of scales covers four steps
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int NTHR = 64 * NW;
  constexpr int ROWS_WG = 16 * NW * MT;
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;
  constexpr int STEP = 16 * R * 8;  // bf16 elements per K step per plane: [octet][row][8]
  constexpr bool FOLD = NPL == 2 && 2 * R <= 16;
  __shared__ __attribute__((aligned(16))) __bf16 lds[NPL][KSMAX * STEP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;
  const uint32_t row_bytes = K / 2;
  const uint32_t srow_bytes = K / 32;

  const int n_items = *g.chunk_count * g.n_blocks;
  const int G = gridDim.x;
  const int i_begin = (int)((long long)blockIdx.x * n_items / G);
  const int i_end = (int)((long long)(blockIdx.x + 1) * n_items / G);
  if (i_begin >= i_end) return;
  // the chunk list is read-only here: reading it through the constant address
  // space with wave-uniform indices keeps those reads on the scalar unit, off
  // the vector memory counter that paces the weight ring
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32 *chunks = (const_i32 *)(g.chunks);  // {expert, row0, nrows, 0} per chunk

  // ---- load cursor: item and K step of the next weight load
  int l_item = i_begin, l_q = 0;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
  uint32_t woff[NTILE], soff[NTILE];
  auto set_load_item = [&](int it) {
    const int c = __builtin_amdgcn_readfirstlane(it / g.n_blocks);
    const int nb = it - c * g.n_blocks;
    const int expert = chunks[4 * c];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
      const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0) + expert * g.w_estride;
      const uint8_t *S = (mat ? g.S1 : g.S0) + expert * g.s_estride;
      wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
      sr[mat] = make_rsrc(S, (uint32_t)N * srow_bytes);
    }
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const int n = min(nb * ROWS_WG + wave * 16 * MT + (t % MT) * 16 + r16, N - 1);
      woff[t] = (uint32_t)n * row_bytes + kg * 16;
      soff[t] = (uint32_t)n * srow_bytes;
    }
  };
  set_load_item(i_begin);

  // wq[0] / scg[0]: the group being computed; [1..AHEAD]: groups requested ahead
  u32x4_t wq[AHEAD + 1][D][NTILE];
  u32x4_t scg[AHEAD + 1][NTILE];
  // Request one whole group -- D consecutive K steps of every tile, one burst
  // of 4 x 64 contiguous bytes per weight row, then its 16 scale bytes -- into
  // slot `bi` and advance the cursor.  Past the last item the requests are
  // kept (so the memory counter pattern stays fixed) but all lanes read one
  // 16-byte line.
  auto load_group = [&](int bi) {
    const bool live = l_item < i_end;
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int t = 0; t < NTILE; ++t)
        wq[bi][d][t] = buf_load16(wr[t / MT], live ? woff[t] : 0u, live ? (uint32_t)(l_q + d) * 64u : 0u);
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
      scg[bi][t] = buf_load16(sr[t / MT], live ? soff[t] : 0u, live ? (uint32_t)l_q * 4u : 0u);
    l_q += D;
    if (l_q == nks) {
      l_q = 0;
      if (++l_item < i_end) set_load_item(l_item);
    }
  };

  // ---- compute cursor
  int c_item = i_begin, c_q = 0;
  int staged_chunk = -1;
  int row0 = 0, nrows = 0, c_nb = 0;

  auto stage = [&](int c) {
    c = __builtin_amdgcn_readfirstlane(c);
    row0 = chunks[4 * c + 1];
    nrows = chunks[4 * c + 2];
    if (c == staged_chunk) return;
    __syncthreads();  // every wave is done with the previous chunk's rows
    constexpr int SG = 2;
    const int esz = (AF == A_BF16) ? 2 : 4;
    const int ngrp = R * nks * 16;
    for (int i0 = tid; i0 < ngrp; i0 += NTHR * SG) {
      u32x4_t araw[SG][(AF == A_BF16) ? 1 : 2];
      int aoff[SG];
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        const int gi = i0 + NTHR * ii;
        const int r = gi % R;
        const int oct = (gi / R) & 15;
        const int q = gi / (16 * R);
        aoff[ii] = (gi < ngrp) ? q * STEP + (oct * R + r) * 8 : -1;
        araw[ii][0] = u32x4_t{0, 0, 0, 0};
        if constexpr (AF != A_BF16) araw[ii][1] = u32x4_t{0, 0, 0, 0};
        if (gi < ngrp && r < nrows) {
          const int p = row0 + r;
          const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
          const char *src = static_cast<const char *>(g.A) + (arow * g.lda + (long long)q * KSTEP + oct * 8) * esz;
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
    __syncthreads();
    staged_chunk = c;
  };

  f32x4_t acc[NTILE], accl[NTILE];
  auto reset_acc = [&]() {
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accl[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  auto begin_item = [&]() {
    const int c = c_item / g.n_blocks;
    c_nb = c_item - c * g.n_blocks;
    stage(c);
    reset_acc();
  };

  auto finish_item = [&]() {
    // hi + lo per output: the lo column R lanes up (folded), or the second accumulator
    f32x4_t af[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      af[t] = acc[t];
      if constexpr (FOLD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) af[t][r] += __shfl_down(af[t][r], R, 64);
      } else if constexpr (NPL == 2) {
        af[t] += accl[t];
      }
    }
    const int tok = r16;
    if (tok < nrows) {
      const long long orow = row0 + tok;
      const int wrow_base = c_nb * ROWS_WG + wave * 16 * MT;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int col0 = wrow_base + m * 16 + 4 * kg;
        const f32x4_t a = af[m];
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (PAIR) {
            const f32x4_t u = af[m + MT];
            v[r] = situ_glu(a[r], u[r], g.beta, g.beta_lin);
          } else {
            v[r] = a[r];
          }
        }
        if (g.rscale != nullptr) {
          const float rs = g.rscale[g.rscale_map ? g.rscale_map[orow] : orow];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] *= rs;
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
  };

  // Lanes whose token column is >= R read row (r16 % R): those MFMA output
  // columns are never stored.  With two activation planes and at most eight
  // rows, one MFMA takes both planes (FOLD): columns 0..R-1 read the rows' hi
  // plane, R..2R-1 their lo plane, and the epilogue adds column r + R to
  // column r, the same two fp32 sums added as with a second accumulator, at
  // half the MFMAs and B reads.
  const int brow = r16 % R;
  const __bf16 *const bsrc = &lds[FOLD ? (r16 / R) & 1 : 0][0];
  // one K step from group slot 0
  auto compute = [&](int d, int q) {
    float scl[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const uint32_t sw = scg[0][t][d];  // the scale dword of K step q
      scl[t] = e8m0_to_float((sw >> (8 * kg)) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = q * STEP + ((4 * kg + j) * R + brow) * 8;
      const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&bsrc[off]);
      bf16x8_t bl;
      if constexpr (NPL == 2 && !FOLD) bl = *reinterpret_cast<const bf16x8_t *>(&lds[1][off]);
      bf16x8_t wa[NTILE];
#pragma unroll
      for (int t = 0; t < NTILE; ++t) wa[t] = fp4x8_to_bf16(wq[0][d][t][j], scl[t]);
#pragma unroll
      for (int t = 0; t < NTILE; ++t) acc[t] = mfma_16x16x32(wa[t], bh, acc[t]);
      if constexpr (NPL == 2 && !FOLD) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) accl[t] = mfma_16x16x32(wa[t], bl, accl[t]);
      }
    }
  };

  // ---- prologue: groups 1..AHEAD are requested before the first staging
#pragma unroll
  for (int i = 1; i <= AHEAD; ++i) load_group(i);
  __builtin_amdgcn_s_waitcnt(0);

  // nks is a multiple of D (host guarantee): items are whole groups
  for (; c_item < i_end; ++c_item) {
    begin_item();
    for (c_q = 0; c_q < nks; c_q += D) {
      // the oldest requested group becomes the computed one (static indices)
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) {
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
          for (int t = 0; t < NTILE; ++t) wq[i][d][t] = wq[i + 1][d][t];
#pragma unroll
        for (int t = 0; t < NTILE; ++t) scg[i][t] = scg[i + 1][t];
      }
      load_group(AHEAD);  // one burst for the group AHEAD groups ahead
#pragma unroll
      for (int d = 0; d < D; ++d) compute(d, c_q + d);
    }
    finish_item();
  }
}

// Affine 2-bit weights (w = s q + b per 64-element group), the same
// persistent weight stream as grouped_stream_kernel (kept a kernel of its own
// so that the MXFP4 kernel's code generation stays as tuned).  The codes enter
// the MFMA as exact integers q (aff2x8_to_bf16), laid out so that each MFMA
// instruction stays inside one group (aff2_octet): a lane loads two dwords of
// codes per K step, one per group.  The two instructions of a group sum into
// a temporary accumulator, which is added to the result times the group's
// scale of each output row (the four rows' scale dwords come from the lanes
// that loaded them).  The bias part sum_g b_g sum_{k in g} a_k is one more
// product per item: the biases of the lane's row (8 groups per lane, the M
// side) against the per-group sums of the staged activation rows (hi + lo,
// the N side).  Activations are staged in the convert's element order.  The
// biases of an item are requested with its first weight group, into one of
// two slots by item parity: the load cursor runs at most one item ahead when
// an item has more than AHEAD groups of K steps (K >= 1536, checked by the
// caller).
template <int AF, bool PAIR, int MT, int AHEAD, int NW>
__global__ __launch_bounds__(64 * NW) void grouped_stream_aff_kernel(GemmArgs g) {
  constexpr int R = PERSIST_ROWS;
  constexpr int D = 4;  // K steps per group: one 16-byte read of scales covers four steps
  constexpr int NMAT = PAIR ? 2 : 1;
  constexpr int NTILE = NMAT * MT;
  constexpr int NTHR = 64 * NW;
  constexpr int ROWS_WG = 16 * NW * MT;
  constexpr int NPL = (AF == A_F32_SPLIT) ? 2 : 1;
  constexpr int STEP = 16 * R * 8;     // bf16 elements per K step per plane: [octet][row][8]
  constexpr int SUMS = 2 * 4 * R * 8;  // per-group activation sums: [slice][octet][row][8] (64 groups)
  constexpr uint32_t STEP_BYTES = 32;  // codes of one row per K step
  // hi and lo planes in one MFMA (columns R..2R-1 take the lo plane), as in
  // grouped_stream_kernel; the bias part folds the group sums' hi and lo alike
  constexpr bool FOLD = NPL == 2 && 2 * R <= 16;
  __shared__ __attribute__((aligned(16))) __bf16 lds[NPL][KSMAX * STEP];
  __shared__ __attribute__((aligned(16))) __bf16 sums[2][SUMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int r16 = lane & 15;
  const int N = g.N, K = g.K;
  const int nks = K / KSTEP;
  const int ngroups = K / 64;
  const uint32_t row_bytes = K / 4;
  const uint32_t srow_bytes = ngroups * 2;  // bf16 scales (or biases) of a row

  const int n_items = *g.chunk_count * g.n_blocks;
  const int G = gridDim.x;
  const int i_begin = (int)((long long)blockIdx.x * n_items / G);
  const int i_end = (int)((long long)(blockIdx.x + 1) * n_items / G);
  if (i_begin >= i_end) return;
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32 *chunks = (const_i32 *)(g.chunks);  // {expert, row0, nrows, 0} per chunk

  // ---- load cursor: item and K step of the next weight load
  int l_item = i_begin, l_q = 0;
  __amdgpu_buffer_rsrc_t wr[NMAT], sr[NMAT];
  uint32_t woff[NTILE], soff[NTILE];
  u32x4_t bq[2][NTILE][2];  // biases of groups 8 kg + 32 i of the lane's row, per item parity
  auto set_load_item = [&](int it) {
    const int c = __builtin_amdgcn_readfirstlane(it / g.n_blocks);
    const int nb = it - c * g.n_blocks;
    const int expert = chunks[4 * c];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
      const uint8_t *W = static_cast<const uint8_t *>(mat ? g.W1 : g.W0) + expert * g.w_estride;
      const uint8_t *S = (mat ? g.S1 : g.S0) + expert * g.s_estride;
      wr[mat] = make_rsrc(W, (uint32_t)N * row_bytes);
      sr[mat] = make_rsrc(S, (uint32_t)N * srow_bytes);
    }
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const int n = min(nb * ROWS_WG + wave * 16 * MT + (t % MT) * 16 + r16, N - 1);
      woff[t] = (uint32_t)n * row_bytes + kg * 4;
      soff[t] = (uint32_t)n * srow_bytes;
    }
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const __amdgpu_buffer_rsrc_t br =
          make_rsrc((t / MT ? g.B1 : g.B0) + expert * (g.s_estride / 2), (uint32_t)N * srow_bytes);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int g0 = 8 * kg + 32 * i;
        bq[it & 1][t][i] = g0 < ngroups ? buf_load16(br, soff[t] + 2 * g0, 0) : u32x4_t{0, 0, 0, 0};
      }
    }
  };
  set_load_item(i_begin);

  // wq[0] / scg[0]: the group being computed; [1..AHEAD]: groups requested ahead
  u32x2_t wq[AHEAD + 1][D][NTILE];
  u32x4_t scg[AHEAD + 1][NTILE];
  // one group of D K steps: per step and tile the lane's dwords kg (group 0)
  // and 4 + kg (group 1) of the row's codes, then the 16 scale bytes of the
  // D steps; past the last item all lanes re-read one line
  auto load_group = [&](int bi) {
    const bool live = l_item < i_end;
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        const uint32_t vo = live ? woff[t] : 0u, so = live ? (uint32_t)(l_q + d) * STEP_BYTES : 0u;
        wq[bi][d][t] = u32x2_t{buf_load4(wr[t / MT], vo, so), buf_load4(wr[t / MT], vo + 16u, so)};
      }
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
      scg[bi][t] = buf_load16(sr[t / MT], live ? soff[t] : 0u, live ? (uint32_t)l_q * 4u : 0u);
    l_q += D;
    if (l_q == nks) {
      l_q = 0;
      if (++l_item < i_end) set_load_item(l_item);
    }
  };

  // ---- compute cursor
  int c_item = i_begin, c_q = 0;
  int staged_chunk = -1;
  int row0 = 0, nrows = 0, c_nb = 0;

  // the chunk's rows in LDS (bf16, or hi + lo), each octet in the convert's
  // element order, then their per-group sums as bf16 hi + lo in the layout of
  // an N-side operand: group 32 i + 8 o + e of row r at [i][o][r][e]
  auto stage = [&](int c) {
    c = __builtin_amdgcn_readfirstlane(c);
    row0 = chunks[4 * c + 1];
    nrows = chunks[4 * c + 2];
    if (c == staged_chunk) return;
    __syncthreads();  // every wave is done with the previous chunk's rows
    constexpr int SG = 2;
    const int esz = (AF == A_BF16) ? 2 : 4;
    const int ngrp = R * nks * 16;
    for (int i0 = tid; i0 < ngrp; i0 += NTHR * SG) {
      u32x4_t araw[SG][(AF == A_BF16) ? 1 : 2];
      int aoff[SG];
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        const int gi = i0 + NTHR * ii;
        const int r = gi % R;
        const int oct = (gi / R) & 15;
        const int q = gi / (16 * R);
        aoff[ii] = (gi < ngrp) ? q * STEP + (oct * R + r) * 8 : -1;
        araw[ii][0] = u32x4_t{0, 0, 0, 0};
        if constexpr (AF != A_BF16) araw[ii][1] = u32x4_t{0, 0, 0, 0};
        if (gi < ngrp && r < nrows) {
          const int p = row0 + r;
          const long long arow = g.a_map ? (long long)(g.a_map[p] / g.a_div) : (long long)p;
          const char *src = static_cast<const char *>(g.A) + (arow * g.lda + (long long)q * KSTEP + oct * 8) * esz;
          araw[ii][0] = reinterpret_cast<const u32x4_t *>(src)[0];
          if constexpr (AF != A_BF16) araw[ii][1] = reinterpret_cast<const u32x4_t *>(src)[1];
        }
      }
#pragma unroll
      for (int ii = 0; ii < SG; ++ii) {
        if (aoff[ii] < 0) continue;
        if constexpr (AF == A_BF16) {
          u32x4_t v = araw[ii][0];
#pragma unroll
          for (int h = 0; h < 4; h += 2) {  // bf16 elements 0..7 -> 0, 2, 1, 3, 4, 6, 5, 7
            const uint32_t a = v[h], b = v[h + 1];
            v[h] = (a & 0xFFFFu) | (b << 16);
            v[h + 1] = (a >> 16) | (b & 0xFFFF0000u);
          }
          *reinterpret_cast<u32x4_t *>(&lds[0][aoff[ii]]) = v;
        } else {
          bf16x8_t hi, lo;
#pragma unroll
          for (int e0 = 0; e0 < 8; ++e0) {
            const int e = aff2_perm(e0);  // slot e0 holds element e
            const float f = __uint_as_float(e < 4 ? araw[ii][0][e] : araw[ii][1][e - 4]);
            if constexpr (AF == A_F32_SPLIT) {
              __bf16 h, l;
              split_bf16(f, h, l);
              hi[e0] = h;
              lo[e0] = l;
            } else {
              hi[e0] = to_bf16(f);
            }
          }
          *reinterpret_cast<bf16x8_t *>(&lds[0][aoff[ii]]) = hi;
          if constexpr (NPL == 2) *reinterpret_cast<bf16x8_t *>(&lds[NPL - 1][aoff[ii]]) = lo;
        }
      }
    }
    __syncthreads();
    for (int gi = tid; gi < 64 * R; gi += NTHR) {
      const int grp = gi / R, r = gi - grp * R;
      float sum = 0.f;
      if (grp < ngroups) {
        const int q = grp >> 1, o0 = 8 * (grp & 1);
#pragma unroll
        for (int o = 0; o < 8; ++o) {
          const int off = q * STEP + ((o0 + o) * R + r) * 8;
#pragma unroll
          for (int p = 0; p < NPL; ++p) {
            const bf16x8_t v = *reinterpret_cast<const bf16x8_t *>(&lds[p][off]);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += from_bf16(v[e]);
          }
        }
      }
      __bf16 h, l;
      split_bf16(sum, h, l);
      const int so = (((grp >> 5) * 4 + ((grp >> 3) & 3)) * R + r) * 8 + (grp & 7);
      sums[0][so] = h;
      sums[1][so] = l;
    }
    __syncthreads();
    staged_chunk = c;
  };

  f32x4_t acc[NTILE], accl[NTILE];
  auto begin_item = [&]() {
    const int c = c_item / g.n_blocks;
    c_nb = c_item - c * g.n_blocks;
    stage(c);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accl[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Lanes whose token column is >= R read row (r16 % R): those MFMA output
  // columns are never stored.
  const int brow = r16 % R;
  const int bpl = FOLD ? (r16 / R) & 1 : 0;
  const __bf16 *const bsrc = &lds[bpl][0];
  auto finish_item = [&]() {
    // the bias part: biases of the lane's row against the staged rows' group sums
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int off = ((i * 4 + kg) * R + brow) * 8;
      const bf16x8_t sh = *reinterpret_cast<const bf16x8_t *>(&sums[bpl][off]);
      bf16x8_t sl;
      if constexpr (!FOLD) sl = *reinterpret_cast<const bf16x8_t *>(&sums[1][off]);
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, bq[c_item & 1][t][i]);
        acc[t] = mfma_16x16x32(bw, sh, acc[t]);
        if constexpr (!FOLD) accl[t] = mfma_16x16x32(bw, sl, accl[t]);
      }
    }
    // hi + lo per output: the lo column R lanes up (folded), or the second accumulator
    f32x4_t af[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      af[t] = acc[t];
      if constexpr (FOLD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) af[t][r] += __shfl_down(af[t][r], R, 64);
      } else {
        af[t] += accl[t];
      }
    }
    const int tok = r16;
    if (tok < nrows) {
      const long long orow = row0 + tok;
      const int wrow_base = c_nb * ROWS_WG + wave * 16 * MT;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int col0 = wrow_base + m * 16 + 4 * kg;
        const f32x4_t a = af[m];
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (PAIR) {
            const f32x4_t u = af[m + MT];
            v[r] = situ_glu(a[r], u[r], g.beta, g.beta_lin);
          } else {
            v[r] = a[r];
          }
        }
        if (g.rscale != nullptr) {
          const float rs = g.rscale[g.rscale_map ? g.rscale_map[orow] : orow];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] *= rs;
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
  };

  // one K step from group slot 0, group by group
  auto compute = [&](int d, int q) {
    // scale dwords (groups 2q, 2q+1) of the lane's output rows 4 kg + r, from
    // the lanes that loaded those rows
    float sc[NTILE][2][4];
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t sw = (uint32_t)__shfl((int)scg[0][t][d], 4 * kg + r, 64);
        sc[t][0][r] = bf16_lo_to_float(sw);
        sc[t][1][r] = bf16_lo_to_float(sw >> 16);
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t ym[NTILE], zm[NTILE];
      f32x4_t tmp[NTILE];
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        ym[t] = wq[0][d][t][h] & 0x33333333u;
        zm[t] = (wq[0][d][t][h] >> 2) & 0x33333333u;
        tmp[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int off = q * STEP + (aff2_octet(h, kg, jj) * R + brow) * 8;
        const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&bsrc[off]);
        bf16x8_t bl;
        if constexpr (NPL == 2 && !FOLD) bl = *reinterpret_cast<const bf16x8_t *>(&lds[1][off]);
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
          const bf16x8_t wa = jj ? aff2x8_to_bf16<2>(ym[t], zm[t]) : aff2x8_to_bf16<0>(ym[t], zm[t]);
          tmp[t] = mfma_16x16x32(wa, bh, tmp[t]);
          if constexpr (NPL == 2 && !FOLD) tmp[t] = mfma_16x16x32(wa, bl, tmp[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < NTILE; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(sc[t][h][r], tmp[t][r], acc[t][r]);
    }
  };

  // ---- prologue: groups 1..AHEAD are requested before the first staging
#pragma unroll
  for (int i = 1; i <= AHEAD; ++i) load_group(i);
  __builtin_amdgcn_s_waitcnt(0);

  for (; c_item < i_end; ++c_item) {
    begin_item();
    for (c_q = 0; c_q < nks; c_q += D) {
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) {
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
          for (int t = 0; t < NTILE; ++t) wq[i][d][t] = wq[i + 1][d][t];
#pragma unroll
        for (int t = 0; t < NTILE; ++t) scg[i][t] = scg[i + 1][t];
      }
      load_group(AHEAD);
#pragma unroll
      for (int d = 0; d < D; ++d) compute(d, c_q + d);
    }
    finish_item();
  }
}

// One 16-row tile per wave and matrix, two groups in flight; gate/up (two
// matrices per wave) runs eight waves per work-group.  Down runs four waves on
// chunks of PERSIST_ROWS rows and eight on chunks of PERSIST_ROWS_WIDE rows,
// whose activation planes leave room for one work-group per CU: eight waves
// keep twice the weight bytes in flight there (batched decode at T = 256:
// 3.07 -> 2.90 ms a step).
constexpr int gs_waves(bool pair, int rows) { return pair ? 8 : rows == PERSIST_ROWS_WIDE ? 8 : 4; }

template <int AF, bool PAIR, int R>
void *kernel_ptr() {
  return reinterpret_cast<void *>(&grouped_stream_kernel<AF, PAIR, 1, 2, gs_waves(PAIR, R), R>);
}
template <int AF, bool PAIR>
void *aff_kernel_ptr() {
  return reinterpret_cast<void *>(&grouped_stream_aff_kernel<AF, PAIR, 1, 2, gs_waves(PAIR, PERSIST_ROWS)>);
}

template <int R>
void *select_mxfp4(int afmt, bool pair) {
  switch (afmt) {
    case A_BF16: return pair ? kernel_ptr<A_BF16, true, R>() : kernel_ptr<A_BF16, false, R>();
    case A_F32_SPLIT: return pair ? kernel_ptr<A_F32_SPLIT, true, R>() : kernel_ptr<A_F32_SPLIT, false, R>();
    default: return pair ? kernel_ptr<A_F32_ROUND, true, R>() : kernel_ptr<A_F32_ROUND, false, R>();
  }
}

void *select_kernel(int wfmt, int afmt, bool pair, int rows) {
  if (wfmt == W_AFF2) {
    switch (afmt) {
      case A_BF16: return pair ? aff_kernel_ptr<A_BF16, true>() : aff_kernel_ptr<A_BF16, false>();
      case A_F32_SPLIT: return pair ? aff_kernel_ptr<A_F32_SPLIT, true>() : aff_kernel_ptr<A_F32_SPLIT, false>();
      default: return pair ? aff_kernel_ptr<A_F32_ROUND, true>() : aff_kernel_ptr<A_F32_ROUND, false>();
    }
  }
  return rows == PERSIST_ROWS ? select_mxfp4<PERSIST_ROWS>(afmt, pair) : select_mxfp4<PERSIST_ROWS_WIDE>(afmt, pair);
}

}  // namespace

int grouped_stream_rows_per_wg(bool pair, int rows) { return 16 * gs_waves(pair, rows); }

bool grouped_stream_fits(int K) {
  const int nks = K / KSTEP;
  return nks % 4 == 0 && nks <= KSMAX;
}

hipError_t launch_grouped_stream(int wfmt, int afmt, bool pair, const GemmArgs &a, hipStream_t st, int rows) {
  if (wfmt != W_MXFP4 && wfmt != W_AFF2) return hipErrorInvalidValue;
  if (rows != PERSIST_ROWS && (rows != PERSIST_ROWS_WIDE || wfmt != W_MXFP4)) return hipErrorInvalidValue;
  void *fn = select_kernel(wfmt, afmt, pair, rows);
  const int threads = 64 * gs_waves(pair, wfmt == W_AFF2 ? PERSIST_ROWS : rows);
  // one resident wave of work-groups (occupancy queried once per kernel and device)
  static std::atomic<int> cache[64][18];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const int slot = (wfmt == W_AFF2 ? 6 : rows == PERSIST_ROWS_WIDE ? 12 : 0) + afmt * 2 + (pair ? 1 : 0);
  int per_cu = cache[dev][slot].load();
  if (per_cu == 0) {
    int blocks = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, 0);
    if (e != hipSuccess) return e;
    per_cu = blocks > 0 ? blocks : 1;
    cache[dev][slot].store(per_cu);
  }
  static std::atomic<int> cus[64];
  int ncu = cus[dev].load();
  if (ncu == 0) {
    hipError_t e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus[dev].store(ncu);
  }
  const long long max_items = (long long)a.grid_logical;  // chunks bound x weight blocks
  long long grid = (long long)ncu * per_cu;
  if (grid > max_items) grid = max_items;
  if (grid < 1) grid = 1;
  GemmArgs args = a;
  void *params[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), params, 0, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
