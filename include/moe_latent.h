/* moe_latent.h -- C ABI of the MI355X (gfx950) Stable LatentMoE layer library.
 *
 * One forward pass of Kimi K3's Stable LatentMoE layer with MXFP4 routed
 * experts, split into the five calls below.  The layer is described on the
 * kimi-k3-mlx README (PipeNetwork/kimi-k3-mlx), Architecture table (MoE,
 * Stable LatentMoE, Activation and Source-format rows), and the tensor
 * layouts in the K3 open-artifact audit (llm-atlas), sections 4.3 and 6.
 *
 * Conventions shared by every call
 *  - Every tensor argument is a caller-owned DEVICE pointer, row-major with
 *    the last dimension contiguous, 16-byte aligned.  bf16 values are passed
 *    as their uint16_t bit patterns.  Weights are [out_features, in_features].
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only ENQUEUES work on `stream`: no call synchronises the host,
 *    allocates or frees memory, or keeps state between calls.  The caller
 *    keeps every buffer alive until the stream has passed the work.
 *  - `ws` is a caller-owned device workspace of at least
 *    moe_workspace_bytes(shape, fn, n) bytes; its contents are scratch.
 *    Calls enqueued on different streams must not share a workspace.
 *  - Arguments are validated before anything is enqueued: on any error code
 *    nothing has been enqueued and no output has been touched.
 *  - Preconditions on device data are documented, not checked (checking would
 *    need a host synchronisation): expert ids in [0, E); at least top_k
 *    finite biased scores per token.
 *  - Asynchronous device faults surface at the caller's next synchronisation.
 *  - Shape limits of the compiled kernels (else MOE_ENOTSUP): hidden, latent,
 *    inter and n_shared*shared_inter multiples of 128; n_experts in
 *    [top_k, 1024]; 1 <= top_k <= 32.
 */
#ifndef MOE_LATENT_H
#define MOE_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

/* return codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)     /* null required pointer, bad size or enum, misaligned pointer */
#define MOE_ENOTSUP (-2)    /* shape outside the compiled tiling, or device is not gfx950 */
#define MOE_EWORKSPACE (-3) /* ws_bytes smaller than moe_workspace_bytes() */
#define MOE_EHIP (-4)       /* a HIP launch or query failed */
#define MOE_EINTERNAL (-5)  /* unexpected host-side failure caught at the boundary */

/* operand modes for activations that are not exact bf16 values (the latent z,
   the expert hidden H, the normalised latent, the shared-expert hidden) */
#define MOE_OPND_BF16X2 0 /* a = hi + lo, two bf16 MFMAs per product (default) */
#define MOE_OPND_BF16 1   /* a rounded once to bf16 (faster, less accurate) */
/* MXFP4 expert GEMMs over prefill-sized segments take fp32 activations as
   three e4m3 terms with power-of-two scales per block of 32 (residual near
   2^-12 of the block maximum) and feed them with the raw e2m1 weights and
   their e8m0 scales to the MX-scaled MFMA; every other product is BF16X2.
   A faster mode that departs from dequantise-to-bf16 arithmetic; its error
   against the exact layer is about 1e-4 of the output rms. */
#define MOE_OPND_MX8X3 2
/* As MOE_OPND_MX8X3 with three e2m3 (OCP MX fp6) terms per block of 32
   (residual near 2^-12 of the block maximum): the MX MFMA runs fp4 x fp6 at
   the fp4 rate, twice the fp8 rate.  Same departure from dequantise-to-bf16
   arithmetic, error of the same order. */
#define MOE_OPND_MX6X3 3

/* mxfp4_grouped_gemm operations */
#define MOE_OP_GATEUP_SITU 0
#define MOE_OP_DOWN 1
#define MOE_OP_GATEUP_SITU_BF16X2 2 /* gate/up + SiTU-GLU, H written as bf16 hi + lo planes */

/* activation dtypes */
#define MOE_DT_F32 0
#define MOE_DT_BF16 1
#define MOE_DT_BF16X2 2 /* bf16 planes: row r holds hi[0..K) then lo[0..K) */

/* moe_workspace_bytes() function selectors */
#define MOE_FN_ROUTE 0
#define MOE_FN_PERMUTE 1
#define MOE_FN_GROUPED_GEMM 2
#define MOE_FN_COMBINE_NORM_UP 3
#define MOE_FN_SHARED_FFN 4
#define MOE_FN_REAP_SALIENCY 5
#define MOE_FN_COMBINE_NORM_UP_REAP 6
#define MOE_FN_GROUPED_GEMM_TWO_BANK 7

/* weight formats of an expert bank (moe_grouped_gemm_two_bank) */
#define MOE_WF_MXFP4 0   /* e2m1 codes packed [E, N, K/2] (low nibble first), e8m0 scales u8 [E, N, K/32] */
#define MOE_WF_AFFINE2 1 /* 2-bit codes packed [E, N, K/4] (element 4b+i in bits 2i..2i+1 of byte b),
                            bf16 scales and biases [E, N, K/64]: w = scale * q + bias */

typedef struct {
  int32_t hidden;       /* H: residual width (7168 for K3) */
  int32_t latent;       /* L: latent width the routed experts run in (3584) */
  int32_t n_experts;    /* E: routed experts (896) */
  int32_t top_k;        /* k: experts per token (16) */
  int32_t inter;        /* I: routed-expert intermediate width (3072) */
  int32_t n_shared;     /* S: shared experts (2) */
  int32_t shared_inter; /* Is: intermediate width of one shared expert (3072) */
  float beta;           /* SiTU-GLU gate saturation (4) */
  float beta_lin;       /* SiTU-GLU linear-branch saturation (25) */
  float rms_eps;        /* RMSNorm epsilon on the combined latent (1e-6) */
  int32_t operand_mode; /* MOE_OPND_BF16X2, MOE_OPND_BF16, MOE_OPND_MX8X3 or MOE_OPND_MX6X3 */
} moe_shape;

int moe_abi_version(void);
const char *moe_strerror(int code);

/* Workspace bytes needed by call `fn` (MOE_FN_*) for `n` rows: n = T tokens
   for route/permute/combine/shared, n = P = T*top_k pairs for the grouped
   GEMM.  Returns 0 for an invalid shape or selector. */
size_t moe_workspace_bytes(const moe_shape *shape, int fn, int n);

/* Router and latent down projection.
 * Follows: kimi-k3-mlx README, Architecture table, MoE row (sigmoid router
 * over 896 experts with the aux-loss-free e_score_correction_bias, top-16)
 * and Stable LatentMoE row (down_proj 7168 -> 3584, shared by every expert);
 * K3 open-artifact audit, section 6 (router weight [896, 7168] bf16, bias
 * [896] fp32).
 *   x         [T, H]  bf16   layer input
 *   w_router  [E, H]  bf16   (NULL: z only)
 *   bias      [E]     fp32   correction bias (selection only)
 *   w_down    [L, H]  bf16   latent down projection; NULL together with z to skip it
 * Outputs:
 *   topk_ids  [T, k]  int32  selected experts, ascending id per token
 *   topk_w    [T, k]  fp32   sigmoid(logit) of each selected expert / their sum
 *   z         [T, L]  fp32   x w_down^T (NULL to skip)
 *   gap       [T]     fp32   k-th minus (k+1)-th largest biased score (NULL to skip;
 *                            +inf when E == k)
 * Logits accumulate in fp32; biased score = fp32 sigmoid + fp32 bias; the k
 * largest win with ties to the lower index; NaN biased scores rank last.
 * With w_router NULL (and bias, topk_ids, topk_w, gap NULL) only z is
 * computed, so that the latent projection can run on another stream than the
 * routing.
 * Errors: MOE_EINVAL for T < 1, a null required pointer, or a routing call
 * missing one of w_router, bias, topk_ids, topk_w. */
int moe_route(const moe_shape *shape, int T, const uint16_t *x, const uint16_t *w_router,
              const float *bias, const uint16_t *w_down, int32_t *topk_ids, float *topk_w,
              float *z, float *gap, void *ws, size_t ws_bytes, void *stream);

/* moe_route with the moe_k_hi cap on promoted experts.
 * Follows: Kimi-K3-Alis-MLX-Dynamic card, Build recipe (experts that matter
 * stay in MXFP4, "promoted"; the serving configuration caps that path at
 * moe_k_hi = 4 promoted experts per token of the 16 routed, and the
 * contribution of a token's 5th and later promoted expert is dropped rather
 * than downgraded).
 *   promoted  [E] uint8, device: nonzero marks a promoted expert
 *   k_hi      >= 0; k_hi >= top_k leaves the routing as moe_route's
 *   the rest  as for moe_route (w_router required)
 * Routing order is the top-k's: larger biased score first, ties to the lower
 * index.  A selected promoted expert with k_hi selected promoted experts ahead
 * of it gets topk_w = 0; ids, gap and the other weights (normalised over all k
 * selected experts) are exactly moe_route's.
 * Errors: those of moe_route; MOE_EINVAL for a null promoted or w_router, or
 * k_hi < 0. */
int moe_route_capped(const moe_shape *shape, int T, const uint16_t *x, const uint16_t *w_router,
                     const float *bias, const uint16_t *w_down, const uint8_t *promoted, int k_hi,
                     int32_t *topk_ids, float *topk_w, float *z, float *gap, void *ws, size_t ws_bytes,
                     void *stream);

/* moe_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments and outputs are moe_route's, without the workspace: the call uses
 * a fixed per-device scratch array of MOE_ROUTE_NOALLOC_SCRATCH_BYTES that the
 * library holds from its first use on a device until the process ends, and it
 * calls no allocating routine.  Its first call on a device looks up that
 * device's copy of the array (a host-side query, no allocation).
 * Every call on one GPU shares the array and leaves its last contents in it
 * (nothing in it needs to start at zero): calls that overlap on one GPU (on
 * different streams, or from different threads) race and must not be made.
 * Size limit: moe_workspace_bytes(shape, MOE_FN_ROUTE, T) must not exceed
 * MOE_ROUTE_NOALLOC_SCRATCH_BYTES (at K3 shapes: T <= 64, the decode sizes).
 * Errors: those of moe_route; MOE_EWORKSPACE when T needs more scratch than
 * the array holds. */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int moe_route_noalloc(const moe_shape *shape, int T, const uint16_t *x, const uint16_t *w_router,
                      const float *bias, const uint16_t *w_down, int32_t *topk_ids, float *topk_w,
                      float *z, float *gap, void *stream);

/* Token permutation: stable counting sort of the pairs p = t*k + j by expert.
 * Follows: kimi-k3-mlx README, REAP section, two-bank paragraph (pairs sorted
 * by expert index give each expert a contiguous slice).
 *   topk_ids        [T, k]  int32 (ascending per token, each id in [0, E))
 * Outputs:
 *   expert_offsets  [E+1]   int32  expert e owns sorted rows offsets[e]..offsets[e+1]
 *   sorted_pair     [T*k]   int32  pair index at each sorted row (tokens ascend in a slice)
 *   pair_pos        [T*k]   int32  sorted row of each pair (inverse of sorted_pair)
 *   active          [E+1]   int32  active[0] = number of experts with pairs,
 *                                  active[1..] = their ids ascending (NULL to skip)
 * Deterministic: no result depends on the order of concurrent updates. */
int moe_permute(const moe_shape *shape, int T, const int32_t *topk_ids, int32_t *expert_offsets,
                int32_t *sorted_pair, int32_t *pair_pos, int32_t *active, void *ws,
                size_t ws_bytes, void *stream);

/* MXFP4 grouped expert GEMM over expert-sorted rows.
 * Follows: K3 open-artifact audit, section 4.3 (w1/w3 weight_packed u8
 * [3072, 1792] and weight_scale u8 [3072, 112]; w2 packed [3584, 1536],
 * scale [3584, 96]); kimi-k3-mlx README, Architecture table Source-format row
 * and Tiers section (e2m1 codes low nibble first, e8m0 scales, group 32),
 * Activation row and Porting notes item 1 (SiTU-GLU in fp32).
 * Weight tensors are the checkpoint bytes as-is, stacked over experts:
 * packed [E, N, K/2] (byte b of a row holds element 2b in its low nibble),
 * scale [E, N, K/32] (element k of row n is code * 2^(scale[n][k/32]-127)).
 * e8m0 range: for scale bytes 2..252 every weight is exact in the kernels
 * (bf16 and MX paths alike), as the OCP MX definition gives it.  Outside that
 * range the result is unspecified but the call stays memory-safe: bytes 0 and
 * 1 give values below 2^-126 that the bf16 path may flush to zero, bytes 253
 * and 254 overflow bf16 for the largest codes in the bf16 path, and 255 (NaN
 * in OCP MX) gives non-finite outputs for the rows that use it.
 *   op = MOE_OP_GATEUP_SITU: H[p] = SiTU-GLU(A_p w1_e^T, A_p w3_e^T) for every
 *        sorted row p of expert e; K = latent, N = inter.
 *        w_packed/w_scale = w1 (gate), w3_packed/w3_scale = w3 (up).
 *        A row of sorted row p: A[sorted_pair[p] / top_k] when sorted_pair is
 *        given (A = z [a_rows, L], gathered), else A[p] (A already permuted,
 *        [a_rows >= P, L]).  C = H [P, inter] fp32.
 *   op = MOE_OP_DOWN: Y[p] = A[p] w2_e^T; K = inter, N = latent.
 *        A = H [a_rows >= P, inter] fp32 in sorted order; w3_* must be NULL.
 *        pair_weight [T*k] fp32 (optional, needs sorted_pair): row p is
 *        scaled by pair_weight[sorted_pair[p]].  C = Y [P, latent] fp32.
 *   P              number of sorted rows (T*k, or an expert slice's rows)
 *   expert_offsets [E+1] device int32 from moe_permute (or a slice of it
 *                  rebased to 0)
 *   a_rows         rows of A.  Gathered A (gate/up with sorted_pair): every
 *                  sorted_pair[p] / top_k must be below a_rows (a device
 *                  precondition), which holds for a call over an expert slice
 *                  with the full token count T; a_rows * K * (4 for fp32, 2 for
 *                  bf16) must stay below 2^31.  Otherwise a_rows >= P.
 *   a_dtype        MOE_DT_F32 (split or rounded per shape->operand_mode),
 *                  MOE_DT_BF16 (exact, single MFMA) or, for MOE_OP_DOWN,
 *                  MOE_DT_BF16X2 (below)
 *   op = MOE_OP_GATEUP_SITU_BF16X2: as MOE_OP_GATEUP_SITU, with C holding H as
 *        bf16 planes instead of fp32: row p of C (uint16 bits, [P, 2 inter])
 *        is hi[0..inter) then lo[0..inter), where hi = bf16(h) and
 *        lo = bf16(h - hi) (round to nearest even) of the fp32 value h the
 *        fp32 call stores, written straight from the epilogue.  A down call
 *        with a_dtype MOE_DT_BF16X2 then reads them with no split pass: hi and
 *        lo in operand mode MOE_OPND_BF16X2, hi alone in MOE_OPND_BF16, with
 *        results bitwise those of the fp32 H call.  Both forms need the tiled
 *        path with no small-expert split (P >= 8 E with these shapes) and
 *        operand mode MOE_OPND_BF16X2 or MOE_OPND_BF16, else MOE_ENOTSUP.
 * Experts with no rows cost nothing and nothing waits on the host: the grid
 * is sized from P and each workgroup reads its work item on the device.
 * Errors: MOE_EINVAL for bad op/dtype (MOE_DT_BF16X2 with a gate/up op), P < 1,
 * a_rows < 1 (or below P when A is not gathered), null required pointers, or
 * w3 given for MOE_OP_DOWN; MOE_ENOTSUP for a gathered A of 2^31 bytes or
 * more, and for the bf16-plane forms outside their limits. */
int mxfp4_grouped_gemm(const moe_shape *shape, int op, int P, const int32_t *expert_offsets,
                       const int32_t *sorted_pair, const void *A, int a_rows, int a_dtype,
                       const uint8_t *w_packed, const uint8_t *w_scale, const uint8_t *w3_packed,
                       const uint8_t *w3_scale, const float *pair_weight, float *C, void *ws,
                       size_t ws_bytes, void *stream);

/* One bank of expert weights for moe_grouped_gemm_two_bank.  All pointers are
 * device pointers; tensors are stacked over the bank's experts, its first
 * expert at index 0.  MXFP4 banks: packed/scale as for mxfp4_grouped_gemm,
 * bias NULL.  AFFINE2 banks: packed u8, scale and bias bf16 bits, all 16-byte
 * aligned.  packed/scale/bias hold w1 (gate) for MOE_OP_GATEUP_SITU and w2
 * (down) for MOE_OP_DOWN; packed3/scale3/bias3 hold w3 (up) for
 * MOE_OP_GATEUP_SITU and are NULL for MOE_OP_DOWN. */
typedef struct {
  int32_t format;    /* MOE_WF_MXFP4 or MOE_WF_AFFINE2 */
  int32_t n_experts; /* experts in the bank (may be 0) */
  const uint8_t *packed;
  const void *scale;
  const uint16_t *bias;
  const uint8_t *packed3;
  const void *scale3;
  const uint16_t *bias3;
} moe_expert_bank;

/* Grouped expert GEMM over one sorted pair list with the experts split into two
 * weight banks.
 * Follows: kimi-k3-mlx README, REAP section, graded-plan and two-bank
 * paragraphs (the graded plan keeps the most salient experts in MXFP4 and
 * stores the middle ones at a lower width; MLX holds one width per tensor, so
 * the two widths sit in two banks; once the pairs are sorted by expert index,
 * the bank that owns a contiguous range of expert indices owns a contiguous
 * slice of the sorted rows, so each bank computes only its own rows; the
 * split point depends on the routing), and Tiers section (the 2-bit affine
 * tier: 2.50 bits per weight).
 * Bank A owns experts 0 .. bank_a->n_experts - 1, bank B the rest
 * (bank_a->n_experts + bank_b->n_experts == shape->n_experts).  The split point
 * of the sorted rows, expert_offsets[bank_a->n_experts], is read on the device:
 * no call waits on the host.  Every other argument, and the result, are as for
 * mxfp4_grouped_gemm: with both banks in one format holding the same experts,
 * H and Y equal mxfp4_grouped_gemm's bit for bit.
 * Affine weights: the codes enter the bf16 MFMA as exact integers q, each
 * 64-element group's fp32 partial sum is multiplied by that group's scale, and
 * the bias part enters as the biases times the per-group sums of the
 * activations in bf16 hi + lo.
 * Limits (else MOE_ENOTSUP): operand modes BF16X2 and BF16 only; with an
 * affine bank, K (latent for gate/up, inter for down) a multiple of 512 and at
 * most 4096, and at decode-sized segments (P < 2 E) K >= 1536.
 * Workspace: moe_workspace_bytes(shape, MOE_FN_GROUPED_GEMM_TWO_BANK, P).
 * Errors: those of mxfp4_grouped_gemm; MOE_EINVAL for a null bank, an unknown
 * format, expert counts that do not add up to n_experts, a missing or extra
 * tensor for the format and op, or a misaligned tensor. */
int moe_grouped_gemm_two_bank(const moe_shape *shape, int op, int P, const int32_t *expert_offsets,
                              const int32_t *sorted_pair, const void *A, int a_rows, int a_dtype,
                              const moe_expert_bank *bank_a, const moe_expert_bank *bank_b,
                              const float *pair_weight, float *C, void *ws, size_t ws_bytes, void *stream);

/* Weighted combine, RMSNorm on the combined latent, up projection.
 * Follows: kimi-k3-mlx README, REAP section caveat paragraph (RMSNorm is
 * applied to the combined expert output before up_proj) and Architecture
 * table, Stable LatentMoE row (up_proj 3584 -> 7168).
 *   Y        [T*k, L] fp32  expert outputs in sorted order (from MOE_OP_DOWN)
 *   pair_pos [T*k]    int32 sorted row of each pair (from moe_permute)
 *   topk_w   [T, k]   fp32  routing weights, or NULL when already folded into Y
 *   gamma    [L]      bf16  RMSNorm weight
 *   w_up     [H, L]   bf16
 *   out      [T, H]   fp32  written (accumulate = 0) or added to (accumulate = 1)
 * y_t = sum_j w_{t,j} Y[pair_pos[t*k+j]] in fixed j order;
 * out_t (+)= (y_t / sqrt(mean(y_t^2) + rms_eps) * gamma) w_up^T. */
int moe_combine_norm_up(const moe_shape *shape, int T, const float *Y, const int32_t *pair_pos,
                        const float *topk_w, const uint16_t *gamma, const uint16_t *w_up,
                        float *out, int accumulate, void *ws, size_t ws_bytes, void *stream);

/* Shared experts on the residual input, run as one SiTU-GLU of width
 * S*Is (gate and up rows concatenated over experts, down columns likewise).
 * Follows: kimi-k3-mlx README, Architecture table MoE row (2 shared experts on
 * every token) and Porting notes item 3 (shared experts do not use the latent).
 *   x       [T, H]      bf16
 *   w_gate  [S*Is, H]   bf16  (expert i owns rows i*Is..(i+1)*Is)
 *   w_up    [S*Is, H]   bf16
 *   w_down  [H, S*Is]   bf16  (expert i owns columns i*Is..(i+1)*Is)
 *   out     [T, H]      fp32  written (accumulate = 0) or added to (accumulate = 1) */
int shared_expert_ffn(const moe_shape *shape, int T, const uint16_t *x, const uint16_t *w_gate,
                      const uint16_t *w_up, const uint16_t *w_down, float *out, int accumulate,
                      void *ws, size_t ws_bytes, void *stream);

/* REAP expert saliency over a calibration batch.
 * Follows: kimi-k3-mlx README, REAP section (each expert scored on a
 * calibration set by S_j = (1/|C|) * sum over tokens of g_j(x) * ||e_j(x)||_2,
 * computed one layer at a time from the layer's router gates and expert
 * outputs).  This call accumulates the numerator and the per-expert token
 * counts; the caller divides by |C| (or by the counts).
 *   P             rows of Y (T * top_k pairs), >= 0
 *   expert_offsets [E+1] int32, expert j owns sorted rows offsets[j] .. offsets[j+1]
 *                 (moe_permute's output)
 *   Y             [P, L] fp32, the expert outputs e_j(x) in expert-sorted order,
 *                 un-weighted (mxfp4_grouped_gemm(MOE_OP_DOWN) without pair weights);
 *                 may be NULL when P == 0
 *   pair_weight   [T*k] fp32 routing weights g in pair order (moe_route's topk_w)
 *   sorted_pair   [P] int32, pair index of each sorted row (moe_permute's output);
 *                 pair_weight and sorted_pair are both given, or both NULL when the
 *                 rows of Y already carry their weight (g >= 0, so ||g e|| = g ||e||)
 *   sal_sum       [E] float64: sum of g * ||e|| over the batch's rows of each expert
 *   counts        [E] int64: the number of those rows
 *   accumulate    0: overwrite sal_sum and counts; 1: add to them (a calibration
 *                 pass calls this once per batch)
 * Deterministic: fixed-order reductions, no atomics.  Workspace:
 * moe_workspace_bytes(shape, MOE_FN_REAP_SALIENCY, P) bytes (one fp32 per row).
 * Errors: MOE_EINVAL (null required pointer, P < 0, accumulate not 0/1, only
 * one of pair_weight / sorted_pair, misaligned Y or ws), MOE_EWORKSPACE. */
int moe_reap_saliency(const moe_shape *shape, int P, const int32_t *expert_offsets, const float *Y,
                      const float *pair_weight, const int32_t *sorted_pair, double *sal_sum,
                      int64_t *counts, int accumulate, void *ws, size_t ws_bytes, void *stream);

/* moe_combine_norm_up with the REAP saliency accumulation fused into it: the
 * combine reads every expert output row of the batch anyway, so the row norms
 * ||e_j(x)||_2 are taken in the same pass instead of a second read of Y.
 * Follows: kimi-k3-mlx README, REAP section (S_j as for moe_reap_saliency) and
 * the sources cited at moe_combine_norm_up.
 *   T .. accumulate   as for moe_combine_norm_up; out is bitwise what that call
 *                     writes.  g is topk_w, or 1 when topk_w is NULL (the rows
 *                     of Y already carry their weight: ||g e|| = g ||e||).
 *   expert_offsets    [E+1] int32 from moe_permute (expert j owns sorted rows
 *                     offsets[j] .. offsets[j+1] of Y)
 *   sal_sum, counts   [E] float64 / int64, as for moe_reap_saliency
 *   reap_accumulate   0: overwrite sal_sum and counts; 1: add to them
 * Deterministic: fixed-order reductions, no atomics.  Workspace:
 * moe_workspace_bytes(shape, MOE_FN_COMBINE_NORM_UP_REAP, T) bytes.
 * Errors: those of moe_combine_norm_up; MOE_EINVAL (null expert_offsets,
 * sal_sum or counts, reap_accumulate not 0/1); MOE_ENOTSUP (latent > 4096:
 * the fused pass holds a whole row per workgroup pass). */
int moe_combine_norm_up_reap(const moe_shape *shape, int T, const float *Y, const int32_t *pair_pos,
                             const float *topk_w, const uint16_t *gamma, const uint16_t *w_up, float *out,
                             int accumulate, const int32_t *expert_offsets, double *sal_sum, int64_t *counts,
                             int reap_accumulate, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LATENT_H */
