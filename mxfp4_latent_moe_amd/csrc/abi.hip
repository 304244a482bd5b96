// C ABI entry points: argument validation, workspace layout, launches.
// Nothing here allocates, frees or synchronises; every call only enqueues.
#include <atomic>
#include <cstring>
#include <mutex>

#include "kernels.h"
#include "moe_latent.h"

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const moe_shape *s) {
  if (s == nullptr) return MOE_EINVAL;
  if (s->hidden <= 0 || s->latent <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->inter <= 0 ||
      s->n_shared < 0 || s->shared_inter < 0)
    return MOE_EINVAL;
  if (s->operand_mode != MOE_OPND_BF16X2 && s->operand_mode != MOE_OPND_BF16 &&
      s->operand_mode != MOE_OPND_MX8X3 && s->operand_mode != MOE_OPND_MX6X3)
    return MOE_EINVAL;
  if (!(s->beta > 0.f) || !(s->beta_lin > 0.f) || !(s->rms_eps >= 0.f)) return MOE_EINVAL;
  if (s->top_k > s->n_experts) return MOE_EINVAL;
  if (s->hidden % 128 || s->latent % 128 || s->inter % 128 || (s->n_shared * s->shared_inter) % 128)
    return MOE_ENOTSUP;
  if (s->n_experts > 1024 || s->top_k > 32) return MOE_ENOTSUP;
  return MOE_OK;
}

// gfx950 check, cached per device
std::mutex g_arch_mu;
int g_arch_ok[64];  // 0 unknown, 1 ok, -1 not gfx950

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= 64) return MOE_ENOTSUP;
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_EHIP;
    g_arch_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return g_arch_ok[dev] == 1 ? MOE_OK : MOE_ENOTSUP;
}

int afmt_of(const moe_shape *s) {
  return s->operand_mode == MOE_OPND_BF16 ? A_F32_ROUND : A_F32_SPLIT;
}

// ---- workspace layouts (offsets from ws)
struct RouteWs {
  size_t logits, partial, total;
  GemmPlan pr, pd;
};
RouteWs route_ws(const moe_shape *s, int T) {
  RouteWs w{};
  w.pr = plan_dense(T, s->n_experts, s->hidden, false);
  w.pd = plan_dense(T, s->latent, s->hidden, false);
  w.logits = 0;
  w.partial = align_up((size_t)T * s->n_experts * sizeof(float));
  w.total = w.partial + align_up(std::max(w.pr.partial_bytes, w.pd.partial_bytes));
  return w;
}

size_t permute_ws(const moe_shape *s, int T) {
  return align_up((size_t)permute_blocks(T) * s->n_experts * sizeof(int32_t));
}

// MX activation terms (fp8 or fp6) are used for fp32 activations on the tiled
// path, while 3 term planes of `rows` rows stay addressable with 32-bit offsets
bool use_mx8(const moe_shape *s, const GemmPlan &pl, long long rows, int K) {
  return (s->operand_mode == MOE_OPND_MX8X3 || s->operand_mode == MOE_OPND_MX6X3) && pl.variant == 3 &&
         3LL * rows * K < (1LL << 32) - 256;
}

struct GroupedWs {
  size_t chunks, count, chunks2, count2, partial, mx, total;
  GemmPlan plan;
};

// Batches of a few rows per expert (P < 8 E) on the tiled path: the experts
// with at most PERSIST_ROWS_WIDE rows run on the persistent streaming kernel
// (one chunk each, its weights streamed once at the decode kernel's rate),
// the larger ones on the tiled kernel.
bool hybrid_grouped(const moe_shape *s, const GemmPlan &pl, int P, int K) {
  return pl.variant == 3 && s->operand_mode != MOE_OPND_MX8X3 && s->operand_mode != MOE_OPND_MX6X3 &&
         grouped_stream_fits(K) && (long long)P < 8LL * s->n_experts;
}
GroupedWs grouped_ws(const moe_shape *s, int P, bool gateup) {
  GroupedWs w{};
  const int K = gateup ? s->latent : s->inter;
  w.plan = gateup ? plan_grouped(P, s->n_experts, s->inter, s->latent, true)
                  : plan_grouped(P, s->n_experts, s->latent, s->inter, false);
  w.chunks = 0;
  w.count = align_up((size_t)w.plan.max_chunks * 16);
  // the streaming kernel's chunk list of a split batch: at most one chunk per expert
  w.chunks2 = w.count + ALIGN;
  w.count2 = w.chunks2 + (w.plan.variant == 3 ? align_up((size_t)s->n_experts * 16) : 0);
  w.partial = w.count2 + ALIGN;
  w.mx = w.partial + align_up(w.plan.partial_bytes);
  // the MX term planes or the bf16 activation planes hold at most P rows
  // (gathered activations with more rows than P are split per sorted row)
  size_t split = 0;
  if (use_mx8(s, w.plan, P, K)) split = mx8_split_bytes(P, K);
  else if (w.plan.variant == 3) split = split_rows_bytes(P, K, s->operand_mode == MOE_OPND_BF16 ? 1 : 2);
  w.total = w.mx + align_up(split);
  return w;
}

// two-bank call: a chunk list and count per bank, then the split-K partials
struct TwoBankWs {
  size_t chunks[2], count[2], partial, planes, sums, total;
  GemmPlan plan;
};
TwoBankWs two_bank_ws(const moe_shape *s, int P, bool gateup) {
  TwoBankWs w{};
  w.plan = gateup ? plan_grouped(P, s->n_experts, s->inter, s->latent, true)
                  : plan_grouped(P, s->n_experts, s->latent, s->inter, false);
  const size_t list = align_up((size_t)w.plan.max_chunks * 16);
  w.chunks[0] = 0;
  w.count[0] = list;
  w.chunks[1] = w.count[0] + ALIGN;
  w.count[1] = w.chunks[1] + list;
  w.partial = w.count[1] + ALIGN;
  w.planes = w.partial + align_up(w.plan.partial_bytes);
  // the tiled path's bf16 activation planes and (for an affine bank) their
  // 64-element group sums, at most P rows as in the single-bank call
  const int K = gateup ? s->latent : s->inter;
  const bool tiled = w.plan.variant == 3;
  w.sums = w.planes + (tiled ? align_up(split_rows_bytes(P, K, s->operand_mode == MOE_OPND_BF16 ? 1 : 2)) : 0);
  w.total = w.sums + (tiled && K % 512 == 0 ? align_up(row_sums_bytes(P, K)) : 0);
  return w;
}

// bf16 planes of fp32 activations for the dense tiled kernel (hi, then lo)
size_t planes_bytes(const GemmPlan &pl, int rows, int K, int afmt) {
  if (pl.variant != 4 || afmt == A_BF16) return 0;
  return align_up((size_t)rows * K * 2 * (afmt == A_F32_SPLIT ? 2 : 1));
}

struct CombineWs {
  size_t yn, partial, planes, total;
  GemmPlan pu;
};
CombineWs combine_ws(const moe_shape *s, int T) {
  CombineWs w{};
  w.pu = plan_dense(T, s->hidden, s->latent, false);
  w.yn = 0;
  w.partial = align_up((size_t)T * s->latent * sizeof(float));
  w.planes = w.partial + align_up(w.pu.partial_bytes);
  w.total = w.planes + planes_bytes(w.pu, T, s->latent, afmt_of(s));
  return w;
}

// the combine's workspace, then one fp32 REAP contribution per pair
size_t combine_reap_ws(const moe_shape *s, int T) {
  return combine_ws(s, T).total + align_up((size_t)T * s->top_k * sizeof(float));
}

struct SharedWs {
  size_t hs, partial, planes, total;
  GemmPlan pgu, pdn;
};
SharedWs shared_ws(const moe_shape *s, int T) {
  SharedWs w{};
  const int NS = s->n_shared * s->shared_inter;
  w.pgu = plan_dense(T, NS, s->hidden, true);
  w.pdn = plan_dense(T, s->hidden, NS, false);
  w.hs = 0;
  w.partial = align_up((size_t)T * NS * sizeof(float));
  w.planes = w.partial + align_up(std::max(w.pgu.partial_bytes, w.pdn.partial_bytes));
  w.total = w.planes + planes_bytes(w.pdn, T, NS, afmt_of(s));
  return w;
}

char *wsp(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

GemmArgs dense_args(const GemmPlan &pl, const void *A, long long lda, const void *W0, const void *W1,
                    int N, int K, float *C, long long ldc, int accumulate, int rows, float *partial,
                    const moe_shape *s) {
  GemmArgs a{};
  a.A = A;
  a.lda = lda;
  a.a_map = nullptr;
  a.a_div = 1;
  a.W0 = W0;
  a.W1 = W1;
  a.w_estride = 0;
  a.s_estride = 0;
  a.N = N;
  a.K = K;
  a.C = C;
  a.ldc = ldc;
  a.accumulate = accumulate;
  a.chunks = nullptr;
  a.chunk_count = nullptr;
  a.dense_rows = rows;
  a.n_blocks = pl.n_blocks;
  a.splits = pl.splits;
  a.grid_logical = (int)pl.grid_logical;
  a.partial = partial;
  a.partial_rows = rows;
  a.beta = s->beta;
  a.beta_lin = s->beta_lin;
  a.A2 = nullptr;
  a.dense_rows_tiles = pl.variant == 4 ? pl.max_chunks : 0;
  return a;
}

// dense GEMM plus, for split K, the finalize pass.  The tiled kernel takes
// fp32 activations as bf16 planes, written first into `planes`.
// planes_ready: a0.A (and a0.A2) already hold the activations as bf16 planes
hipError_t run_dense(const GemmPlan &pl, int afmt, bool pair, const GemmArgs &a0, void *planes,
                     hipStream_t st, bool planes_ready = false) {
  GemmArgs a = a0;
  if (pl.variant == 4 && afmt != A_BF16 && !planes_ready) {
    uint16_t *hi = static_cast<uint16_t *>(planes);
    uint16_t *lo = afmt == A_F32_SPLIT ? hi + (size_t)a.dense_rows * a.K : nullptr;
    hipError_t e = launch_split_planes(static_cast<const float *>(a.A), a.lda, a.dense_rows, a.K, hi, lo, st);
    if (e != hipSuccess) return e;
    a.A = hi;
    a.A2 = lo;
    a.lda = a.K;
  }
  hipError_t e = launch_gemm(pl, W_BF16, afmt, pair, a, st);
  if (e != hipSuccess || pl.splits == 1) return e;
  FinalizeArgs f{};
  f.partial = a.partial;
  f.splits = pl.splits;
  f.rows = a.dense_rows;
  f.N = a.N;
  f.pair = pair ? 1 : 0;
  f.C = a.C;
  f.ldc = a.ldc;
  f.accumulate = a.accumulate;
  f.rscale = nullptr;
  f.rscale_map = nullptr;
  f.beta = a.beta;
  f.beta_lin = a.beta_lin;
  return launch_finalize(f, st);
}

template <typename F>
int guarded(F &&f) {
  try {
    return f();
  } catch (...) {
    return MOE_EINTERNAL;
  }
}

// ---- the fixed routing scratch of moe_route_noalloc: one copy per device,
// alive until the process ends.  Host code never uses the array's name as an
// address; it uses the device address hipGetSymbolAddress returned for the
// current device.
constexpr size_t NOALLOC_SCRATCH_BYTES = MOE_ROUTE_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

}  // namespace

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device.
static int scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= 64) return MOE_ENOTSUP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Router, top-k (capped when `promoted` is given) and the latent projection.
static int route_impl(const moe_shape *s, int T, const uint16_t *x, const uint16_t *w_router, const float *bias,
                      const uint16_t *w_down, const uint8_t *promoted, int k_hi, int32_t *topk_ids, float *topk_w,
                      float *z, float *gap, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (T <= 0 || !x || !ws) return MOE_EINVAL;
  if ((w_down == nullptr) != (z == nullptr)) return MOE_EINVAL;
  // routing needs the router, bias and both outputs; without a router only z is computed
  const bool routing = w_router != nullptr;
  if (routing && (!bias || !topk_ids || !topk_w)) return MOE_EINVAL;
  if (!routing && (bias || topk_ids || topk_w || gap || !z)) return MOE_EINVAL;
  if ((routing && !aligned16(w_router)) || (w_down && !aligned16(w_down)) || !aligned16(x) ||
      (z && !aligned16(z)) || !aligned16(ws))
    return MOE_EINVAL;
  const RouteWs w = route_ws(s, T);
  if (ws_bytes < w.total) return MOE_EWORKSPACE;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float *logits = reinterpret_cast<float *>(wsp(ws, w.logits));
  float *partial = reinterpret_cast<float *>(wsp(ws, w.partial));
  if (routing) {
    GemmArgs a = dense_args(w.pr, x, s->hidden, w_router, nullptr, s->n_experts, s->hidden, logits,
                            s->n_experts, 0, T, partial, s);
    // no finalize pass: the top-k kernel adds the split-K partials itself
    if (launch_gemm(w.pr, W_BF16, A_BF16, false, a, st) != hipSuccess) return MOE_EHIP;
    const float *part = w.pr.splits > 1 ? partial : nullptr;
    if (launch_topk(logits, part, w.pr.splits, bias, T, s->n_experts, s->top_k, topk_ids, topk_w, gap, promoted,
                    k_hi, st) != hipSuccess)
      return MOE_EHIP;
  }
  if (z) {
    GemmArgs d = dense_args(w.pd, x, s->hidden, w_down, nullptr, s->latent, s->hidden, z, s->latent, 0, T,
                            partial, s);
    if (run_dense(w.pd, A_BF16, false, d, nullptr, st) != hipSuccess) return MOE_EHIP;
  }
  return MOE_OK;
}

// combine + RMSNorm writing y_n straight into the bf16 planes the tiled
// up_proj reads (no fp32 y_n, no split pass), then up_proj
static bool combine_planes_ok(const moe_shape *s, const CombineWs &w) {
  return w.pu.variant == 4 && s->latent <= 4096 && s->latent % 4 == 0;
}
static int combine_planes_up(const moe_shape *s, int T, const float *Y, const int32_t *pair_pos, const float *topk_w,
                             const uint16_t *gamma, const uint16_t *w_up, float *out, int accumulate,
                             const CombineWs &w, void *ws, hipStream_t st) {
  const int afmt = afmt_of(s);
  uint16_t *hi = reinterpret_cast<uint16_t *>(wsp(ws, w.planes));
  uint16_t *lo = afmt == A_F32_SPLIT ? hi + (size_t)T * s->latent : nullptr;
  if (launch_combine_norm_planes(Y, pair_pos, topk_w, gamma, T, s->top_k, s->latent, s->rms_eps, hi, lo, st) !=
      hipSuccess)
    return MOE_EHIP;
  GemmArgs a = dense_args(w.pu, hi, s->latent, w_up, nullptr, s->hidden, s->latent, out, s->hidden, accumulate, T,
                          reinterpret_cast<float *>(wsp(ws, w.partial)), s);
  a.A2 = lo;
  if (run_dense(w.pu, afmt, false, a, nullptr, st, true) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

// The combine call, with the REAP saliency pass fused in when sal_sum is given
// (its per-row contributions go to the workspace after the combine's own).
static int combine_norm_up_impl(const moe_shape *s, int T, const float *Y, const int32_t *pair_pos,
                                const float *topk_w, const uint16_t *gamma, const uint16_t *w_up, float *out,
                         int accumulate, const int32_t *expert_offsets, double *sal_sum, int64_t *counts,
                         int reap_accumulate, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (T <= 0 || !Y || !pair_pos || !gamma || !w_up || !out || !ws) return MOE_EINVAL;
  if (accumulate != 0 && accumulate != 1) return MOE_EINVAL;
  if (!aligned16(Y) || !aligned16(w_up) || !aligned16(out) || !aligned16(ws)) return MOE_EINVAL;
  const bool reap = sal_sum != nullptr;
  if (reap && s->latent > 4096) return MOE_ENOTSUP;
  const CombineWs w = combine_ws(s, T);
  const size_t need = reap ? combine_reap_ws(s, T) : w.total;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!reap && combine_planes_ok(s, w))
    return combine_planes_up(s, T, Y, pair_pos, topk_w, gamma, w_up, out, accumulate, w, ws, st);
  float *yn = reinterpret_cast<float *>(wsp(ws, w.yn));
  float *contrib = reap ? reinterpret_cast<float *>(wsp(ws, w.total)) : nullptr;
  if (launch_combine_norm(Y, pair_pos, topk_w, gamma, T, s->top_k, s->latent, s->rms_eps, yn, contrib, st) !=
      hipSuccess)
    return MOE_EHIP;
  if (reap && launch_reap_experts(contrib, expert_offsets, s->n_experts, sal_sum,
                                  reinterpret_cast<long long *>(counts), reap_accumulate, st) != hipSuccess)
    return MOE_EHIP;
  GemmArgs a = dense_args(w.pu, yn, s->latent, w_up, nullptr, s->hidden, s->latent, out, s->hidden, accumulate,
                          T, reinterpret_cast<float *>(wsp(ws, w.partial)), s);
  if (run_dense(w.pu, afmt_of(s), false, a, wsp(ws, w.planes), st) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}


extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, size, enum or alignment)";
    case MOE_ENOTSUP: return "unsupported shape or device (needs gfx950 and the compiled tiling)";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_EINTERNAL: return "internal error";
    default: return "unknown error code";
  }
}

size_t moe_workspace_bytes(const moe_shape *s, int fn, int n) {
  if (check_shape(s) != MOE_OK || n <= 0) return 0;
  switch (fn) {
    case MOE_FN_ROUTE: return route_ws(s, n).total;
    case MOE_FN_PERMUTE: return permute_ws(s, n);
    case MOE_FN_GROUPED_GEMM: {
      const size_t a = grouped_ws(s, n, true).total, b = grouped_ws(s, n, false).total;
      return a > b ? a : b;
    }
    case MOE_FN_COMBINE_NORM_UP: return combine_ws(s, n).total;
    case MOE_FN_SHARED_FFN:
      if (s->n_shared * s->shared_inter == 0) return ALIGN;
      return shared_ws(s, n).total;
    case MOE_FN_REAP_SALIENCY: return align_up((size_t)n * sizeof(float));
    case MOE_FN_COMBINE_NORM_UP_REAP: return combine_reap_ws(s, n);
    case MOE_FN_GROUPED_GEMM_TWO_BANK: {
      const size_t a = two_bank_ws(s, n, true).total, b = two_bank_ws(s, n, false).total;
      return a > b ? a : b;
    }
    default: return 0;
  }
}

int moe_route(const moe_shape *s, int T, const uint16_t *x, const uint16_t *w_router,
              const float *bias, const uint16_t *w_down, int32_t *topk_ids, float *topk_w, float *z,
              float *gap, void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    return route_impl(s, T, x, w_router, bias, w_down, nullptr, 0, topk_ids, topk_w, z, gap, ws, ws_bytes, stream);
  });
}

int moe_route_noalloc(const moe_shape *s, int T, const uint16_t *x, const uint16_t *w_router, const float *bias,
                      const uint16_t *w_down, int32_t *topk_ids, float *topk_w, float *z, float *gap, void *stream) {
  return guarded([&]() -> int {
    int rc = check_shape(s);
    if (rc) return rc;
    if (T <= 0) return MOE_EINVAL;
    // the same workspace layout moe_route uses, in the fixed scratch
    if (route_ws(s, T).total > NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    void *ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return route_impl(s, T, x, w_router, bias, w_down, nullptr, 0, topk_ids, topk_w, z, gap, ws,
                      NOALLOC_SCRATCH_BYTES, stream);
  });
}

int moe_route_capped(const moe_shape *s, int T, const uint16_t *x, const uint16_t *w_router, const float *bias,
                     const uint16_t *w_down, const uint8_t *promoted, int k_hi, int32_t *topk_ids, float *topk_w,
                     float *z, float *gap, void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    if (!promoted || !w_router || k_hi < 0) return MOE_EINVAL;
    return route_impl(s, T, x, w_router, bias, w_down, promoted, k_hi, topk_ids, topk_w, z, gap, ws, ws_bytes,
                      stream);
  });
}

int moe_permute(const moe_shape *s, int T, const int32_t *topk_ids, int32_t *expert_offsets,
                int32_t *sorted_pair, int32_t *pair_pos, int32_t *active, void *ws,
                size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    int rc = check_shape(s);
    if (rc) return rc;
    if (T <= 0 || !topk_ids || !expert_offsets || !sorted_pair || !pair_pos || !ws)
      return MOE_EINVAL;
    if ((long long)T * s->top_k > 0x7fffffffLL) return MOE_EINVAL;
    if (ws_bytes < permute_ws(s, T)) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (launch_permute(topk_ids, T, s->top_k, s->n_experts, static_cast<int32_t *>(ws),
                       expert_offsets, sorted_pair, pair_pos, active, st) != hipSuccess)
      return MOE_EHIP;
    return MOE_OK;
  });
}

int mxfp4_grouped_gemm(const moe_shape *s, int op, int P, const int32_t *expert_offsets,
                       const int32_t *sorted_pair, const void *A, int a_rows, int a_dtype,
                       const uint8_t *w_packed, const uint8_t *w_scale, const uint8_t *w3_packed,
                       const uint8_t *w3_scale, const float *pair_weight, float *C, void *ws,
                       size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    int rc = check_shape(s);
    if (rc) return rc;
    if (op != MOE_OP_GATEUP_SITU && op != MOE_OP_DOWN && op != MOE_OP_GATEUP_SITU_BF16X2) return MOE_EINVAL;
    if (a_dtype != MOE_DT_F32 && a_dtype != MOE_DT_BF16 && (a_dtype != MOE_DT_BF16X2 || op != MOE_OP_DOWN))
      return MOE_EINVAL;
    if (P <= 0 || !expert_offsets || !A || !w_packed || !w_scale || !C || !ws) return MOE_EINVAL;
    const bool gateup = op != MOE_OP_DOWN;
    // H as bf16 hi + lo planes: written by the gate/up epilogue, read by down
    const bool planes_out = op == MOE_OP_GATEUP_SITU_BF16X2, planes_in = a_dtype == MOE_DT_BF16X2;
    // gate/up with sorted_pair gathers rows of A (z [T, L]); otherwise A holds the P sorted rows
    const bool gathered = gateup && sorted_pair != nullptr;
    if (a_rows < 1 || (!gathered && a_rows < P)) return MOE_EINVAL;
    if (gathered && (long long)a_rows * (gateup ? s->latent : s->inter) * (a_dtype == MOE_DT_BF16 ? 2 : 4) >=
                        (1LL << 31))
      return MOE_ENOTSUP;
    if (gateup && (!w3_packed || !w3_scale)) return MOE_EINVAL;
    if (!gateup && (w3_packed || w3_scale)) return MOE_EINVAL;
    if (gateup && pair_weight) return MOE_EINVAL;
    if (pair_weight && !sorted_pair) return MOE_EINVAL;
    if (!aligned16(A) || !aligned16(w_packed) || !aligned16(C) || !aligned16(ws) ||
        (w3_packed && !aligned16(w3_packed)) || (reinterpret_cast<uintptr_t>(w_scale) & 3u) ||
        (w3_scale && (reinterpret_cast<uintptr_t>(w3_scale) & 3u)))
      return MOE_EINVAL;
    const GroupedWs w = grouped_ws(s, P, gateup);
    const int N = gateup ? s->inter : s->latent;
    const int K = gateup ? s->latent : s->inter;
    const bool hybrid = hybrid_grouped(s, w.plan, P, K);
    // the bf16-plane forms: the tiled path with no small-expert split, bf16 operand modes
    if ((planes_out || planes_in) && (w.plan.variant != 3 || hybrid ||
                                      (s->operand_mode != MOE_OPND_BF16X2 && s->operand_mode != MOE_OPND_BF16)))
      return MOE_ENOTSUP;
    if (ws_bytes < w.total) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t *chunks = reinterpret_cast<int32_t *>(wsp(ws, w.chunks));
    int32_t *count = reinterpret_cast<int32_t *>(wsp(ws, w.count));
    // the tiled kernel's chunks: every expert, or in a split batch the experts above the streaming kernel's rows
    if (launch_plan_chunks(expert_offsets, s->n_experts, w.plan.chunk_rows, chunks, count, st,
                           hybrid ? PERSIST_ROWS_WIDE + 1 : 1) != hipSuccess)
      return MOE_EHIP;
    GemmArgs a{};
    a.A = A;
    a.lda = K;
    a.a_map = gathered ? sorted_pair : nullptr;
    a.a_div = s->top_k;
    a.a_rows = a_rows;
    a.W0 = w_packed;
    a.W1 = w3_packed;
    a.S0 = w_scale;
    a.S1 = w3_scale;
    a.w_estride = (long long)N * (K / 2);
    a.s_estride = (long long)N * (K / 32);
    a.N = N;
    a.K = K;
    a.C = C;
    a.ldc = N;
    a.accumulate = 0;
    if (planes_out) {
      a.c_hi = reinterpret_cast<uint16_t *>(C);
      a.c_lo = a.c_hi + N;
      a.ldc = 2 * N;
    }
    a.rscale = pair_weight;
    a.rscale_map = pair_weight ? sorted_pair : nullptr;
    a.chunks = chunks;
    a.chunk_count = count;
    a.dense_rows = 0;
    a.n_blocks = w.plan.n_blocks;
    a.splits = w.plan.splits;
    a.grid_logical = (int)w.plan.grid_logical;
    a.partial = reinterpret_cast<float *>(wsp(ws, w.partial));
    a.partial_rows = P;
    a.beta = s->beta;
    a.beta_lin = s->beta_lin;
    int afmt = a_dtype == MOE_DT_BF16 ? A_BF16 : afmt_of(s);
    if (a_dtype == MOE_DT_F32 && use_mx8(s, w.plan, P, K)) {
      // split the fp32 activation rows into three MX terms, then the MX-scaled GEMM.
      // Gathered rows of z [a_rows, K]: the split covers z's rows and the GEMM gathers
      // them through sorted_pair, or, when z has more rows than the call has pairs (an
      // expert slice), the split gathers row p = z[sorted_pair[p] / k] and the GEMM
      // reads the P split rows in order.  Down reads H [P, K] in order.
      const bool split_gathers = gathered && a_rows > P;
      const long long rows = (gathered && !split_gathers) ? (long long)a_rows : (long long)P;
      uint8_t *mx = reinterpret_cast<uint8_t *>(wsp(ws, w.mx));
      const bool fp6 = s->operand_mode == MOE_OPND_MX6X3;
      if (launch_mx_split(fp6, static_cast<const float *>(A), K, (int)rows, K, split_gathers ? sorted_pair : nullptr,
                          s->top_k, mx, st) != hipSuccess)
        return MOE_EHIP;
      a.mxq = mx;
      a.mxs = mx + (size_t)rows * K * 3;
      a.mx_rows = rows;
      if (split_gathers) a.a_map = nullptr;
      afmt = fp6 ? A_MX6X3 : A_MX8X3;
    }
    if (hybrid) {
      // the small experts on the streaming kernel, which stages their rows itself
      int32_t *chunks2 = reinterpret_cast<int32_t *>(wsp(ws, w.chunks2));
      int32_t *count2 = reinterpret_cast<int32_t *>(wsp(ws, w.count2));
      if (launch_plan_chunks(expert_offsets, s->n_experts, PERSIST_ROWS_WIDE, chunks2, count2, st, 1,
                             PERSIST_ROWS_WIDE) != hipSuccess)
        return MOE_EHIP;
      GemmArgs as = a;
      as.chunks = chunks2;
      as.chunk_count = count2;
      as.n_blocks = (N + grouped_stream_rows_per_wg(gateup, PERSIST_ROWS_WIDE) - 1) /
                    grouped_stream_rows_per_wg(gateup, PERSIST_ROWS_WIDE);
      as.splits = 1;
      as.grid_logical = s->n_experts * as.n_blocks;
      if (launch_grouped_stream(W_MXFP4, afmt, gateup, as, st, PERSIST_ROWS_WIDE) != hipSuccess) return MOE_EHIP;
    }
    if (w.plan.variant == 3 && afmt != A_MX8X3 && afmt != A_MX6X3) {
      // bf16 activation planes: bf16 activations are one plane already; fp32
      // ones are split first (hi + lo, or rounded), over the same rows as the
      // MX split above
      int npl = 1;
      if (planes_in) {
        // the caller's planes: hi and lo (or hi alone for a rounded operand), rows of 2 K
        npl = afmt == A_F32_SPLIT ? 2 : 1;
        a.lda = 2LL * K;
      } else if (a_dtype == MOE_DT_F32) {
        npl = afmt == A_F32_SPLIT ? 2 : 1;
        const bool split_gathers = gathered && a_rows > P;
        const long long rows = (gathered && !split_gathers) ? (long long)a_rows : (long long)P;
        uint16_t *planes = reinterpret_cast<uint16_t *>(wsp(ws, w.mx));
        if (launch_split_rows(npl, static_cast<const float *>(A), K, rows, K, split_gathers ? sorted_pair : nullptr,
                              s->top_k, planes, nullptr, st) != hipSuccess)
          return MOE_EHIP;
        a.A = planes;
        a.lda = (long long)npl * K;
        a.a_rows = rows;
        if (split_gathers) a.a_map = nullptr;
      }
      const int rows_wg = prefill_pl_rows_per_wg(gateup, W_MXFP4);
      a.n_blocks = (N + rows_wg - 1) / rows_wg;
      const long long logical = (long long)w.plan.max_chunks * a.n_blocks;
      a.grid_logical = (int)logical;
      if (launch_prefill_planes(W_MXFP4, npl, gateup, a, (logical + 7) / 8 * 8, st) != hipSuccess) return MOE_EHIP;
      return MOE_OK;
    }
    GemmPlan pl = w.plan;
    if (afmt == A_MX8X3 || afmt == A_MX6X3) {
      // the MX kernel covers fewer weight rows per work-group
      pl.n_blocks = (N + prefill_mx_rows_per_wg(gateup) - 1) / prefill_mx_rows_per_wg(gateup);
      pl.grid_logical = (long long)pl.max_chunks * pl.n_blocks;
      a.n_blocks = pl.n_blocks;
      a.grid_logical = (int)pl.grid_logical;
    }
    if (launch_gemm(pl, W_MXFP4, afmt, gateup, a, st) != hipSuccess) return MOE_EHIP;
    if (w.plan.splits > 1) {
      FinalizeArgs f{};
      f.partial = a.partial;
      f.splits = w.plan.splits;
      f.rows = P;
      f.N = N;
      f.pair = gateup ? 1 : 0;
      f.C = C;
      f.ldc = N;
      f.accumulate = 0;
      f.rscale = pair_weight;
      f.rscale_map = pair_weight ? sorted_pair : nullptr;
      f.beta = s->beta;
      f.beta_lin = s->beta_lin;
      if (launch_finalize(f, st) != hipSuccess) return MOE_EHIP;
    }
    return MOE_OK;
  });
}

int moe_grouped_gemm_two_bank(const moe_shape *s, int op, int P, const int32_t *expert_offsets,
                              const int32_t *sorted_pair, const void *A, int a_rows, int a_dtype,
                              const moe_expert_bank *bank_a, const moe_expert_bank *bank_b,
                              const float *pair_weight, float *C, void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    int rc = check_shape(s);
    if (rc) return rc;
    if (op != MOE_OP_GATEUP_SITU && op != MOE_OP_DOWN) return MOE_EINVAL;
    if (a_dtype != MOE_DT_F32 && a_dtype != MOE_DT_BF16) return MOE_EINVAL;
    if (P <= 0 || !expert_offsets || !A || !C || !ws || !bank_a || !bank_b) return MOE_EINVAL;
    const bool gateup = op == MOE_OP_GATEUP_SITU;
    const bool gathered = gateup && sorted_pair != nullptr;
    if (a_rows < 1 || (!gathered && a_rows < P)) return MOE_EINVAL;
    const int N = gateup ? s->inter : s->latent;
    const int K = gateup ? s->latent : s->inter;
    if (gathered && (long long)a_rows * K * (a_dtype == MOE_DT_BF16 ? 2 : 4) >= (1LL << 31)) return MOE_ENOTSUP;
    if (gateup && pair_weight) return MOE_EINVAL;
    if (pair_weight && !sorted_pair) return MOE_EINVAL;
    if (!aligned16(A) || !aligned16(C) || !aligned16(ws)) return MOE_EINVAL;
    const moe_expert_bank *banks[2] = {bank_a, bank_b};
    bool any_affine = false;
    for (const moe_expert_bank *b : banks) {
      if (b->format != MOE_WF_MXFP4 && b->format != MOE_WF_AFFINE2) return MOE_EINVAL;
      if (b->n_experts < 0) return MOE_EINVAL;
      if (b->n_experts == 0) continue;
      const bool aff = b->format == MOE_WF_AFFINE2;
      any_affine |= aff;
      if (!b->packed || !b->scale || (aff != (b->bias != nullptr))) return MOE_EINVAL;
      if (gateup && (!b->packed3 || !b->scale3 || (aff != (b->bias3 != nullptr)))) return MOE_EINVAL;
      if (!gateup && (b->packed3 || b->scale3 || b->bias3)) return MOE_EINVAL;
      const uintptr_t salign = aff ? 15u : 3u;
      if (!aligned16(b->packed) || (reinterpret_cast<uintptr_t>(b->scale) & salign) || (b->bias && !aligned16(b->bias)) ||
          (b->packed3 && !aligned16(b->packed3)) || (b->scale3 && (reinterpret_cast<uintptr_t>(b->scale3) & salign)) ||
          (b->bias3 && !aligned16(b->bias3)))
        return MOE_EINVAL;
    }
    if ((long long)bank_a->n_experts + bank_b->n_experts != s->n_experts) return MOE_EINVAL;
    // the affine path runs with bf16 operands, on rows whose 64-element groups
    // come in whole 16-byte runs of biases
    if (s->operand_mode != MOE_OPND_BF16X2 && s->operand_mode != MOE_OPND_BF16) return MOE_ENOTSUP;
    const TwoBankWs w = two_bank_ws(s, P, gateup);
    if (any_affine) {
      if (K % 512 || K > 4096) return MOE_ENOTSUP;
      // the decode kernel keeps an item's biases in flight across at most one item boundary
      if (w.plan.variant != 2 && w.plan.variant != 3) return MOE_ENOTSUP;
      if (w.plan.variant == 2 && K / 128 < 12) return MOE_ENOTSUP;
    }
    if (ws_bytes < w.total) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    GemmArgs a{};
    a.A = A;
    a.lda = K;
    a.a_map = gathered ? sorted_pair : nullptr;
    a.a_div = s->top_k;
    a.a_rows = a_rows;
    a.N = N;
    a.K = K;
    a.C = C;
    a.ldc = N;
    a.accumulate = 0;
    a.rscale = pair_weight;
    a.rscale_map = pair_weight ? sorted_pair : nullptr;
    a.dense_rows = 0;
    a.n_blocks = w.plan.n_blocks;
    a.splits = w.plan.splits;
    a.partial = reinterpret_cast<float *>(wsp(ws, w.partial));
    a.partial_rows = P;
    a.beta = s->beta;
    a.beta_lin = s->beta_lin;
    const int afmt = a_dtype == MOE_DT_BF16 ? A_BF16 : afmt_of(s);
    // the tiled path reads bf16 activation planes: bf16 activations as they
    // are, fp32 ones split once (over the same rows as in the single-bank
    // call); an affine bank also takes the rows' 64-element group sums
    const bool tiled = w.plan.variant == 3;
    int npl = 1;
    if (tiled) {
      const bool split_gathers = gathered && a_rows > P;
      const long long rows = (gathered && !split_gathers) ? (long long)a_rows : (long long)P;
      const int32_t *map = split_gathers ? sorted_pair : nullptr;
      float *sums = any_affine ? reinterpret_cast<float *>(wsp(ws, w.sums)) : nullptr;
      if (a_dtype == MOE_DT_F32) {
        npl = afmt == A_F32_SPLIT ? 2 : 1;
        uint16_t *planes = reinterpret_cast<uint16_t *>(wsp(ws, w.planes));
        if (launch_split_rows(npl, static_cast<const float *>(A), K, rows, K, map, s->top_k, planes, sums, st) !=
            hipSuccess)
          return MOE_EHIP;
        a.A = planes;
        a.lda = (long long)npl * K;
        a.a_rows = rows;
        if (split_gathers) a.a_map = nullptr;
      } else if (sums) {
        // bf16 activations are their own plane (gathered through sorted_pair
        // as given); their group sums follow the rows the split would have
        if (launch_row_sums(static_cast<const uint16_t *>(A), K, rows, K, map, s->top_k, sums, st) != hipSuccess)
          return MOE_EHIP;
        a.asum_sorted = split_gathers ? 1 : 0;
      }
      a.asum = sums;
    }
    // bank A owns experts [0, E_a), bank B [E_a, E): each bank's chunks come from
    // its slice of the offsets on the device, so its sorted rows are found with
    // no host round trip
    int e0 = 0;
    for (int bi = 0; bi < 2; ++bi) {
      const moe_expert_bank *b = banks[bi];
      const int ne = b->n_experts;
      if (ne == 0) continue;
      const bool aff = b->format == MOE_WF_AFFINE2;
      int32_t *chunks = reinterpret_cast<int32_t *>(wsp(ws, w.chunks[bi]));
      int32_t *count = reinterpret_cast<int32_t *>(wsp(ws, w.count[bi]));
      if (launch_plan_chunks(expert_offsets + e0, ne, w.plan.chunk_rows, chunks, count, st) != hipSuccess)
        return MOE_EHIP;
      GemmArgs ab = a;
      ab.W0 = b->packed;
      ab.W1 = b->packed3;
      ab.S0 = static_cast<const uint8_t *>(b->scale);
      ab.S1 = static_cast<const uint8_t *>(b->scale3);
      ab.B0 = b->bias;
      ab.B1 = b->bias3;
      ab.w_estride = (long long)N * (K / (aff ? 4 : 2));
      ab.s_estride = aff ? (long long)N * (K / 64) * 2 : (long long)N * (K / 32);
      ab.chunks = chunks;
      ab.chunk_count = count;
      GemmPlan pl = w.plan;
      if (tiled) {
        // weight rows per work-group of the plane kernel in the bank's format
        const int rows_wg = prefill_pl_rows_per_wg(gateup, aff ? W_AFF2 : W_MXFP4);
        pl.n_blocks = (N + rows_wg - 1) / rows_wg;
        ab.n_blocks = pl.n_blocks;
      }
      pl.max_chunks = P / pl.chunk_rows + (ne < P ? ne : P);
      pl.grid_logical = (long long)pl.max_chunks * pl.n_blocks * pl.splits;
      ab.grid_logical = (int)pl.grid_logical;
      if (tiled) {
        if (launch_prefill_planes(aff ? W_AFF2 : W_MXFP4, npl, gateup, ab, (pl.grid_logical + 7) / 8 * 8, st) !=
            hipSuccess)
          return MOE_EHIP;
      } else if (launch_gemm(pl, aff ? W_AFF2 : W_MXFP4, afmt, gateup, ab, st) != hipSuccess) {
        return MOE_EHIP;
      }
      e0 += ne;
    }
    if (w.plan.splits > 1) {
      FinalizeArgs f{};
      f.partial = a.partial;
      f.splits = w.plan.splits;
      f.rows = P;
      f.N = N;
      f.pair = gateup ? 1 : 0;
      f.C = C;
      f.ldc = N;
      f.accumulate = 0;
      f.rscale = pair_weight;
      f.rscale_map = pair_weight ? sorted_pair : nullptr;
      f.beta = s->beta;
      f.beta_lin = s->beta_lin;
      if (launch_finalize(f, st) != hipSuccess) return MOE_EHIP;
    }
    return MOE_OK;
  });
}

int moe_combine_norm_up(const moe_shape *s, int T, const float *Y, const int32_t *pair_pos,
                        const float *topk_w, const uint16_t *gamma, const uint16_t *w_up,
                        float *out, int accumulate, void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    return combine_norm_up_impl(s, T, Y, pair_pos, topk_w, gamma, w_up, out, accumulate, nullptr, nullptr,
                                nullptr, 0, ws, ws_bytes, stream);
  });
}

int moe_combine_norm_up_reap(const moe_shape *s, int T, const float *Y, const int32_t *pair_pos,
                             const float *topk_w, const uint16_t *gamma, const uint16_t *w_up, float *out,
                             int accumulate, const int32_t *expert_offsets, double *sal_sum, int64_t *counts,
                             int reap_accumulate, void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    if (!expert_offsets || !sal_sum || !counts) return MOE_EINVAL;
    if (reap_accumulate != 0 && reap_accumulate != 1) return MOE_EINVAL;
    return combine_norm_up_impl(s, T, Y, pair_pos, topk_w, gamma, w_up, out, accumulate, expert_offsets,
                                sal_sum, counts, reap_accumulate, ws, ws_bytes, stream);
  });
}

int shared_expert_ffn(const moe_shape *s, int T, const uint16_t *x, const uint16_t *w_gate,
                      const uint16_t *w_up, const uint16_t *w_down, float *out, int accumulate,
                      void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    int rc = check_shape(s);
    if (rc) return rc;
    if (T <= 0 || !x || !out || !ws) return MOE_EINVAL;
    if (accumulate != 0 && accumulate != 1) return MOE_EINVAL;
    const int NS = s->n_shared * s->shared_inter;
    if (NS == 0) return MOE_EINVAL;
    if (!w_gate || !w_up || !w_down) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
        !aligned16(out) || !aligned16(ws))
      return MOE_EINVAL;
    const SharedWs w = shared_ws(s, T);
    if (ws_bytes < w.total) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *hs = reinterpret_cast<float *>(wsp(ws, w.hs));
    float *partial = reinterpret_cast<float *>(wsp(ws, w.partial));
    GemmArgs g = dense_args(w.pgu, x, s->hidden, w_gate, w_up, NS, s->hidden, hs, NS, 0, T, partial,
                            s);
    const int afmt = afmt_of(s);
    // whole-K gate/up tiles write h straight into the bf16 planes the tiled
    // down_proj reads (no fp32 h, no split pass)
    const bool planes = w.pgu.variant == 4 && w.pgu.splits == 1 && w.pdn.variant == 4 && NS % 4 == 0;
    if (planes) {
      g.c_hi = reinterpret_cast<uint16_t *>(wsp(ws, w.planes));
      g.c_lo = afmt == A_F32_SPLIT ? g.c_hi + (size_t)T * NS : nullptr;
    }
    if (run_dense(w.pgu, A_BF16, true, g, nullptr, st) != hipSuccess) return MOE_EHIP;
    GemmArgs d = dense_args(w.pdn, planes ? static_cast<const void *>(g.c_hi) : hs, NS, w_down, nullptr, s->hidden,
                            NS, out, s->hidden, accumulate, T, partial, s);
    if (planes) d.A2 = g.c_lo;
    if (run_dense(w.pdn, afmt, false, d, wsp(ws, w.planes), st, planes) != hipSuccess) return MOE_EHIP;
    return MOE_OK;
  });
}

int moe_reap_saliency(const moe_shape *s, int P, const int32_t *expert_offsets, const float *Y,
                      const float *pair_weight, const int32_t *sorted_pair, double *sal_sum, int64_t *counts,
                      int accumulate, void *ws, size_t ws_bytes, void *stream) {
  return guarded([&]() -> int {
    int rc = check_shape(s);
    if (rc) return rc;
    if (P < 0 || !expert_offsets || !sal_sum || !counts || (P > 0 && (!Y || !ws))) return MOE_EINVAL;
    if (accumulate != 0 && accumulate != 1) return MOE_EINVAL;
    if ((pair_weight == nullptr) != (sorted_pair == nullptr)) return MOE_EINVAL;
    if ((Y && !aligned16(Y)) || (ws && !aligned16(ws))) return MOE_EINVAL;
    if (ws_bytes < (size_t)P * sizeof(float)) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    if (launch_reap(Y, P, s->latent, pair_weight, sorted_pair, expert_offsets, s->n_experts, sal_sum,
                    reinterpret_cast<long long *>(counts), accumulate, static_cast<float *>(ws),
                    static_cast<hipStream_t>(stream)) != hipSuccess)
      return MOE_EHIP;
    return MOE_OK;
  });
}

}  // extern "C"
