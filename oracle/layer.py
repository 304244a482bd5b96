"""Float64 CPU oracle of one Stable LatentMoE layer forward (test infrastructure only).

The layer, as the pages state it:
  * kimi-k3-mlx README, Architecture table, MoE row: 896 routed experts,
    top-16, moe_intermediate_size 3072, a sigmoid router plus the aux-loss-free
    `e_score_correction_bias`, 2 shared experts on every token.
  * same table, Stable LatentMoE row: routed experts run in a 3584-d latent,
    not the 7168-d residual: down_proj -> experts -> RMSNorm -> up_proj.
  * same table, Activation row: SiTU-GLU, beta*tanh(g/beta)*sigmoid(g) *
    beta_lin*tanh(u/beta_lin) with beta = 4, beta_lin = 25; Porting notes
    item 1: computed in fp32 (bf16 rounding near tanh saturation is visible).
  * Porting notes item 3: experts work in the latent; shared experts do not.
  * AWQ section: one latent (the output of the routed-expert down projection)
    feeds every expert of the layer, and w1, w3 consume it.
  * REAP section, caveat paragraph: RMSNorm acts on the *combined* expert
    output, before up_proj.  Two-bank paragraph: pairs sorted by expert index
    give each expert a contiguous slice.
  * K3 open-artifact audit, section 4.3: w1/w3 packed [3072, 1792], w2 packed
    [3584, 1536], scales [N, K/32]; section 6: router weight [896, 7168] bf16,
    correction bias [896] fp32.

Readings where the pages are silent (each is listed with its reason in the
design notes of this repository):
  * the router reads the 7168-d input x (its weight is [896, 7168]);
  * the bias only selects; weights are the unbiased sigmoid scores of the
    selected experts divided by their sum; no scaling factor, no groups;
  * ties in the biased score go to the lower expert index; the selected ids
    are reported in ascending order (slot j = j-th smallest id);
  * the top-k decision is taken on float32 biased scores
    (float32(sigmoid) + float32 bias, rounded to float32);
  * w1 is the gate, w3 the up projection, w2 the down projection;
  * shared experts use SiTU-GLU too and run on x; their output is added after
    up_proj; RMSNorm eps = 1e-6, gamma given;
  * pairs are numbered p = t*k + j; the permutation is the stable sort of the
    pairs by expert id, so tokens ascend within each expert's slice.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit

from .mxfp4 import dequant

BETA = 4.0
BETA_LIN = 25.0
RMS_EPS = 1e-6


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def situ_glu(g, u, beta: float = BETA, beta_lin: float = BETA_LIN):
    """SiTU-GLU: beta*tanh(g/beta)*sigmoid(g) * beta_lin*tanh(u/beta_lin).
    kimi-k3-mlx README, Architecture table, Activation row."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return beta * np.tanh(g / beta) * expit(g) * (beta_lin * np.tanh(u / beta_lin))


def router_scores(x_bits, w_router_bits) -> tuple:
    """Router logits x W_r^T and sigmoid scores, float64.
    kimi-k3-mlx README, Architecture table, MoE row (sigmoid router); K3
    open-artifact audit, section 6 (router weight [E, H] bf16)."""
    logits = bf16_to_f64(x_bits) @ bf16_to_f64(w_router_bits).T
    return logits, expit(logits)


def select_topk(scores: np.ndarray, bias, top_k: int) -> dict:
    """Biased top-k selection and weight normalisation.

    Decision values: float32(score) + float32(bias), rounded to float32; the k
    largest win, ties to the lower expert index; ids are reported ascending.
    Weights: the selected unbiased scores divided by their sum.  gap: k-th
    minus (k+1)-th largest decision value (+inf when E == k).
    kimi-k3-mlx README, Architecture table, MoE row (aux-loss-free
    e_score_correction_bias); K3 open-artifact audit, section 6 (fp32 bias).
    """
    biased32 = scores.astype(np.float32) + np.asarray(bias, dtype=np.float32)
    T, E = biased32.shape
    if not 0 < top_k <= E:
        raise ValueError("need 0 < top_k <= n_experts")
    idx = np.broadcast_to(np.arange(E), (T, E))
    # total order: larger biased score first, then lower index
    order = np.lexsort((idx, -biased32.astype(np.float64)), axis=1)
    ids = np.sort(order[:, :top_k], axis=1).astype(np.int32)
    ranked = np.take_along_axis(biased32, order, axis=1).astype(np.float64)
    if top_k < E:
        gap = ranked[:, top_k - 1] - ranked[:, top_k]
    else:
        gap = np.full(T, np.inf)
    sel = np.take_along_axis(scores, ids.astype(np.int64), axis=1)
    weights = sel / sel.sum(axis=1, keepdims=True)
    return {"biased32": biased32, "ids": ids, "weights": weights, "gap": gap}


def route(x_bits, w_router_bits, bias, top_k: int) -> dict:
    """Sigmoid router with selection-only correction bias, top-k, weights normalised to 1.

    Returns logits, scores (float64), biased32 (float32 decision values), ids
    (int32 [T, k], ascending), weights (float64 [T, k]), gap (float64 [T]).
    """
    logits, scores = router_scores(x_bits, w_router_bits)
    return {"logits": logits, "scores": scores, **select_topk(scores, bias, top_k)}


def permute(ids: np.ndarray, n_experts: int) -> dict:
    """Stable counting sort of the pairs p = t*k + j by expert id.

    kimi-k3-mlx README, REAP section (two-bank paragraph): once the pairs are
    sorted by expert index each expert owns a contiguous slice.
    Returns offsets [E+1], sorted_pair [P] (pair at each sorted position),
    pair_pos [P] (sorted position of each pair), counts [E], active (ascending
    ids of experts with at least one pair).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    pair_pos = np.empty(P, dtype=np.int32)
    pair_pos[sorted_pair] = np.arange(P, dtype=np.int32)
    active = np.nonzero(counts)[0].astype(np.int32)
    return {"offsets": offsets.astype(np.int32), "sorted_pair": sorted_pair,
            "pair_pos": pair_pos, "counts": counts, "active": active}


def latent_down(x_bits, w_down_bits) -> np.ndarray:
    """z = x W_down^T (float64).  Stable LatentMoE row; AWQ section (one latent for all experts)."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_down_bits).T


def dequant_expert(raw: dict) -> dict:
    """Dequantise one expert's {w1, w3, w2}_{packed, scale} to float64 [N, K] matrices."""
    return {w: dequant(raw[w + "_packed"], raw[w + "_scale"]) for w in ("w1", "w3", "w2")}


def expert_mlp(z_rows: np.ndarray, deq: dict, beta: float = BETA, beta_lin: float = BETA_LIN):
    """One routed expert on its rows: G = Z W1^T, U = Z W3^T, H = SiTU-GLU(G, U), Y = H W2^T.
    K3 open-artifact audit section 4.3 (shapes); Architecture table, Activation row."""
    G = z_rows @ deq["w1"].T
    U = z_rows @ deq["w3"].T
    H = situ_glu(G, U, beta, beta_lin)
    Y = H @ deq["w2"].T
    return H, Y


class ExpertCache:
    """Dequantised experts on demand.  `fetch(e)` returns the raw checkpoint-layout dict."""

    def __init__(self, fetch, max_items: int = 64):
        self.fetch = fetch
        self.max_items = max_items
        self._d: dict = {}

    def __call__(self, e: int) -> dict:
        e = int(e)
        if e not in self._d:
            if len(self._d) >= self.max_items:
                self._d.pop(next(iter(self._d)))
            self._d[e] = dequant_expert(self.fetch(e))
        return self._d[e]


def routed_experts(z: np.ndarray, ids: np.ndarray, get_expert, n_experts: int,
                   beta: float = BETA, beta_lin: float = BETA_LIN, keep: bool = False, map_fn=map) -> dict:
    """Expert outputs for every pair, laid out in expert-sorted order.

    Returns Y_pair [T, k, L] (un-weighted expert output of each pair) and,
    with keep=True, H_sorted / Y_sorted in sorted-pair order, H_pair
    [T, k, I] in pair order, plus the permutation.  The experts are
    independent; map_fn (default: the builtin map) applies the per-expert
    step to the active experts, so a caller may hand it a thread pool's map
    without changing any arithmetic.
    """
    T, k = ids.shape
    perm = permute(ids, n_experts)
    L = z.shape[1]
    Y_pair = np.zeros((T * k, L))
    H_sorted = H_pair = None
    Y_sorted = np.zeros((T * k, L)) if keep else None
    offs, sp = perm["offsets"], perm["sorted_pair"]

    def one_expert(e):
        rows = sp[offs[e]:offs[e + 1]]
        H, Y = expert_mlp(z[rows // k], get_expert(e), beta, beta_lin)
        return e, rows, H, Y

    for e, rows, H, Y in map_fn(one_expert, perm["active"]):
        Y_pair[rows] = Y
        if keep:
            if H_sorted is None:
                H_sorted = np.zeros((T * k, H.shape[1]))
                H_pair = np.zeros((T * k, H.shape[1]))
            H_sorted[offs[e]:offs[e + 1]] = H
            H_pair[rows] = H
            Y_sorted[offs[e]:offs[e + 1]] = Y
    out = {"Y_pair": Y_pair.reshape(T, k, L), "perm": perm}
    if keep:
        out["H_sorted"] = H_sorted
        out["Y_sorted"] = Y_sorted
        out["H_pair"] = H_pair.reshape(T, k, -1)
    return out


def combine(Y_pair: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """y_t = sum_j w_{t,j} Y_{t,j} in the latent (REAP section, caveat paragraph)."""
    return np.einsum("tk,tkl->tl", weights, Y_pair)


def rmsnorm(y: np.ndarray, gamma_bits, eps: float = RMS_EPS) -> np.ndarray:
    """y / sqrt(mean(y^2) + eps) * gamma, on the combined routed latent."""
    ms = np.mean(y * y, axis=1, keepdims=True)
    return y / np.sqrt(ms + eps) * bf16_to_f64(gamma_bits)


def up_proj(y_n: np.ndarray, w_up_bits) -> np.ndarray:
    return y_n @ bf16_to_f64(w_up_bits).T


def shared_experts(x_bits, sh_gate_bits, sh_up_bits, sh_down_bits, n_shared: int, shared_inter: int,
                   beta: float = BETA, beta_lin: float = BETA_LIN) -> np.ndarray:
    """Sum over the shared experts of SiTU-GLU(x Wg_i^T, x Wu_i^T) Wd_i^T, each expert on its own.
    Architecture table, MoE row (2 shared experts on every token); Porting notes item 3
    (shared experts do not use the latent)."""
    x = bf16_to_f64(x_bits)
    Wg, Wu, Wd = bf16_to_f64(sh_gate_bits), bf16_to_f64(sh_up_bits), bf16_to_f64(sh_down_bits)
    out = np.zeros((x.shape[0], Wd.shape[0]))
    for i in range(n_shared):
        r = slice(i * shared_inter, (i + 1) * shared_inter)
        h = situ_glu(x @ Wg[r].T, x @ Wu[r].T, beta, beta_lin)
        out += h @ Wd[:, r].T
    return out


def layer_forward(x_bits, dense: dict, bias, get_expert, shape, eps: float = RMS_EPS,
                  beta: float = BETA, beta_lin: float = BETA_LIN, keep: bool = False, map_fn=map) -> dict:
    """One forward pass of the layer for the given token rows.

    dense: w_router, w_down, w_up, gamma, sh_gate, sh_up, sh_down (bf16 bits);
    get_expert(e) -> dequantised {w1, w3, w2}.  Every output row depends only
    on its own input row, so any subset of tokens can be evaluated on its own
    (the permutation diagnostics then refer to that subset).  map_fn as for
    routed_experts.
    """
    r = route(x_bits, dense["w_router"], bias, shape.top_k)
    z = latent_down(x_bits, dense["w_down"])
    re = routed_experts(z, r["ids"], get_expert, shape.n_experts, beta, beta_lin, keep=keep, map_fn=map_fn)
    y = combine(re["Y_pair"], r["weights"])
    y_n = rmsnorm(y, dense["gamma"], eps)
    routed = up_proj(y_n, dense["w_up"])
    shared = shared_experts(x_bits, dense["sh_gate"], dense["sh_up"], dense["sh_down"],
                            shape.n_shared, shape.shared_inter, beta, beta_lin)
    out = {"out": routed + shared, "routed": routed, "shared": shared, "z": z, "y": y,
           "y_n": y_n, "perm": re["perm"], **r}
    if keep:
        out["H_sorted"] = re["H_sorted"]
        out["Y_sorted"] = re["Y_sorted"]
        out["Y_pair"] = re["Y_pair"]
        out["H_pair"] = re["H_pair"]
    return out

