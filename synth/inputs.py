"""Seeded synthetic workloads for one Stable LatentMoE layer.

Every tensor has its own numpy PCG64 stream, keyed by a SeedSequence of
(master seed, domain, tensor id, sub-index).  The domain is the weight set for
weights (workloads that share a weight set share every weight byte) and the
workload id for activations.  Routed-expert tensors are keyed per expert, so
any subset of experts can be regenerated on its own.

Storage types follow the checkpoint description in the K3 open-artifact audit
(section 4.3, the MXFP4 routed-expert table): packed e2m1 codes as u8
[N, K/2], e8m0 scales as u8 [N, K/32]; everything else bf16 (kept here as
uint16 bit patterns), the correction bias fp32 (audit section 6).

Recipes (std is the standard deviation of a normal draw, then rounded to bf16
with round-to-nearest-even):
  x ~ N(0, 1); router ~ N(0, router_std); latent down/up projections and
  shared-expert matrices ~ N(0, fan_in**-0.5); RMSNorm gamma = 1;
  packed bytes uniform over 0..255 (so each nibble is uniform over the 16
  codes); scale bytes uniform over the workload's exponent range.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

MASTER_SEED = 0

# stream ids (one per tensor)
T_X, T_ROUTER, T_BIAS, T_DOWN, T_UP = 1, 2, 3, 4, 5
T_SH_GATE, T_SH_UP, T_SH_DOWN = 6, 7, 8
T_W1P, T_W1S, T_W3P, T_W3S, T_W2P, T_W2S = 10, 11, 12, 13, 14, 15
T_ZIPF_PERM, T_MB_COUNTS, T_MB_A = 20, 21, 22
T_GAMMA = 23
# affine 2-bit bank: packed codes, bf16 scales, bf16 biases of w1, w3, w2
T_Q1P, T_Q1S, T_Q1B, T_Q3P, T_Q3S, T_Q3B, T_Q2P, T_Q2S, T_Q2B = 30, 31, 32, 33, 34, 35, 36, 37, 38
T_PAIRED = 39
_WSET_DOMAIN = 1000


@dataclass(frozen=True)
class LayerShape:
    hidden: int        # H, residual width
    latent: int        # L, latent width the routed experts run in
    n_experts: int     # E
    top_k: int         # k
    inter: int         # I, routed-expert intermediate width
    n_shared: int      # S
    shared_inter: int  # Is, intermediate width of one shared expert


# Kimi K3 shapes: kimi-k3-mlx README, Architecture table (MoE and Stable
# LatentMoE rows); K3 open-artifact audit section 4.3 (expert tensor shapes).
K3_SHAPE = LayerShape(7168, 3584, 896, 16, 3072, 2, 3072)
TINY_SHAPE = LayerShape(256, 128, 32, 4, 128, 1, 128)
# The first layer is dense with a bf16 FFN of intermediate 33792 (K3 open-artifact audit section
# 4.1 tensor table: gate/up 33792 x 7168, down 7168 x 33792; findrepo.work summary, architecture
# table, Dense layer row); it runs through the shared-expert call as one expert of that width.
LAYER0_FFN_SHAPE = LayerShape(7168, 3584, 896, 16, 3072, 1, 33792)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    shape: LayerShape
    tokens: int
    wset: int
    router_std: float
    bias_std: float
    bias_mode: str            # "normal" or "zipf"
    exp_lo: int
    exp_hi: int
    zipf_s: float = 1.1
    grouped_only: bool = False  # isolated grouped-GEMM microbenchmark
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", 1, TINY_SHAPE, 8, 1, 0.02, 0.1, "normal", 119, 121,
                     notes="T=8, H=256, L=128, E=32, k=4, I=128, one shared expert"),
    "decode": Workload("decode", 2, K3_SHAPE, 16, 2, 0.01, 0.05, "normal", 118, 120,
                       notes="full K3 shapes, T=16"),
    "batched_decode": Workload("batched_decode", 3, K3_SHAPE, 256, 2, 0.01, 0.05, "zipf", 118, 120,
                               notes="full K3 shapes, T=256, bias calibrated to Zipf(1.1) load"),
    "prefill": Workload("prefill", 4, K3_SHAPE, 4096, 2, 0.01, 0.05, "normal", 118, 120,
                        notes="full K3 shapes, T=4096"),
    "microbench": Workload("microbench", 5, K3_SHAPE, 4096, 2, 0.01, 0.05, "normal", 118, 120,
                           grouped_only=True,
                           notes="isolated grouped GEMM, Multinomial(65536, Zipf(1.1)) segments"),
    # the dense first layer's FFN (intermediate 33792, bf16) as one "shared expert" of width 33792
    "dense_ffn": Workload("dense_ffn", 6, LAYER0_FFN_SHAPE, 4096, 3, 0.01, 0.05, "normal", 118, 120,
                          notes="layer-0 dense FFN, H=7168, intermediate 33792, bf16, T=16 and T=4096"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _stream(domain: int, tid: int, sub: int = 0, seed: int = MASTER_SEED) -> np.random.SeedSequence:
    return np.random.SeedSequence([seed, domain, tid, sub])


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(ss: np.random.SeedSequence, shape, std: float, chunk_rows: int = 0) -> np.ndarray:
    """bf16 bits of N(0, std) draws.  With chunk_rows > 0 the rows are drawn in
    chunks, chunk i from the i-th child stream, so a prefix of rows does not
    depend on the total row count."""
    rows = shape[0]
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    if chunk_rows <= 0:
        v = _rng(ss).standard_normal(rows * cols, dtype=np.float32) * np.float32(std)
        return f32_to_bf16_bits(v).reshape(shape)
    out = np.empty((rows, cols), dtype=np.uint16)
    starts = list(range(0, rows, chunk_rows))
    children = ss.spawn(len(starts))

    def job(i):
        r0 = starts[i]
        r1 = min(rows, r0 + chunk_rows)
        v = _rng(children[i]).standard_normal((r1 - r0) * cols, dtype=np.float32) * np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(v).reshape(r1 - r0, cols)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(len(starts))))
    return out.reshape(shape)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_tokens(wl: Workload, tokens: int | None = None) -> np.ndarray:
    """x: bf16 bits [T, H], N(0, 1)."""
    T = wl.tokens if tokens is None else tokens
    return _normal_bf16(_stream(wl.cfg_id, T_X), (T, wl.shape.hidden), 1.0, chunk_rows=1024)


def gen_dense(wl: Workload) -> dict:
    """Router, latent projections, RMSNorm gamma and shared experts (bf16 bits).

    Shared experts are returned concatenated: gate/up rows [S*Is, H] (expert i
    owns rows i*Is..(i+1)*Is), down columns [H, S*Is] (same split).
    """
    sh = wl.shape
    d = _WSET_DOMAIN + wl.wset
    H, L, E, S, Is = sh.hidden, sh.latent, sh.n_experts, sh.n_shared, sh.shared_inter
    out = {
        "w_router": _normal_bf16(_stream(d, T_ROUTER), (E, H), wl.router_std, chunk_rows=256),
        "w_down": _normal_bf16(_stream(d, T_DOWN), (L, H), H ** -0.5, chunk_rows=512),
        "w_up": _normal_bf16(_stream(d, T_UP), (H, L), L ** -0.5, chunk_rows=512),
        "gamma": np.full((L,), 0x3F80, dtype=np.uint16),
    }
    gate = np.empty((S * Is, H), np.uint16)
    up = np.empty((S * Is, H), np.uint16)
    down = np.empty((H, S * Is), np.uint16)
    for i in range(S):
        gate[i * Is:(i + 1) * Is] = _normal_bf16(_stream(d, T_SH_GATE, i), (Is, H), H ** -0.5, chunk_rows=512)
        up[i * Is:(i + 1) * Is] = _normal_bf16(_stream(d, T_SH_UP, i), (Is, H), H ** -0.5, chunk_rows=512)
        down[:, i * Is:(i + 1) * Is] = _normal_bf16(_stream(d, T_SH_DOWN, i), (H, Is), Is ** -0.5, chunk_rows=512)
    out["sh_gate"], out["sh_up"], out["sh_down"] = gate, up, down
    return out


def gen_gamma_random(wl: Workload, std: float = 0.1) -> np.ndarray:
    """A non-trivial RMSNorm weight for diagnostics: bf16 bits of 1 + N(0, std), [L]."""
    ss = _stream(_WSET_DOMAIN + wl.wset, T_GAMMA)
    v = 1.0 + std * _rng(ss).standard_normal(wl.shape.latent)
    return f32_to_bf16_bits(v.astype(np.float32))


def gen_bias(wl: Workload, zipf_bias_path: str | None = None) -> np.ndarray:
    """Correction bias fp32 [E].  "normal": N(0, bias_std), part of the weight set.
    "zipf": read from the calibration file (one fp32 value per line)."""
    if wl.bias_mode == "zipf":
        if zipf_bias_path is None:
            raise ValueError("zipf-calibrated bias needs the calibration file path")
        vals = np.loadtxt(zipf_bias_path, dtype=np.float64)
        if vals.shape != (wl.shape.n_experts,):
            raise ValueError(f"bias file has shape {vals.shape}")
        return vals.astype(np.float32)
    d = _WSET_DOMAIN + wl.wset
    return (_rng(_stream(d, T_BIAS)).standard_normal(wl.shape.n_experts) * wl.bias_std).astype(np.float32)


def _expert_dims(sh: LayerShape, which: str):
    if which in ("w1", "w3"):
        return sh.inter, sh.latent
    if which == "w2":
        return sh.latent, sh.inter
    raise ValueError(which)


_TIDS = {"w1": (T_W1P, T_W1S), "w3": (T_W3P, T_W3S), "w2": (T_W2P, T_W2S)}


def gen_expert(wl: Workload, e: int, which: str, out_packed=None, out_scale=None):
    """One expert matrix in checkpoint layout: packed u8 [N, K/2], scale u8 [N, K/32].

    Packed bytes are the raw little-endian bytes of PCG64 64-bit outputs;
    scale bytes are uniform integers in [exp_lo, exp_hi].
    """
    N, K = _expert_dims(wl.shape, which)
    d = _WSET_DOMAIN + wl.wset
    tp, ts = _TIDS[which]
    nbytes = N * K // 2
    bg = np.random.PCG64(_stream(d, tp, e))
    raw = bg.random_raw((nbytes + 7) // 8).view(np.uint8)[:nbytes].reshape(N, K // 2)
    sc = _rng(_stream(d, ts, e)).integers(wl.exp_lo, wl.exp_hi + 1, size=(N, K // 32), dtype=np.uint8)
    if out_packed is not None:
        out_packed[...] = raw
        out_scale[...] = sc
        return out_packed, out_scale
    return raw, sc


def gen_expert_stack(wl: Workload, experts=None, out: dict | None = None) -> dict:
    """Stacked expert tensors {w1,w3,w2}_{packed,scale} [n, N, K/2] / [n, N, K/32] for the
    listed experts (default: all), generated in parallel threads."""
    sh = wl.shape
    ids = list(range(sh.n_experts)) if experts is None else list(experts)
    n = len(ids)
    if out is None:
        out = {}
        for w in ("w1", "w3", "w2"):
            N, K = _expert_dims(sh, w)
            out[w + "_packed"] = np.empty((n, N, K // 2), np.uint8)
            out[w + "_scale"] = np.empty((n, N, K // 32), np.uint8)

    def job(i):
        for w in ("w1", "w3", "w2"):
            gen_expert(wl, ids[i], w, out[w + "_packed"][i], out[w + "_scale"][i])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(n)))
    return out


def zipf_probabilities(n: int, s: float) -> np.ndarray:
    """p_r = r^-s / sum_{j<=n} j^-s for ranks r = 1..n."""
    r = np.arange(1, n + 1, dtype=np.float64)
    w = r ** (-s)
    return w / w.sum()


def zipf_permutation(wl: Workload) -> np.ndarray:
    """Seeded permutation: expert perm[r-1] holds Zipf rank r."""
    return _rng(_stream(wl.cfg_id, T_ZIPF_PERM)).permutation(wl.shape.n_experts)


def gen_microbench_counts(wl: Workload) -> np.ndarray:
    """Per-expert row counts ~ Multinomial(T*k, Zipf(s) over a seeded permutation)."""
    E = wl.shape.n_experts
    p_rank = zipf_probabilities(E, wl.zipf_s)
    perm = zipf_permutation(wl)
    p = np.empty(E)
    p[perm] = p_rank
    return _rng(_stream(wl.cfg_id, T_MB_COUNTS)).multinomial(wl.tokens * wl.shape.top_k, p).astype(np.int64)


def gen_microbench_activations(wl: Workload, rows: int | None = None) -> np.ndarray:
    """A: bf16 bits [P, L] of N(0, 1), already in expert-sorted row order."""
    P = wl.tokens * wl.shape.top_k if rows is None else rows
    return _normal_bf16(_stream(wl.cfg_id, T_MB_A), (P, wl.shape.latent), 1.0, chunk_rows=2048)


_QTIDS = {"w1": (T_Q1P, T_Q1S, T_Q1B), "w3": (T_Q3P, T_Q3S, T_Q3B), "w2": (T_Q2P, T_Q2S, T_Q2B)}
AFFINE_GROUP = 64


def gen_expert_affine2(wl: Workload, e: int, which: str):
    """One expert matrix of the affine 2-bit bank: packed u8 [N, K/4] (raw
    PCG64 bytes, so every 2-bit code is uniform over 0..3), bf16 scales and
    biases [N, K/64].  scale = 2^-7 * U[0.5, 1.5), bias = -1.5 * scale *
    U[0.8, 1.2) (each rounded to bf16): the grid scale * q + bias then spans
    about [-1.5, 1.5] scales, the magnitude of the MXFP4 experts' weights."""
    N, K = _expert_dims(wl.shape, which)
    d = _WSET_DOMAIN + wl.wset
    tp, ts, tb = _QTIDS[which]
    nbytes = N * K // 4
    raw = np.random.PCG64(_stream(d, tp, e)).random_raw((nbytes + 7) // 8).view(np.uint8)[:nbytes].reshape(N, K // 4)
    G = K // AFFINE_GROUP
    sc = np.float32(2.0 ** -7) * _rng(_stream(d, ts, e)).uniform(0.5, 1.5, size=(N, G)).astype(np.float32)
    sc_bits = f32_to_bf16_bits(sc)
    sc_r = bf16_bits_to_f32(sc_bits)
    bi = np.float32(-1.5) * sc_r * _rng(_stream(d, tb, e)).uniform(0.8, 1.2, size=(N, G)).astype(np.float32)
    return raw, sc_bits, f32_to_bf16_bits(bi)


def gen_expert_affine2_stack(wl: Workload, experts) -> dict:
    """Stacked affine-bank tensors {w1,w3,w2}_{packed,scale,bias} for the listed experts."""
    ids = list(experts)
    out = {}
    for w in ("w1", "w3", "w2"):
        N, K = _expert_dims(wl.shape, w)
        out[w + "_packed"] = np.empty((len(ids), N, K // 4), np.uint8)
        out[w + "_scale"] = np.empty((len(ids), N, K // AFFINE_GROUP), np.uint16)
        out[w + "_bias"] = np.empty((len(ids), N, K // AFFINE_GROUP), np.uint16)

    def job(i):
        for w in ("w1", "w3", "w2"):
            p, s_, b = gen_expert_affine2(wl, ids[i], w)
            out[w + "_packed"][i], out[w + "_scale"][i], out[w + "_bias"][i] = p, s_, b

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(len(ids))))
    return out


def gen_expert_paired(wl: Workload, e: int, which: str) -> dict:
    """The same weight matrix in both bank formats.  Every element is
    c * 2^(x - 127) with c in {0, 0.5, 1, 1.5} (e2m1 codes 0..3) and one
    exponent x in [exp_lo, exp_hi] per group of 64; MXFP4: those codes with
    e8m0 scale x for both 32-blocks of the group; affine 2-bit: code q = c / 0.5
    (the same code value), scale 2^(x - 128) as a bf16 (exponent field x - 1,
    no mantissa), bias 0.  Returns {fp4_packed, fp4_scale, q2_packed,
    q2_scale, q2_bias}."""
    N, K = _expert_dims(wl.shape, which)
    d = _WSET_DOMAIN + wl.wset
    rng = _rng(_stream(d, T_PAIRED, e * 3 + {"w1": 0, "w3": 1, "w2": 2}[which]))
    codes = rng.integers(0, 4, size=(N, K), dtype=np.uint8)
    x = rng.integers(wl.exp_lo, wl.exp_hi + 1, size=(N, K // AFFINE_GROUP), dtype=np.uint8)
    fp4 = (codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))).astype(np.uint8)
    q2 = (codes[:, 0::4] | (codes[:, 1::4] << np.uint8(2)) | (codes[:, 2::4] << np.uint8(4))
          | (codes[:, 3::4] << np.uint8(6))).astype(np.uint8)
    return {"fp4_packed": fp4, "fp4_scale": np.repeat(x, 2, axis=1),
            "q2_packed": q2, "q2_scale": ((x.astype(np.uint16) - 1) << np.uint16(7)).astype(np.uint16),
            "q2_bias": np.zeros((N, K // AFFINE_GROUP), np.uint16)}
