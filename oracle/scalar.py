"""A second, structurally different oracle for tiny shapes (test infrastructure only).

Plain Python loops, one token and one (token, expert) pair at a time: no
permutation, no matrix library, its own bit-level e2m1 decoding.  It follows
the same passages as `oracle.layer` (kimi-k3-mlx README Architecture table,
Porting notes, Tiers and REAP sections; K3 open-artifact audit sections 4.3
and 6) and exists so that a slip in one of the two oracles shows up as a
disagreement between them.  Only for tiny shapes: its cost is a few million
Python multiply-adds.
"""
from __future__ import annotations

import math
import struct


def _f32(v: float) -> float:
    """Round a Python float to the nearest float32 value."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e2m1_decode(code: int) -> float:
    """OCP MX e2m1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
    exponent field 0 is subnormal (mantissa * 0.5)."""
    sign = -1.0 if code & 8 else 1.0
    ex = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if ex == 0 else math.ldexp(1.0 + 0.5 * m, ex - 1)
    return sign * mag


def _weight(packed_row, scale_row, kidx: int) -> float:
    byte = int(packed_row[kidx // 2])
    code = (byte >> 4) if (kidx & 1) else (byte & 15)
    return e2m1_decode(code) * math.ldexp(1.0, int(scale_row[kidx // 32]) - 127)


def _dot(a, b) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def _situ(g: float, u: float, beta: float, beta_lin: float) -> float:
    return beta * math.tanh(g / beta) * (1.0 / (1.0 + math.exp(-g))) * beta_lin * math.tanh(u / beta_lin)


def layer_forward_token(x_row, dense, bias, experts, shape, eps=1e-6, beta=4.0, beta_lin=25.0):
    """Output row (list of H floats) and routing (ids, weights) for one token.

    x_row: H bf16 bit patterns.  dense: bf16-bit matrices as nested sequences.
    experts: experts[e][w] with w in {w1, w3, w2} -> (packed [N][K/2], scale [N][K/32]).
    """
    H, L, E, k = shape.hidden, shape.latent, shape.n_experts, shape.top_k
    I, S, Is = shape.inter, shape.n_shared, shape.shared_inter
    x = [_bf16(v) for v in x_row]

    # router: sigmoid scores, float32 decision values, lowest index wins ties
    scores = []
    dec = []
    for e in range(E):
        s = 1.0 / (1.0 + math.exp(-_dot(x, [_bf16(v) for v in dense["w_router"][e]])))
        scores.append(s)
        dec.append(_f32(_f32(s) + _f32(float(bias[e]))))
    ranked = sorted(range(E), key=lambda e: (-dec[e], e))
    ids = sorted(ranked[:k])
    tot = math.fsum(scores[e] for e in ids)
    wts = [scores[e] / tot for e in ids]

    # latent down projection
    z = [_dot(x, [_bf16(v) for v in dense["w_down"][c]]) for c in range(L)]

    # routed experts, one pair at a time, combined by weight
    y = [0.0] * L
    for e, w in zip(ids, wts):
        w1p, w1s = experts[e]["w1"]
        w3p, w3s = experts[e]["w3"]
        w2p, w2s = experts[e]["w2"]
        h = []
        for i in range(I):
            g = math.fsum(z[c] * _weight(w1p[i], w1s[i], c) for c in range(L))
            u = math.fsum(z[c] * _weight(w3p[i], w3s[i], c) for c in range(L))
            h.append(_situ(g, u, beta, beta_lin))
        for c in range(L):
            yc = math.fsum(h[i] * _weight(w2p[c], w2s[c], i) for i in range(I))
            y[c] += w * yc

    # RMSNorm on the combined latent, then up_proj
    rms = math.sqrt(math.fsum(v * v for v in y) / L + eps)
    gamma = [_bf16(v) for v in dense["gamma"]]
    yn = [y[c] / rms * gamma[c] for c in range(L)]
    out = [_dot(yn, [_bf16(v) for v in dense["w_up"][hh]]) for hh in range(H)]

    # shared experts on x, added after up_proj
    for s_i in range(S):
        hs = []
        for i in range(s_i * Is, (s_i + 1) * Is):
            g = _dot(x, [_bf16(v) for v in dense["sh_gate"][i]])
            u = _dot(x, [_bf16(v) for v in dense["sh_up"][i]])
            hs.append(_situ(g, u, beta, beta_lin))
        for hh in range(H):
            row = dense["sh_down"][hh]
            out[hh] += math.fsum(hs[i] * _bf16(row[s_i * Is + i]) for i in range(Is))
    return out, ids, wts
