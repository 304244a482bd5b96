"""Affine low-bit expert bank and the two-bank expert lookup, float64 (test infrastructure only).

Passages followed:
  * kimi-k3-mlx README, Tiers section: the lossy tiers re-quantize the MXFP4
    experts onto MLX's affine grid (2bit and mixed2: 2.50 expert bpw; 3bit:
    3.50; affine 4-bit: 4.5 bpw).
  * Kimi-K3-Alis-MLX-Dynamic card, "Why promotion instead of higher affine
    precision": the affine grid is uniform, with a scale and a bias.
  * kimi-k3-mlx README, REAP section, graded-plan and two-bank paragraphs:
    the graded plan keeps the most salient experts in MXFP4 and stores the
    middle ones at a lower width; MLX fixes one width per expert tensor, so the
    two widths live in two banks; once the pairs are sorted by expert index,
    the bank that owns a contiguous range of expert indices owns a contiguous
    slice of the sorted pairs.

Readings (the pages give the bpw figures, not the layout):
  * element value = scale * q + bias, q an unsigned code 0 .. 2^bits - 1;
  * one bf16 scale and one bf16 bias per group of 64 consecutive input
    elements of a row: bits + 2 * 16 / 64 gives the printed 2.50 / 3.50 / 4.5
    bpw (the closures in the pins);
  * bits = 2 for the low bank (the 2-bit tier); codes packed low bits first,
    element 4b + i of a row in bits 2i .. 2i + 1 of byte b (the same
    low-bits-first order as the MXFP4 codes);
  * bank A (MXFP4) owns experts 0 .. n_bank_a - 1, bank B (affine) owns
    n_bank_a .. E - 1, its tensors indexed from 0.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
BITS = 2


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def unpack_q2(packed: np.ndarray) -> np.ndarray:
    """u8 [..., K/4] -> 2-bit codes u8 [..., K]; element 4b + i sits in bits 2i .. 2i+1 of byte b."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (packed.shape[-1] * 4,), dtype=np.uint8)
    for i in range(4):
        codes[..., i::4] = (packed >> np.uint8(2 * i)) & np.uint8(3)
    return codes


def dequant_affine2(packed: np.ndarray, scale_bits: np.ndarray, bias_bits: np.ndarray) -> np.ndarray:
    """Affine 2-bit weights float64 [..., N, K] = scale[n, k // 64] * q + bias[n, k // 64]."""
    q = unpack_q2(packed).astype(np.float64)
    K = q.shape[-1]
    if scale_bits.shape[-1] * GROUP != K or bias_bits.shape != scale_bits.shape:
        raise ValueError(f"scale/bias groups {scale_bits.shape} do not match K={K}")
    s = np.repeat(bf16_to_f64(scale_bits), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(bias_bits), GROUP, axis=-1)
    return q * s + b


def dequant_expert_affine2(raw: dict) -> dict:
    """One affine expert {w1, w3, w2}_{packed, scale, bias} -> float64 [N, K] matrices."""
    return {w: dequant_affine2(raw[w + "_packed"], raw[w + "_scale"], raw[w + "_bias"]) for w in ("w1", "w3", "w2")}


def two_bank_expert(get_a, get_b, n_bank_a: int):
    """Expert lookup of a two-bank layer: e < n_bank_a from bank A (get_a(e)),
    the rest from bank B (get_b(e - n_bank_a)); both return dequantised
    {w1, w3, w2}."""
    def get(e):
        e = int(e)
        return get_a(e) if e < n_bank_a else get_b(e - n_bank_a)
    return get
