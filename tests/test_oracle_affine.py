"""Pins of the affine low-bit bank and the two-bank expert lookup (oracle/affine.py).

Each checks the oracle against something other than itself: the pages'
printed bpw and tier sizes, an independent scalar decode, the MXFP4 oracle on
values both formats hold exactly, and the single-bank layer.
"""
import json
import os
import struct

import numpy as np
import pytest

import synth
from oracle import affine, layer, mxfp4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "k3_printed_numbers.json")


def _printed():
    return {k: v["value"] for k, v in json.load(open(GOLDEN)).items() if not k.startswith("_")}


def test_bpw_and_tier_size_closures():
    """bits + two 16-bit parameters per 64 elements gives the printed 2.50 / 3.50 /
    4.5 bpw, and the printed tier sizes follow from the routed-expert parameter
    count: experts at the tier's bpw plus the non-expert rest (115 GB in bf16,
    or 4-bit affine at 4.5 bpw)."""
    P = _printed()
    for bits, bpw in P["affine_bpw_by_bits"].items():
        assert int(bits) + 2 * 16 / affine.GROUP == bpw
    assert affine.BITS + 2 * 16 / affine.GROUP == P["affine_bpw_by_bits"]["2"]
    routed = 2_722_740_830_208
    rest_bf16 = P["mxfp4_tier_rest_gb"] * 1e9
    rest_4bit = rest_bf16 * 4.5 / 16
    sizes = P["tier_sizes_tb"]
    assert round((routed * 4.25 / 8 + rest_bf16) / 1e12, 2) == sizes["mxfp4"]
    assert round((routed * 3.5 / 8 + rest_4bit) / 1e12, 2) == sizes["3bit"]
    assert round((routed * 2.5 / 8 + rest_bf16) / 1e12, 2) == sizes["mixed2"]
    assert round((routed * 2.5 / 8 + rest_4bit) / 1e12, 2) == sizes["2bit"]
    # the two-bank memory figure: 392 of 896 experts in the 2-bit bank at the same expert count
    assert round((504 * 4.25 + 392 * 2.5) / (896 * 4.25), 2) == P["two_bank_memory_same_experts"]


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def test_dequant_all_bytes_against_scalar_decode():
    """Every byte value in every position of a group, with sampled bf16 scales and
    biases, against a per-element decode written with Python integers."""
    rng = np.random.default_rng(4)
    packed = np.arange(256, dtype=np.uint8).reshape(16, 16)  # 16 rows x 64 elements: one group each
    scale = synth.f32_to_bf16_bits(rng.uniform(-2, 2, (16, 1)).astype(np.float32) * np.float32(2.0 ** -6))
    bias = synth.f32_to_bf16_bits(rng.standard_normal((16, 1)).astype(np.float32) * np.float32(0.01))
    got = affine.dequant_affine2(packed, scale, bias)
    for n in range(16):
        for k in range(64):
            byte = int(packed[n, k // 4])
            q = (byte >> (2 * (k % 4))) & 3
            want = q * _bf16(scale[n, 0]) + _bf16(bias[n, 0])
            assert got[n, k] == want


def test_scale_and_bias_groups_of_64():
    """Element k of a row takes group k // 64: a one-hot scale or bias moves exactly that group."""
    packed = np.full((2, 64), 0xFF, np.uint8)  # every code 3, K = 256: four groups
    for g in range(4):
        scale = np.zeros((2, 4), np.uint16)
        scale[:, g] = 0x3F80  # 1.0
        w = affine.dequant_affine2(packed, scale, np.zeros((2, 4), np.uint16))
        assert (w[:, 64 * g:64 * (g + 1)] == 3.0).all() and np.count_nonzero(w) == 2 * 64
        bias = np.zeros((2, 4), np.uint16)
        bias[:, g] = 0xBF80  # -1.0
        w = affine.dequant_affine2(packed, np.zeros((2, 4), np.uint16), bias)
        assert (w[:, 64 * g:64 * (g + 1)] == -1.0).all() and np.count_nonzero(w) == 2 * 64


def test_unpack_inverts_integer_packing():
    """Codes packed as sum q_i 4^i (element 4b + i in bits 2i..2i+1 of byte b) unpack to themselves."""
    rng = np.random.default_rng(7)
    q = rng.integers(0, 4, size=(5, 96))
    packed = np.array([[sum(int(q[r, 4 * b + i]) * 4 ** i for i in range(4)) for b in range(24)] for r in range(5)],
                      dtype=np.uint8)
    assert (affine.unpack_q2(packed) == q).all()


def test_paired_encodings_dequantize_identically():
    """The generator's paired MXFP4 / affine encodings hold the same values, as both
    oracles read them: codes 0..3 with e8m0 x equal q * 2^(x - 128) + 0."""
    wl = synth.workload("tiny")
    for which in ("w1", "w3", "w2"):
        pr = synth.gen_expert_paired(wl, 3, which)
        a = mxfp4.dequant(pr["fp4_packed"], pr["fp4_scale"])
        b = affine.dequant_affine2(pr["q2_packed"], pr["q2_scale"], pr["q2_bias"])
        assert np.array_equal(a, b)
        assert (a >= 0).all() and len(np.unique(a)) > 4


def test_two_bank_equal_values_match_single_bank():
    """A two-bank layer whose bank B holds, in the affine format, exactly the
    values bank A would hold gives the single-bank layer's output bit for bit
    (README, REAP section, two-bank paragraph: equal weights must reproduce the
    plain expert layer exactly)."""
    wl = synth.workload("tiny")
    sh = wl.shape
    x, d, b = synth.gen_tokens(wl), synth.gen_dense(wl), synth.gen_bias(wl)
    pairs = {e: {w: synth.gen_expert_paired(wl, e, w) for w in ("w1", "w3", "w2")} for e in range(sh.n_experts)}
    fp4 = lambda e: {w: mxfp4.dequant(pairs[e][w]["fp4_packed"], pairs[e][w]["fp4_scale"])  # noqa: E731
                     for w in ("w1", "w3", "w2")}
    q2 = lambda e: affine.dequant_expert_affine2({f"{w}_{k}": pairs[e][w][f"q2_{k}"]  # noqa: E731
                                                  for w in ("w1", "w3", "w2") for k in ("packed", "scale", "bias")})
    single = layer.layer_forward(x, d, b, fp4, sh, keep=True)
    n_a = 13
    two = layer.layer_forward(x, d, b, affine.two_bank_expert(fp4, lambda i: q2(i + n_a), n_a), sh, keep=True)
    for key in ("out", "H_sorted", "Y_sorted"):
        assert np.array_equal(single[key], two[key]), key


def test_two_bank_lookup_routes_by_index_range():
    """Experts below the split come from bank A, the rest from bank B re-indexed from 0."""
    seen = []
    get = affine.two_bank_expert(lambda e: ("A", e), lambda i: ("B", i), 5)
    for e in (0, 4, 5, 9):
        seen.append(get(e))
    assert seen == [("A", 0), ("A", 4), ("B", 0), ("B", 4)]
