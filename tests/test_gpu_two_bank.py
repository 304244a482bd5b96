"""Two-bank grouped GEMM (moe_grouped_gemm_two_bank) on the GPU through the C ABI.

kimi-k3-mlx README, REAP section, two-bank paragraph: one sorted pair list,
each bank computing only its own contiguous slice of the sorted rows; with the
two banks given the same weights and precision the result must match the
plain expert layer exactly.  Here the split point is read on the device.

A mid-size shape keeps the oracle fast while the affine path meets its limits
(K a multiple of 512, at least 1536 at decode sizes): H 2048, L 2048, E 64,
top-4, I 1536, one shared expert of 512.  T = 16 runs the decode kernel
(P < 2E), T = 256 the prefill kernel.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from synth.device import to_dev, to_dev_bf16, upload_tokens, upload_weights
from oracle import affine, layer, mxfp4
from gpu_common import TOL, check_routing, rel_max_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

MID = synth.LayerShape(2048, 2048, 64, 4, 1536, 1, 512)
N_A = 24  # experts 0..23 in bank A (MXFP4), 24..63 in bank B


def _wl(T):
    return synth.Workload(f"twobank{T}", 13, MID, T, 13, 0.02, 0.1, "normal", 119, 121)


@pytest.fixture(scope="module")
def mx():
    import mxfp4_latent_moe_amd as m
    m.load()
    return m


def _affine_bank(wl, experts):
    st = synth.gen_expert_affine2_stack(wl, experts)
    return {k: to_dev(v, DEV) for k, v in st.items()}


def _routing(mx, wl, w, x):
    from mxfp4_latent_moe_amd import ops
    s = mx.shape_of(wl.shape)
    T = x.shape[0]
    moe = mx.LatentMoE(s, w, DEV, h_planes=False)
    b = moe.forward(x)
    torch.cuda.synchronize()
    return s, b, T * wl.shape.top_k


@pytest.mark.parametrize("T", [16, 256])
@pytest.mark.parametrize("n_a", [N_A, 0, 64])
def test_same_format_banks_bitwise(mx, T, n_a):
    """Both banks MXFP4, holding experts [0, n_a) and [n_a, 64) of the same stack:
    H and Y bitwise equal to mxfp4_grouped_gemm's, also with one bank empty."""
    from mxfp4_latent_moe_amd import _lib, ops
    wl = _wl(T)
    w = upload_weights(wl, DEV)
    x = upload_tokens(wl, DEV)
    s, b, P = _routing(mx, wl, w, x)
    say(f"case: two MXFP4 banks, split at {n_a}, T={T}")
    ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_GROUPED_GEMM_TWO_BANK, P), dtype=torch.uint8, device=DEV)
    H = torch.empty_like(b["H"])
    Y = torch.empty_like(b["Y"])
    hi = {k: v[n_a:] for k, v in w.items() if k[:2] in ("w1", "w3", "w2")}
    for op, A, C in ((ops.MOE_OP_GATEUP_SITU, b["z"], H), (ops.MOE_OP_DOWN, H, Y)):
        ba = ops.expert_bank(_lib.MOE_WF_MXFP4, n_a, w, op)
        bb = ops.expert_bank(_lib.MOE_WF_MXFP4, MID.n_experts - n_a, hi, op)
        ops.grouped_gemm_two_bank(s, op, P, b["offsets"], b["sorted_pair"], A, ba, bb, None, C, ws)
    torch.cuda.synchronize()
    assert torch.equal(H, b["H"]) and torch.equal(Y, b["Y"])


@pytest.mark.parametrize("T", [16, 256])
def test_affine_bank_on_paired_values(mx, T):
    """Bank B in the affine format holding exactly the values that the MXFP4
    encoding of the same experts holds (codes 0..3, power-of-two scales, zero
    bias): the two-bank H and Y equal the single MXFP4 bank's to fp32 rounding
    (the products are the same; the affine path sums each 64-element group
    on its own before scaling it, so only the order of the additions differs),
    and the layer output too."""
    from mxfp4_latent_moe_amd import _lib, ops
    wl = _wl(T)
    w = upload_weights(wl, DEV, experts=False)
    E = MID.n_experts
    paired = {e: {m: synth.gen_expert_paired(wl, e, m) for m in ("w1", "w3", "w2")} for e in range(E)}
    for m in ("w1", "w3", "w2"):
        w[m + "_packed"] = to_dev(np.stack([paired[e][m]["fp4_packed"] for e in range(E)]), DEV)
        w[m + "_scale"] = to_dev(np.stack([paired[e][m]["fp4_scale"] for e in range(E)]), DEV)
    bank_b = {"format": _lib.MOE_WF_AFFINE2, "n_experts": E - N_A}
    for m in ("w1", "w3", "w2"):
        for k in ("packed", "scale", "bias"):
            bank_b[f"{m}_{k}"] = to_dev(np.stack([paired[e][m][f"q2_{k}"] for e in range(N_A, E)]), DEV)
    x = upload_tokens(wl, DEV)
    s = mx.shape_of(MID)
    say(f"case: affine bank B on paired values, T={T}")
    single = {k: v.clone() for k, v in mx.LatentMoE(s, w, DEV, h_planes=False).forward(x).items()}
    two = mx.LatentMoE(s, {k: (v[:N_A] if k[:2] in ("w1", "w3", "w2") else v) for k, v in w.items()}, DEV,
                       bank_b=bank_b).forward(x)
    torch.cuda.synchronize()
    assert torch.equal(two["topk_ids"], single["topk_ids"]) and torch.equal(two["sorted_pair"], single["sorted_pair"])
    eh = rel_max_err(two["H"].cpu().numpy(), single["H"].cpu().numpy())
    ey = rel_max_err(two["Y"].cpu().numpy(), single["Y"].cpu().numpy())
    eo = rel_max_err(two["out"].cpu().numpy(), single["out"].cpu().numpy())
    say(f"paired T={T}: H {eh:.2e} Y {ey:.2e} out {eo:.2e}; bitwise H {torch.equal(two['H'], single['H'])}")
    assert eh < 1e-4 and ey < 1e-4 and eo < 1e-4


@pytest.mark.parametrize("T", [16, 256])
def test_two_bank_layer_against_oracle(mx, T):
    """The two-bank layer (experts 0..23 MXFP4, 24..63 affine 2-bit with random
    codes, scales and biases) against the oracle's layer with the two-bank
    expert lookup: ids exact outside near-ties; the output, and H and Y of
    every pair, within 1e-3 of the oracle's rms (the affine codes are exact
    and their scales and biases are applied in fp32, so the error is the
    fp32 accumulation's: measured 3e-5 to 1.2e-4)."""
    from mxfp4_latent_moe_amd import _lib
    wl = _wl(T)
    w = upload_weights(wl, DEV)
    E = MID.n_experts
    bank_b = {"format": _lib.MOE_WF_AFFINE2, "n_experts": E - N_A, **_affine_bank(wl, range(N_A, E))}
    wa = {k: (v[:N_A] if k[:2] in ("w1", "w3", "w2") else v) for k, v in w.items()}
    x_bits = synth.gen_tokens(wl)
    say(f"case: two-bank layer vs oracle, T={T}")
    g = mx.LatentMoE(mx.shape_of(MID), wa, DEV, bank_b=bank_b).forward(to_dev_bf16(x_bits, DEV))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items() if k not in ("ws", "ws_shared")}
    st = synth.gen_expert_stack(wl, range(N_A))
    aff = synth.gen_expert_affine2_stack(wl, range(N_A, E))
    get_a = lambda e: layer.dequant_expert({k: v[e] for k, v in st.items()})  # noqa: E731
    get_b = lambda i: affine.dequant_expert_affine2({k: v[i] for k, v in aff.items()})  # noqa: E731
    d = synth.gen_dense(wl)
    bias = synth.gen_bias(wl)
    r = layer.layer_forward(x_bits, d, bias, affine.two_bank_expert(get_a, get_b, N_A), MID, keep=True)
    excl = check_routing(g["topk_ids"], g["topk_w"], r)
    same = (g["topk_ids"] == r["ids"]).all(axis=1)
    k = MID.top_k
    pp = g["pair_pos"].reshape(-1, k)[same].reshape(-1)
    errH = rel_max_err(g["H"][pp], r["H_pair"][same].reshape(pp.size, -1))
    errY = rel_max_err(g["Y"][pp], r["Y_pair"][same].reshape(pp.size, -1))
    err = rel_max_err(g["out"][same], r["out"][same])
    # the affine bank alone: pairs routed to experts >= N_A
    bpairs = (g["topk_ids"][same] >= N_A).reshape(-1)
    errHb = rel_max_err(g["H"][pp[bpairs]], r["H_pair"][same].reshape(pp.size, -1)[bpairs])
    say(f"two-bank T={T}: excluded {excl.size}; H {errH:.2e} (affine pairs {errHb:.2e}), Y {errY:.2e}, out {err:.2e}")
    assert err <= TOL and err < 1e-3 and errH < 1e-3 and errY < 1e-3
