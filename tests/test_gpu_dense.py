"""Parity of the dense products through the C ABI.

A mid-size layer shape keeps the oracle fast while the dense products still
take the tiled kernel: T = 1100 tokens are four whole 256-token tiles and a
ragged one of 76, the weight tiles leave CUs idle so K is split (partial sums
and the finalize pass), and two shared experts check the concatenated GLU.
At decode-sized token counts (T <= 64) the same products run on the
persistent streaming kernel, checked at T = 1, 17 and 64.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from synth.device import to_dev, to_dev_bf16
from oracle import layer
from gpu_common import GAP_EXCLUDE, rel_max_err, say

pytestmark = pytest.mark.gpu

MID_SHAPE = synth.LayerShape(1024, 512, 64, 4, 256, 2, 384)
MID = synth.Workload("mid1100", 12, MID_SHAPE, 1100, 12, 0.02, 0.1, "normal", 119, 121)


@pytest.fixture(scope="module")
def mx():
    import mxfp4_latent_moe_amd as m
    m.load()
    return m


def _shape(mx, operand_mode):
    s = MID_SHAPE
    return mx.make_shape(s.hidden, s.latent, s.n_experts, s.top_k, s.inter, s.n_shared, s.shared_inter,
                         operand_mode=operand_mode)


@pytest.mark.parametrize("mode,tol", [(0, 1e-4), (1, 1e-2)])
def test_shared_expert_ffn_tiled(mx, mode, tol):
    """out = out0 + SiTU(x Wg^T, x Wu^T) Wd^T for both operand modes (hi+lo, rounded)."""
    from mxfp4_latent_moe_amd import _lib, ops
    dev = torch.device("cuda:0")
    s = MID_SHAPE
    T = MID.tokens
    x_bits = synth.gen_tokens(MID)
    d = synth.gen_dense(MID)
    out0 = np.random.default_rng(5).standard_normal((T, s.hidden)).astype(np.float32)
    say(f"case: shared_expert_ffn T={T} H={s.hidden} S*Is={s.n_shared * s.shared_inter} mode {mode}")
    sh = _shape(mx, mode)
    ws = torch.empty(ops.workspace_bytes(sh, _lib.MOE_FN_SHARED_FFN, T), dtype=torch.uint8, device=dev)
    out = to_dev(out0, dev)
    ops.shared_ffn(sh, to_dev_bf16(x_bits, dev), to_dev_bf16(d["sh_gate"], dev), to_dev_bf16(d["sh_up"], dev),
                   to_dev_bf16(d["sh_down"], dev), out, 1, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64) - out0
    ref = layer.shared_experts(x_bits, d["sh_gate"], d["sh_up"], d["sh_down"], s.n_shared, s.shared_inter)
    err = rel_max_err(got, ref)
    say(f"shared_expert_ffn mode {mode}: max|gpu-oracle|/rms = {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("mode,tol", [(0, 1e-4), (1, 1e-2)])
@pytest.mark.parametrize("T", [1, 17, 64])
def test_shared_expert_ffn_decode_sizes(mx, T, mode, tol):
    """The same product at decode-sized token counts, where it runs on the
    persistent streaming kernel: one token, a whole 16-row chunk plus a ragged
    one-row chunk, and four whole chunks; the K splits go through the
    finalize pass.  Both operand modes (h split hi + lo, or rounded)."""
    from mxfp4_latent_moe_amd import _lib, ops
    dev = torch.device("cuda:0")
    s = MID_SHAPE
    x_bits = synth.gen_tokens(MID, T)
    d = synth.gen_dense(MID)
    out0 = np.random.default_rng(6).standard_normal((T, s.hidden)).astype(np.float32)
    say(f"case: shared_expert_ffn T={T} mode {mode} (decode sizes)")
    sh = _shape(mx, mode)
    ws = torch.empty(ops.workspace_bytes(sh, _lib.MOE_FN_SHARED_FFN, T), dtype=torch.uint8, device=dev)
    out = to_dev(out0, dev)
    ops.shared_ffn(sh, to_dev_bf16(x_bits, dev), to_dev_bf16(d["sh_gate"], dev), to_dev_bf16(d["sh_up"], dev),
                   to_dev_bf16(d["sh_down"], dev), out, 1, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64) - out0
    ref = layer.shared_experts(x_bits, d["sh_gate"], d["sh_up"], d["sh_down"], s.n_shared, s.shared_inter)
    err = rel_max_err(got, ref)
    say(f"shared_expert_ffn T={T} mode {mode}: max|gpu-oracle|/rms = {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("E,T", [(64, 1100), (62, 1100), (242, 1100), (62, 300), (62, 100), (242, 40)])
def test_route_tiled(mx, E, T):
    """Router logits + top-k and the latent projection z: at T = 1100 and 300
    on the tiled kernel (at 300 one ragged token tile, K split), at T = 100
    and 40 on the mid-size and streaming kernels.
    Expert counts that are not a multiple of 4 leave a ragged group of logit
    columns at the end of every row."""
    from mxfp4_latent_moe_amd import _lib, ops
    dev = torch.device("cuda:0")
    s = synth.LayerShape(MID_SHAPE.hidden, MID_SHAPE.latent, E, MID_SHAPE.top_k, MID_SHAPE.inter,
                         MID_SHAPE.n_shared, MID_SHAPE.shared_inter)
    wl = synth.Workload(f"mid{T}e{E}", 12, s, T, 12, 0.02, 0.1, "normal", 119, 121)
    x_bits = synth.gen_tokens(wl)
    d = synth.gen_dense(wl)
    bias = synth.gen_bias(wl)
    say(f"case: moe_route T={T} H={s.hidden} E={s.n_experts} L={s.latent}")
    sh = mx.make_shape(s.hidden, s.latent, s.n_experts, s.top_k, s.inter, s.n_shared, s.shared_inter)
    ws = torch.empty(ops.workspace_bytes(sh, _lib.MOE_FN_ROUTE, T), dtype=torch.uint8, device=dev)
    ids = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, s.top_k), dtype=torch.float32, device=dev)
    z = torch.empty((T, s.latent), dtype=torch.float32, device=dev)
    gap = torch.empty((T,), dtype=torch.float32, device=dev)
    ops.route(sh, to_dev_bf16(x_bits, dev), to_dev_bf16(d["w_router"], dev), to_dev(bias, dev),
              to_dev_bf16(d["w_down"], dev), ids, w, z, gap, ws)
    torch.cuda.synchronize()
    r = layer.route(x_bits, d["w_router"], bias, s.top_k)
    keep = r["gap"] >= GAP_EXCLUDE
    assert (ids.cpu().numpy()[keep] == r["ids"][keep]).all()
    np.testing.assert_allclose(w.cpu().numpy()[keep], r["weights"][keep], rtol=2e-5, atol=1e-7)
    zref = layer.latent_down(x_bits, d["w_down"])
    err = rel_max_err(z.cpu().numpy(), zref)
    say(f"moe_route: z max|gpu-oracle|/rms = {err:.3e}, near-tie tokens {int((~keep).sum())}")
    assert err <= 1e-5
