"""REAP saliency through the C ABI against the oracle (README, REAP section).

Tiny layer end to end (the layer's own Y, routing weights and permutation), and
a full-size batch of synthetic expert outputs: 4096 tokens x top-16 over 896
experts with Zipf-distributed loads, L = 3584.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from synth.device import to_dev, to_dev_bf16, upload_weights
from oracle import layer, reap
from gpu_common import check_routing, rel_max_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def mx():
    import mxfp4_latent_moe_amd as m
    m.load()
    return m


def _sal(mx, s, P, offsets, Y, pw, sp, sal, cnt, acc):
    from mxfp4_latent_moe_amd import _lib, ops
    ws = torch.empty(max(256, ops.workspace_bytes(s, _lib.MOE_FN_REAP_SALIENCY, P)), dtype=torch.uint8, device=DEV)
    ops.reap_saliency(s, P, offsets, Y, pw, sp, sal, cnt, acc, ws)
    torch.cuda.synchronize()


def test_reap_tiny_layer(mx):
    wl = synth.workload("tiny")
    T = 37
    x_bits = synth.gen_tokens(synth.Workload("tiny37", 11, wl.shape, T, wl.wset, wl.router_std, wl.bias_std,
                                             "normal", wl.exp_lo, wl.exp_hi))
    say(f"case: REAP saliency on the tiny layer, T={T}")
    sh = wl.shape
    s = mx.shape_of(sh)
    layer_ = mx.LatentMoE(s, upload_weights(wl, DEV), DEV)
    b = layer_.forward(to_dev_bf16(x_bits, DEV))
    torch.cuda.synchronize()
    st = synth.gen_expert_stack(wl)
    cache = layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()})
    ref = layer.layer_forward(x_bits, synth.gen_dense(wl), synth.gen_bias(wl), cache, sh, keep=True)
    excl = check_routing(b["topk_ids"].cpu().numpy(), b["topk_w"].cpu().numpy(), ref)
    assert excl.size == 0, "this seed has near-tie tokens"
    want = reap.reap_saliency(ref["Y_pair"], ref["ids"], ref["weights"], sh.n_experts)
    E, P = sh.n_experts, T * sh.top_k
    sal = torch.empty(E, dtype=torch.float64, device=DEV)
    cnt = torch.empty(E, dtype=torch.int64, device=DEV)
    _sal(mx, s, P, b["offsets"], b["Y"], b["topk_w"], b["sorted_pair"], sal, cnt, 0)
    got_s, got_c = sal.cpu().numpy(), cnt.cpu().numpy()
    assert (got_c == want["count"]).all()
    err = rel_max_err(got_s, want["sum"])
    say(f"tiny REAP: max|gpu-oracle|/rms of the sums = {err:.3e}")
    assert err <= 1e-4
    # a second batch accumulates: the same batch again doubles both, exactly
    _sal(mx, s, P, b["offsets"], b["Y"], b["topk_w"], b["sorted_pair"], sal, cnt, 1)
    assert (sal.cpu().numpy() == 2 * got_s).all() and (cnt.cpu().numpy() == 2 * got_c).all()


def test_reap_full_size_synthetic(mx):
    sh = synth.K3_SHAPE
    T, k, E, L = 4096, sh.top_k, sh.n_experts, sh.latent
    rng = np.random.default_rng(2024)
    # distinct experts per token drawn with Zipf(1.1) probabilities over a permutation of the experts
    p = synth.zipf_probabilities(E, 1.1)[np.argsort(rng.permutation(E))]
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    P = T * k
    sorted_pair = np.argsort(ids.reshape(-1), kind="stable").astype(np.int32)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Y_sorted = rng.standard_normal((P, L), dtype=np.float32)
    say(f"case: REAP saliency full size, P={P}, L={L}, largest segment {counts.max()}, empty experts "
        f"{int((counts == 0).sum())}")
    Y_pair = np.empty_like(Y_sorted)
    Y_pair[sorted_pair] = Y_sorted
    want = reap.reap_saliency(Y_pair.reshape(T, k, L), ids, w, E)
    s = mx.shape_of(sh)
    sal = torch.empty(E, dtype=torch.float64, device=DEV)
    cnt = torch.empty(E, dtype=torch.int64, device=DEV)
    Yd = to_dev(Y_sorted, DEV)
    args = (to_dev(offsets, DEV), Yd, to_dev(w.reshape(-1), DEV), to_dev(sorted_pair, DEV))
    _sal(mx, s, P, *args, sal, cnt, 0)
    got_s = sal.cpu().numpy()
    assert (cnt.cpu().numpy() == want["count"]).all()
    err = rel_max_err(got_s, want["sum"])
    say(f"full-size REAP: max|gpu-oracle|/rms of the sums = {err:.3e}")
    assert err <= 1e-5
    # deterministic: a second run is bitwise identical
    _sal(mx, s, P, *args, sal, cnt, 0)
    assert (sal.cpu().numpy() == got_s).all()
    # rows that already carry their weight (pair weights folded into the down GEMM)
    Yw = to_dev(Y_sorted * w.reshape(-1)[sorted_pair][:, None], DEV)
    _sal(mx, s, P, args[0], Yw, None, None, sal, cnt, 0)
    err_w = rel_max_err(sal.cpu().numpy(), want["sum"])
    say(f"full-size REAP, pre-weighted rows: {err_w:.3e}")
    assert err_w <= 1e-5


def _combine(mx, s, T, Y, pair_pos, topk_w, gamma, w_up, reap_out=None, reap_acc=0):
    """moe_combine_norm_up, or with reap_out = (offsets, sal, cnt) the fused call; returns out."""
    from mxfp4_latent_moe_amd import _lib, ops
    out = torch.empty((T, s.hidden), dtype=torch.float32, device=DEV)
    if reap_out is None:
        ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP, T), dtype=torch.uint8, device=DEV)
        ops.combine_norm_up(s, T, Y, pair_pos, topk_w, gamma, w_up, out, 0, ws)
    else:
        ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP_REAP, T), dtype=torch.uint8,
                         device=DEV)
        ops.combine_norm_up_reap(s, T, Y, pair_pos, topk_w, gamma, w_up, out, 0, *reap_out, reap_acc, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_combine_reap_tiny_layer(mx):
    """The fused combine + REAP call on the tiny layer (L = 128: the first wave
    straddles the end of the row): out bitwise equal to moe_combine_norm_up, the
    sums equal to the oracle's and to moe_reap_saliency's, accumulation exact."""
    wl = synth.workload("tiny")
    T = 37
    x_bits = synth.gen_tokens(synth.Workload("tiny37", 11, wl.shape, T, wl.wset, wl.router_std, wl.bias_std,
                                             "normal", wl.exp_lo, wl.exp_hi))
    say(f"case: fused combine + REAP on the tiny layer, T={T}")
    sh = wl.shape
    s = mx.shape_of(sh)
    w = upload_weights(wl, DEV)
    b = mx.LatentMoE(s, w, DEV).forward(to_dev_bf16(x_bits, DEV))
    torch.cuda.synchronize()
    E, P = sh.n_experts, T * sh.top_k
    plain = _combine(mx, s, T, b["Y"], b["pair_pos"], b["topk_w"], w["gamma"], w["w_up"])
    sal = torch.empty(E, dtype=torch.float64, device=DEV)
    cnt = torch.empty(E, dtype=torch.int64, device=DEV)
    fused = _combine(mx, s, T, b["Y"], b["pair_pos"], b["topk_w"], w["gamma"], w["w_up"], (b["offsets"], sal, cnt))
    assert np.array_equal(fused, plain)
    got_s, got_c = sal.cpu().numpy(), cnt.cpu().numpy()
    # against the separate saliency pass over the same rows, and against the oracle
    sal2 = torch.empty(E, dtype=torch.float64, device=DEV)
    cnt2 = torch.empty(E, dtype=torch.int64, device=DEV)
    _sal(mx, s, P, b["offsets"], b["Y"], b["topk_w"], b["sorted_pair"], sal2, cnt2, 0)
    assert (got_c == cnt2.cpu().numpy()).all()
    assert rel_max_err(got_s, sal2.cpu().numpy()) <= 1e-6
    st = synth.gen_expert_stack(wl)
    cache = layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()})
    ref = layer.layer_forward(x_bits, synth.gen_dense(wl), synth.gen_bias(wl), cache, sh, keep=True)
    excl = check_routing(b["topk_ids"].cpu().numpy(), b["topk_w"].cpu().numpy(), ref)
    assert excl.size == 0, "this seed has near-tie tokens"
    want = reap.reap_saliency(ref["Y_pair"], ref["ids"], ref["weights"], E)
    assert (got_c == want["count"]).all()
    err = rel_max_err(got_s, want["sum"])
    say(f"tiny fused REAP: max|gpu-oracle|/rms of the sums = {err:.3e}")
    assert err <= 1e-4
    _combine(mx, s, T, b["Y"], b["pair_pos"], b["topk_w"], w["gamma"], w["w_up"], (b["offsets"], sal, cnt), 1)
    assert (sal.cpu().numpy() == 2 * got_s).all() and (cnt.cpu().numpy() == 2 * got_c).all()


def test_combine_reap_full_size_synthetic(mx):
    """The fused call at K3 shapes on 4096 tokens with Zipf loads: out bitwise
    equal to moe_combine_norm_up, sums within 1e-5 of the oracle, for weighted
    rows and for rows that already carry their weight."""
    sh = synth.K3_SHAPE
    T, k, E, L = 4096, sh.top_k, sh.n_experts, sh.latent
    rng = np.random.default_rng(2025)
    p = synth.zipf_probabilities(E, 1.1)[np.argsort(rng.permutation(E))]
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    P = T * k
    sorted_pair = np.argsort(ids.reshape(-1), kind="stable").astype(np.int32)
    pair_pos = np.empty(P, np.int32)
    pair_pos[sorted_pair] = np.arange(P, dtype=np.int32)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Y_sorted = rng.standard_normal((P, L), dtype=np.float32)
    Y_pair = np.empty_like(Y_sorted)
    Y_pair[sorted_pair] = Y_sorted
    want = reap.reap_saliency(Y_pair.reshape(T, k, L), ids, w, E)
    gamma = to_dev_bf16(synth.gen_gamma_random(synth.workload("prefill")), DEV)
    w_up = torch.randn((sh.hidden, L), device=DEV).mul_(L ** -0.5).to(torch.bfloat16)
    s = mx.shape_of(sh)
    say(f"case: fused combine + REAP full size, T={T}, P={P}")
    offs, pp = to_dev(offsets, DEV), to_dev(pair_pos, DEV)
    sal = torch.empty(E, dtype=torch.float64, device=DEV)
    cnt = torch.empty(E, dtype=torch.int64, device=DEV)
    for rows, tw in ((Y_sorted, w), (Y_sorted * w.reshape(-1)[sorted_pair][:, None], None)):
        Yd = to_dev(rows, DEV)
        twd = None if tw is None else to_dev(tw, DEV)
        fused = _combine(mx, s, T, Yd, pp, twd, gamma, w_up, (offs, sal, cnt))
        assert np.array_equal(fused, _combine(mx, s, T, Yd, pp, twd, gamma, w_up))
        assert (cnt.cpu().numpy() == want["count"]).all()
        err = rel_max_err(sal.cpu().numpy(), want["sum"])
        say(f"full-size fused REAP ({'weighted' if tw is not None else 'pre-weighted'} rows): {err:.3e}")
        assert err <= 1e-5
