"""GPU parity at full Kimi K3 shapes (H=7168, L=3584, E=896, k=16, I=3072, 2 shared experts).

The whole layer runs on the GPU for every token of each workload, in the
launch configuration the benchmark times.  The float64 oracle checks: expert
ids and the permutation for every token (exact outside near-ties), z for every
token, and the full layer output, H and Y for sampled tokens (the oracle
evaluates one token at a time; each output row depends only on its token).
"""
import numpy as np
import pytest
import torch

import synth
from synth.device import to_dev, upload_tokens, upload_weights
from oracle import layer
from gpu_common import (TOL, ZIPF_BIAS, check_permutation, check_routing, expert_cache, rel_max_err,
                        say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


@pytest.fixture(scope="module")
def mx():
    import mxfp4_latent_moe_amd as mx
    mx.load()
    return mx


@pytest.fixture(scope="module")
def k3(mx):
    say("fixture: generating and uploading the full K3 weight set (15.7 GB of experts)")
    wl = synth.workload("decode")
    w = upload_weights(wl, DEV)
    torch.cuda.synchronize()
    dense = synth.gen_dense(wl)
    return {"w": w, "dense": dense, "cache": expert_cache(wl)}


def _run_layer(mx, k3, wl, bias_np=None, operand_mode=0, **schedule):
    w = dict(k3["w"])
    if bias_np is not None:
        w["bias"] = to_dev(bias_np, DEV)
    moe = mx.LatentMoE(mx.shape_of(wl.shape, operand_mode), w, DEV, **schedule)
    x = upload_tokens(wl, DEV)
    bufs = moe.forward(x)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in bufs.items() if k not in ("ws",)}


def _full_check(mx, k3, wl, bias, sample, tag, operand_mode=0, inter_tol=1e-4):
    say(f"case: {tag} (T={wl.tokens}) full layer on GPU")
    g = _run_layer(mx, k3, wl, None if wl.bias_mode == "normal" else bias, operand_mode)
    x_bits = synth.gen_tokens(wl)
    d = k3["dense"]
    say(f"case: {tag} oracle routing for all tokens")
    ref = layer.route(x_bits, d["w_router"], bias, wl.shape.top_k)
    excl = check_routing(g["topk_ids"], g["topk_w"], ref)
    same = (g["topk_ids"] == ref["ids"]).all(axis=1)
    say(f"{tag}: {excl.size} near-tie tokens excluded, {int((~same).sum())} of them with a different set")
    # outputs are compared only where the GPU chose the oracle's expert set
    sample = np.array([t for t in sample if same[t]])
    check_permutation(g, ref["ids"], wl.shape.n_experts, excl)
    zs = sample if wl.tokens > 256 else np.arange(wl.tokens)
    z_ref = layer.latent_down(x_bits[zs], d["w_down"])
    assert rel_max_err(g["z"][zs], z_ref) < 1e-5
    say(f"case: {tag} oracle layer for tokens {list(sample)}")
    r = layer.layer_forward(x_bits[sample], d, bias, k3["cache"], wl.shape, keep=True)
    err = rel_max_err(g["out"][sample], r["out"])
    say(f"{tag}: max|gpu-oracle|/rms over sampled tokens = {err:.3e} (excluded near-ties: {excl.size})")
    assert err <= TOL
    # the per-pair intermediates of the sampled tokens
    k = wl.shape.top_k
    pp = g["pair_pos"].reshape(-1, k)[sample]
    Y_pair = r["Y_pair"]  # [s, k, L] oracle, unweighted
    assert rel_max_err(g["Y"][pp.reshape(-1)], Y_pair.reshape(-1, Y_pair.shape[-1])) < inter_tol
    return err


def test_decode_T16(mx, k3):
    wl = synth.workload("decode")
    bias = synth.gen_bias(wl)
    err = _full_check(mx, k3, wl, bias, np.array([0, 7, 15]), "decode")
    assert err < 1e-3


@pytest.mark.parametrize("wl_name", ["decode", "batched_decode"])
def test_schedules_bitwise_equal(mx, k3, wl_name):
    """The layer's stream schedules (z, at decode sizes, joined before the
    expert GEMMs and the shared experts before the combine; the whole side
    stream joined before the expert GEMMs; one stream) run the same kernels on
    the same data, so every buffer is bitwise the same."""
    wl = synth.workload(wl_name)
    bias = None if wl.bias_mode == "normal" else synth.gen_bias(wl, ZIPF_BIAS)
    say(f"case: {wl_name} (T={wl.tokens}) layer under three stream schedules")
    base = _run_layer(mx, k3, wl, bias)
    for sched in ({"overlap_shared": False}, {"late_shared_join": False}):
        g = _run_layer(mx, k3, wl, bias, **sched)
        for key in ("topk_ids", "topk_w", "z", "sorted_pair", "pair_pos", "H", "Y", "out"):
            assert np.array_equal(g[key], base[key]), (sched, key)


def test_batched_decode_T256_zipf(mx, k3):
    wl = synth.workload("batched_decode")
    bias = synth.gen_bias(wl, ZIPF_BIAS)
    _full_check(mx, k3, wl, bias, np.array([3, 128, 255]), "batched_decode")


def test_prefill_T4096(mx, k3):
    wl = synth.workload("prefill")
    bias = synth.gen_bias(wl)
    _full_check(mx, k3, wl, bias, np.array([0, 2049, 4095]), "prefill")


def test_prefill_T4096_mx8x3(mx, k3):
    """Prefill through the MX-scaled expert GEMMs (three fp8 activation terms)."""
    from mxfp4_latent_moe_amd import _lib
    wl = synth.workload("prefill")
    bias = synth.gen_bias(wl)
    # three fp8 terms leave about 2^-12 of each 32-block's maximum: intermediates within 2e-3
    err = _full_check(mx, k3, wl, bias, np.array([1, 1500, 4094]), "prefill mx8x3", _lib.MOE_OPND_MX8X3,
                      inter_tol=2e-3)
    assert err < 2e-3


def test_prefill_T4096_mx6x3(mx, k3):
    """Prefill through the MX-scaled expert GEMMs (three fp6 activation terms)."""
    from mxfp4_latent_moe_amd import _lib
    wl = synth.workload("prefill")
    bias = synth.gen_bias(wl)
    err = _full_check(mx, k3, wl, bias, np.array([2, 2500, 4093]), "prefill mx6x3", _lib.MOE_OPND_MX6X3,
                      inter_tol=2e-3)
    assert err < 2e-3


def test_microbench_grouped_gemm(mx, k3):
    """Isolated grouped GEMM: segments ~ Multinomial(65536, Zipf(1.1)); A bf16 already permuted."""
    from mxfp4_latent_moe_amd import ops
    wl = synth.workload("microbench")
    sh = wl.shape
    counts = synth.gen_microbench_counts(wl)
    P = int(counts.sum())
    offsets = np.zeros(sh.n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    say("case: microbench upload A [65536, 3584] bf16")
    A_bits = synth.gen_microbench_activations(wl)
    A = torch.from_numpy(A_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    s = mx.shape_of(sh)
    w = k3["w"]
    ws = torch.empty(ops.workspace_bytes(s, ops.MOE_FN_GROUPED_GEMM, P), dtype=torch.uint8, device=DEV)
    H = torch.empty((P, sh.inter), dtype=torch.float32, device=DEV)
    Y = torch.empty((P, sh.latent), dtype=torch.float32, device=DEV)
    off_d = to_dev(offsets, DEV)
    say("case: microbench gate/up + down on GPU")
    ops.grouped_gemm(s, ops.MOE_OP_GATEUP_SITU, P, off_d, None, A, w["w1_packed"], w["w1_scale"],
                     w["w3_packed"], w["w3_scale"], None, H, ws)
    ops.grouped_gemm(s, ops.MOE_OP_DOWN, P, off_d, None, H, w["w2_packed"], w["w2_scale"], None, None,
                     None, Y, ws)
    torch.cuda.synchronize()
    hot = int(np.argmax(counts))
    cold = [int(e) for e in np.argsort(counts)[:3]]
    mid = int(np.argsort(counts)[sh.n_experts // 2])
    errs = []
    for e in [hot, mid] + cold:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rows = np.arange(r0, r1) if r1 - r0 <= 40 else np.r_[r0:r0 + 20, r1 - 20:r1]
        say(f"case: microbench oracle expert {e} ({r1 - r0} rows, checking {rows.size})")
        Hr, Yr = layer.expert_mlp(layer.bf16_to_f64(A_bits[rows]), k3["cache"](e))
        Hg = H[torch.from_numpy(rows).to(DEV)].cpu().numpy()
        Yg = Y[torch.from_numpy(rows).to(DEV)].cpu().numpy()
        assert rel_max_err(Hg, Hr) < 1e-4
        errs.append(rel_max_err(Yg, Yr))
    say(f"microbench: max|gpu-oracle|/rms on Y over sampled rows = {max(errs):.3e}")
    assert max(errs) <= TOL


def test_expert_slice_partition_invariance(mx, k3):
    """One GPU's share under expert parallelism: the grouped GEMMs run over a
    contiguous 112-expert slice (weights, offsets and rows of that slice only)
    give bit-identical H and Y rows to the full 896-expert call."""
    from mxfp4_latent_moe_amd import ops
    wl = synth.workload("decode")
    sh = wl.shape
    say("case: decode layer, then each of the 8 expert slices of 112 experts")
    g = _run_layer(mx, k3, wl)
    w = k3["w"]
    offsets = g["offsets"]
    n_slice = sh.n_experts // 8
    for e0 in range(0, sh.n_experts, n_slice):
        r0, r1 = int(offsets[e0]), int(offsets[e0 + n_slice])
        if r1 == r0:
            continue
        sub = synth.LayerShape(sh.hidden, sh.latent, n_slice, sh.top_k, sh.inter, sh.n_shared, sh.shared_inter)
        s = mx.shape_of(sub)
        P = r1 - r0
        off = to_dev((offsets[e0:e0 + n_slice + 1] - r0).astype(np.int32), DEV)
        sp = to_dev(g["sorted_pair"][r0:r1].astype(np.int32), DEV)
        z = to_dev(g["z"], DEV)
        ws = torch.empty(ops.workspace_bytes(s, ops.MOE_FN_GROUPED_GEMM, P), dtype=torch.uint8, device=DEV)
        H = torch.empty((P, sh.inter), dtype=torch.float32, device=DEV)
        Y = torch.empty((P, sh.latent), dtype=torch.float32, device=DEV)
        sl = slice(e0, e0 + n_slice)
        ops.grouped_gemm(s, ops.MOE_OP_GATEUP_SITU, P, off, sp, z, w["w1_packed"][sl], w["w1_scale"][sl],
                         w["w3_packed"][sl], w["w3_scale"][sl], None, H, ws)
        ops.grouped_gemm(s, ops.MOE_OP_DOWN, P, off, sp, H, w["w2_packed"][sl], w["w2_scale"][sl], None, None,
                         None, Y, ws)
        torch.cuda.synchronize()
        assert (H.cpu().numpy() == g["H"][r0:r1]).all(), e0
        assert (Y.cpu().numpy() == g["Y"][r0:r1]).all(), e0
