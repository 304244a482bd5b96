"""GPU top-k selection against the oracle on exactly representable scores.

Logits are taken from {-120, 0, 20}, whose sigmoids are exactly 0, 1/2 and 1
in float32 on both sides, and biases from {-inf, -1, -1/2, 0, 1/2}, so every
biased decision value is exact and ties are exact ties: the GPU's ids,
weights and gaps must equal the oracle's for every token, with no near-tie
exclusion.  Ties go to the lower expert index (kimi-k3-mlx README,
Architecture table, MoE row: sigmoid router, correction bias in the
selection only).  Covers E not a multiple of the 64-wide wavefront, k = 1,
k = E, experts masked by a -inf bias, and a ragged token count.
"""
import numpy as np
import pytest
import torch

from synth.device import to_dev, to_dev_bf16
from synth.inputs import LayerShape
from oracle import layer
from gpu_common import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def mx():
    import mxfp4_latent_moe_amd as mx
    mx.load()
    return mx


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert (bits & 0xFFFF).max() == 0  # exactly representable in bf16
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("E,k,T", [(896, 16, 301), (200, 16, 77), (200, 1, 40), (32, 32, 9), (1024, 32, 65)])
def test_topk_exact_ties(mx, E, k, T):
    from mxfp4_latent_moe_amd import ops
    H = 256
    rng = np.random.default_rng(1000 + E + k)
    say(f"case: top-k E={E} k={k} T={T}")
    # token t's logits are column h(t) of the router: one-hot tokens
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), rng.integers(0, H, T)] = 1.0
    w_router = rng.choice(np.array([-120.0, 0.0, 20.0], np.float32), size=(E, H), p=[0.3, 0.5, 0.2])
    bias = rng.choice(np.array([-np.inf, -1.0, -0.5, 0.0, 0.5], np.float32), size=E, p=[0.1, 0.2, 0.2, 0.3, 0.2])
    x_bits, w_bits = _bf16_bits(x), _bf16_bits(w_router)
    ref = layer.route(x_bits, w_bits, bias, k)

    s = mx.shape_of(LayerShape(H, 128, E, k, 128, 0, 0))
    ws = torch.empty(ops.workspace_bytes(s, ops.MOE_FN_ROUTE, T), dtype=torch.uint8, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    gap = torch.empty((T,), dtype=torch.float32, device=DEV)
    ops.route(s, to_dev_bf16(x_bits, DEV), to_dev_bf16(w_bits, DEV), to_dev(bias, DEV), None, ids, w, None,
              gap, ws)
    torch.cuda.synchronize()
    g_ids, g_w, g_gap = ids.cpu().numpy(), w.cpu().numpy(), gap.cpu().numpy()
    assert np.array_equal(g_ids, ref["ids"])
    # the oracle's weights come from float64 scores, where sigmoid(-120) is
    # about 8e-53 rather than the float32 zero: an absolute floor far below
    # float32's normal range covers that
    np.testing.assert_allclose(g_w, ref["weights"], rtol=1e-6, atol=1e-30)
    # gap: exact decision values, so exactly the oracle's (0 at a tie, inf at k = E)
    np.testing.assert_array_equal(g_gap, ref["gap"].astype(np.float32))
    if k < E:
        assert (ref["gap"] == 0).any()  # the case has ties at the k-th place


@pytest.mark.parametrize("E,k,T,k_hi", [(896, 16, 301, 4), (200, 16, 77, 2), (200, 16, 77, 0), (32, 32, 9, 5)])
def test_route_capped_exact(mx, E, k, T, k_hi):
    """moe_route_capped on exactly representable scores: the capped weights are
    the oracle's cap (Kimi-K3-Alis-MLX-Dynamic card, Build recipe) for every
    token, ties in routing order going to the lower index."""
    from mxfp4_latent_moe_amd import ops
    from oracle.promotion import cap_promoted
    H = 256
    rng = np.random.default_rng(2000 + E + k + k_hi)
    say(f"case: capped top-k E={E} k={k} T={T} k_hi={k_hi}")
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), rng.integers(0, H, T)] = 1.0
    w_router = rng.choice(np.array([-120.0, 0.0, 20.0], np.float32), size=(E, H), p=[0.3, 0.5, 0.2])
    bias = rng.choice(np.array([-np.inf, -1.0, -0.5, 0.0, 0.5], np.float32), size=E, p=[0.1, 0.2, 0.2, 0.3, 0.2])
    promoted = rng.random(E) < 0.4
    x_bits, w_bits = _bf16_bits(x), _bf16_bits(w_router)
    ref = layer.route(x_bits, w_bits, bias, k)
    want = cap_promoted(ref["ids"], ref["weights"], ref["biased32"], promoted, k_hi)
    assert (want == 0).any() or k_hi >= k

    s = mx.shape_of(LayerShape(H, 128, E, k, 128, 0, 0))
    ws = torch.empty(ops.workspace_bytes(s, ops.MOE_FN_ROUTE, T), dtype=torch.uint8, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    gap = torch.empty((T,), dtype=torch.float32, device=DEV)
    ops.route_capped(s, to_dev_bf16(x_bits, DEV), to_dev_bf16(w_bits, DEV), to_dev(bias, DEV), None,
                     to_dev(promoted.astype(np.uint8), DEV), k_hi, ids, w, None, gap, ws)
    torch.cuda.synchronize()
    g_ids, g_w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(g_ids, ref["ids"])
    np.testing.assert_array_equal(gap.cpu().numpy(), ref["gap"].astype(np.float32))
    # the experts the cap drops are exactly 0 on the GPU; every other weight
    # matches (an expert whose float64 weight is ~1e-53, sigmoid(-120), is
    # the float32 zero already, hence the absolute floor)
    dropped = (want == 0) & (ref["weights"] != 0)
    assert (g_w[dropped] == 0).all()
    np.testing.assert_allclose(g_w, want, rtol=1e-6, atol=1e-30)


def test_route_capped_full_size(mx):
    """K3 router on 4096 tokens, 90 of 896 experts promoted, k_hi = 4: ids, gap
    and every kept weight bitwise moe_route's; the dropped set the oracle's
    outside near-ties at the cap; about the hypergeometric share of tokens
    loses a contribution."""
    import synth
    from mxfp4_latent_moe_amd import ops
    from oracle.promotion import cap_promoted
    from gpu_common import check_routing
    wl = synth.workload("prefill")
    sh = wl.shape
    T, E, k, k_hi = wl.tokens, sh.n_experts, sh.top_k, 4
    rng = np.random.default_rng(77)
    promoted = np.zeros(E, bool)
    promoted[rng.choice(E, 90, replace=False)] = True
    x_bits = synth.gen_tokens(wl)
    w_bits = synth.gen_dense(wl)["w_router"]
    bias = synth.gen_bias(wl)
    say(f"case: capped routing at K3 shapes, T={T}, 90 promoted, k_hi={k_hi}")
    s = mx.shape_of(sh)
    ws = torch.empty(ops.workspace_bytes(s, ops.MOE_FN_ROUTE, T), dtype=torch.uint8, device=DEV)
    xd, wd, bd = to_dev_bf16(x_bits, DEV), to_dev_bf16(w_bits, DEV), to_dev(bias, DEV)
    out = {}
    for capped in (False, True):
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        gap = torch.empty((T,), dtype=torch.float32, device=DEV)
        if capped:
            ops.route_capped(s, xd, wd, bd, None, to_dev(promoted.astype(np.uint8), DEV), k_hi, ids, w, None, gap,
                             ws)
        else:
            ops.route(s, xd, wd, bd, None, ids, w, None, gap, ws)
        torch.cuda.synchronize()
        out[capped] = (ids.cpu().numpy(), w.cpu().numpy(), gap.cpu().numpy())
    (i0, w0, g0), (i1, w1, g1) = out[False], out[True]
    assert np.array_equal(i0, i1) and np.array_equal(g0, g1)
    kept = w1 != 0
    assert np.array_equal(w1[kept], w0[kept])
    X = promoted[i1].sum(axis=1)
    assert np.array_equal((~kept).sum(axis=1), np.maximum(X - k_hi, 0))
    ref = layer.route(x_bits, w_bits, bias, k)
    excl = set(check_routing(i1, w0, ref).tolist())
    # near-ties among a token's promoted experts at the cap boundary are excluded
    b = ref["biased32"].astype(np.float64)
    for t in range(T):
        pv = np.sort(b[t, ref["ids"][t][promoted[ref["ids"][t]]]])[::-1]
        if len(pv) > k_hi and pv[k_hi - 1] - pv[k_hi] < 1e-5:
            excl.add(t)
    keep = np.array(sorted(set(range(T)) - excl))
    want = cap_promoted(ref["ids"][keep], ref["weights"][keep], ref["biased32"][keep], promoted, k_hi)
    assert np.array_equal(w1[keep] == 0, want == 0)
    rate = (~kept).any(axis=1).mean()
    say(f"capped routing: {rate:.4f} of tokens lose a contribution, {len(excl)} excluded")
    assert 0.005 < rate < 0.04
