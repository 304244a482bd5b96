"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: the
pages' printed numbers (tests/golden/k3_printed_numbers.json), closed forms
and limits, brute force on tiny inputs, a library routine for a special case,
or invariants the pages state.  A plausible slip (wrong nibble order, sign
bit, scale offset, tie rule, weight normalisation, norm placement, missing
shared term) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import layer, mxfp4, scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _printed():
    with open(os.path.join(GOLDEN, "k3_printed_numbers.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


# ---------------------------------------------------------------- (a) e2m1 / e8m0

# OCP MX v1.0 e2m1 values typed out by code 0..15 (sign bit 3).
E2M1_TYPED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
EXPONENTS = [0, 1, 2, 100, 117, 118, 119, 120, 121, 127, 128, 200, 253, 254]


def test_dequant_all_bytes_all_sampled_scales():
    """Every packed byte x sampled e8m0 exponents: element 2b = low nibble, 2b+1 = high nibble."""
    bytes_ = np.arange(256, dtype=np.uint8)
    for e in EXPONENTS:
        packed = np.repeat(bytes_[:, None], 16, axis=1)          # [256, 16] -> K = 32
        scale = np.full((256, 1), e, dtype=np.uint8)
        got = mxfp4.dequant(packed, scale)
        s = math.ldexp(1.0, e - 127)
        for b in range(256):
            lo, hi = E2M1_TYPED[b & 15] * s, E2M1_TYPED[b >> 4] * s
            assert got[b, 0] == lo and got[b, 1] == hi, (b, e)
            assert math.copysign(1.0, got[b, 0]) == math.copysign(1.0, lo)
            assert (got[b, 0::2] == lo).all() and (got[b, 1::2] == hi).all()


def test_e8m0_matches_torch_float8_e8m0fnu():
    e = torch.arange(256, dtype=torch.uint8)
    ref = e.view(torch.float8_e8m0fnu).double().numpy()
    got = mxfp4.e8m0_to_f64(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert (got[:255] == ref[:255]).all()


def test_e2m1_table_matches_bit_formula():
    for c in range(16):
        assert scalar.e2m1_decode(c) == E2M1_TYPED[c]
        assert mxfp4.E2M1_VALUES[c] == E2M1_TYPED[c]
        assert math.copysign(1, mxfp4.E2M1_VALUES[c]) == math.copysign(1, E2M1_TYPED[c])


def test_dequant_scale_groups_of_32():
    """scale[n, g] applies to k // 32 == g only."""
    packed = np.full((2, 64), 0x22, dtype=np.uint8)  # every code 2 -> 1.0
    scale = np.array([[127, 128, 126, 130], [1, 2, 3, 254]], dtype=np.uint8)
    got = mxfp4.dequant(packed, scale)
    for n in range(2):
        for k in range(128):
            assert got[n, k] == math.ldexp(1.0, int(scale[n, k // 32]) - 127)


# ---------------------------------------------------------------- (b) SiTU-GLU

def test_situ_limits_and_bound():
    P = _printed()
    beta, beta_lin = P["situ_beta"], P["situ_beta_lin"]
    assert (beta, beta_lin) == (layer.BETA, layer.BETA_LIN)
    u = np.linspace(-80, 80, 161)
    # g -> +inf: beta*1*1 * beta_lin*tanh(u/beta_lin)
    np.testing.assert_allclose(layer.situ_glu(60.0, u), beta * beta_lin * np.tanh(u / beta_lin), rtol=1e-12, atol=1e-12)
    # g -> -inf: -> 0 (with the sign opposite to u)
    f = layer.situ_glu(-60.0, u)
    assert np.abs(f).max() < 1e-20 and (np.sign(f) == -np.sign(u)).all()
    # u -> +-inf: +-beta_lin * (gate part)
    g = np.linspace(-20, 20, 81)
    gate = beta * np.tanh(g / beta) / (1 + np.exp(-g))
    np.testing.assert_allclose(layer.situ_glu(g, 1e4), beta_lin * gate, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(layer.situ_glu(g, -1e4), -beta_lin * gate, rtol=1e-12, atol=1e-300)
    # zeros, the supremum beta*beta_lin (reached only in rounding at saturation)
    assert (layer.situ_glu(0.0, u) == 0).all() and (layer.situ_glu(g, 0.0) == 0).all()
    G, U = np.meshgrid(np.linspace(-1e3, 1e3, 401), np.linspace(-1e3, 1e3, 401))
    assert np.abs(layer.situ_glu(G, U)).max() <= beta * beta_lin
    G, U = np.meshgrid(np.linspace(-30, 30, 301), np.linspace(-60, 60, 301))
    assert np.abs(layer.situ_glu(G, U)).max() < beta * beta_lin


def test_situ_small_signal_is_swiglu():
    """|g| << beta, |u| << beta_lin: SiTU-GLU -> SiLU(g)*u with relative deviation
    g^2/(3 beta^2) + u^2/(3 beta_lin^2) (Taylor of tanh), SiLU from torch."""
    g = np.array([-0.2, -0.05, 0.01, 0.1, 0.3])
    u = np.array([-1.0, -0.3, 0.2, 0.7, 1.5])
    G, U = np.meshgrid(g, u)
    silu = torch.nn.functional.silu(torch.from_numpy(G)).numpy()
    ratio = layer.situ_glu(G, U) / (silu * U)
    pred = (1 - G ** 2 / 48) * (1 - U ** 2 / 1875)
    assert np.abs(ratio - pred).max() < 1e-4
    assert np.abs(ratio - 1).max() > 1e-4  # the correction is really there


def test_situ_matches_scalar_oracle():
    rng = np.random.default_rng(5)
    for g, u in rng.normal(0, 6, size=(200, 2)):
        assert abs(layer.situ_glu(g, u) - scalar._situ(g, u, 4.0, 25.0)) <= 1e-12 * (1 + abs(scalar._situ(g, u, 4.0, 25.0)))


# ---------------------------------------------------------------- (c) exhaustive top-k

def _route_with_biased(values, k):
    """x = 0 makes every sigmoid score exactly 0.5, so biased32 = 0.5 + bias exactly."""
    E = len(values)
    x = np.zeros((1, 32), np.uint16)
    w = np.zeros((E, 32), np.uint16)
    bias = np.array(values, np.float32) - np.float32(0.5)
    return layer.route(x, w, bias, k)


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (5, 3), (6, 2), (6, 4), (7, 3)])
def test_topk_exhaustive_with_ties(E, k):
    alphabet = [0.25, 0.5, 0.75]
    for vals in itertools.product(alphabet, repeat=E):
        r = _route_with_biased(vals, k)
        # brute force: the one k-subset whose every member beats every non-member
        # under (larger value, then lower index)
        winners = [S for S in itertools.combinations(range(E), k)
                   if all((-vals[a], a) < (-vals[b], b) for a in S for b in range(E) if b not in S)]
        assert len(winners) == 1
        assert tuple(r["ids"][0]) == winners[0], vals
        np.testing.assert_allclose(r["weights"][0], np.full(k, 1.0 / k), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- (d) routing weights

def test_weights_sum_to_one_and_use_unbiased_scores():
    wl = synth.workload("tiny")
    x = synth.gen_tokens(wl)
    d = synth.gen_dense(wl)
    b = synth.gen_bias(wl)
    r = layer.route(x, d["w_router"], b, wl.shape.top_k)
    np.testing.assert_allclose(r["weights"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    sel = np.take_along_axis(r["scores"], r["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(r["weights"], sel / sel.sum(axis=1, keepdims=True), rtol=1e-14)
    # the bias selects but does not weight: raising the bias of selected experts
    # keeps the selection and leaves the weights unchanged
    b2 = b.copy()
    b2[np.unique(r["ids"])] += np.float32(0.5)
    r2 = layer.route(x, d["w_router"], b2, wl.shape.top_k)
    assert (r2["ids"] == r["ids"]).all()
    assert (r2["weights"] == r["weights"]).all()
    # sigmoid of the router logits (library logistic vs closed form)
    np.testing.assert_allclose(r["scores"], 1 / (1 + np.exp(-r["logits"])), rtol=1e-14)
    assert (np.diff(r["ids"], axis=1) > 0).all()
    assert (r["gap"] >= 0).all()


# ---------------------------------------------------------------- (e) closures against the pages

def test_parameter_and_byte_closures():
    P = _printed()
    sh = synth.K3_SHAPE
    layers = P["moe_layers"]
    per_expert = 3 * sh.latent * sh.inter
    routed = sh.n_experts * per_expert * layers
    assert routed == 2_722_740_830_208
    assert round(routed / 1e9, 1) == P["routed_expert_params_B"]
    shared = sh.n_shared * 3 * sh.hidden * sh.shared_inter * layers
    assert round(shared / 1e9, 1) == P["shared_expert_params_B"]
    latent = 2 * sh.hidden * sh.latent * layers
    assert round(latent / 1e9, 1) == P["latent_updown_params_B"]
    assert round(100 * routed / (P["total_params_B"] * 1e9), 2) == P["routed_share_pct"]
    assert sh.n_experts * 3 * layers == P["expert_tensor_count"]
    assert [sh.n_experts, sh.hidden] == P["router_shape"]
    assert round(sh.n_experts * sh.hidden * 2 / 1e6, 2) == P["router_mb"]
    # checkpoint layout produced by the generator == the audit's table
    wl = synth.workload("decode")
    w1p, w1s = synth.gen_expert(wl, 0, "w1")
    w2p, w2s = synth.gen_expert(wl, 0, "w2")
    assert list(w1p.shape) == P["w13_packed_shape"] and list(w1s.shape) == P["w13_scale_shape"]
    assert list(w2p.shape) == P["w2_packed_shape"] and list(w2s.shape) == P["w2_scale_shape"]
    assert w1p.nbytes == P["packed_bytes"] == w2p.nbytes
    assert w1s.nbytes == P["scale_bytes"] == w2s.nbytes
    expert_bytes = 2 * (w1p.nbytes + w1s.nbytes) + w2p.nbytes + w2s.nbytes
    assert expert_bytes == P["expert_bytes"]
    assert expert_bytes * 8 / per_expert == P["expert_bpw"]
    assert round(expert_bytes * sh.n_experts * layers / 1e12, 2) == P["expert_tb"]
    # the oracle dequantises exactly this layout
    deq = layer.dequant_expert({"w1_packed": w1p, "w1_scale": w1s, "w3_packed": w1p, "w3_scale": w1s,
                                "w2_packed": w2p, "w2_scale": w2s})
    assert deq["w1"].shape == (sh.inter, sh.latent) and deq["w2"].shape == (sh.latent, sh.inter)


# ---------------------------------------------------------------- whole layer

def _tiny():
    wl = synth.workload("tiny")
    x = synth.gen_tokens(wl)
    d = synth.gen_dense(wl)
    b = synth.gen_bias(wl)
    st = synth.gen_expert_stack(wl)
    return wl, x, d, b, st


def test_two_oracles_agree_on_tiny():
    wl, x, d, b, st = _tiny()
    sh = wl.shape
    cache = layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()})
    r = layer.layer_forward(x, d, b, cache, sh)
    experts = [{w: (st[w + "_packed"][e].tolist(), st[w + "_scale"][e].tolist()) for w in ("w1", "w3", "w2")}
               for e in range(sh.n_experts)]
    dl = {k: v.tolist() for k, v in d.items()}
    rms = np.sqrt(np.mean(r["out"] ** 2))
    for t in range(wl.tokens):
        o, ids, w = scalar.layer_forward_token(x[t].tolist(), dl, b.tolist(), experts, sh)
        assert ids == r["ids"][t].tolist()
        np.testing.assert_allclose(w, r["weights"][t], rtol=1e-13)
        assert np.abs(np.array(o) - r["out"][t]).max() <= 1e-12 * rms


def test_permutation_brute_force():
    rng = np.random.default_rng(3)
    for E, T, k in [(8, 5, 3), (32, 8, 4), (6, 11, 6)]:
        ids = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1)
        p = layer.permute(ids, E)
        pos = 0
        for e in range(E):
            members = [t * k + j for t in range(T) for j in range(k) if ids[t, j] == e]
            assert p["offsets"][e] == pos
            assert p["sorted_pair"][pos:pos + len(members)].tolist() == members
            pos += len(members)
        assert p["offsets"][E] == T * k
        assert (p["sorted_pair"][p["pair_pos"]] == np.arange(T * k)).all()
        assert p["active"].tolist() == sorted(set(ids.reshape(-1).tolist()))


def test_rmsnorm_removes_per_token_weight_scale():
    """RMSNorm acts on the combined output, so scaling a token's routing weights by
    c > 0 leaves the output unchanged when eps = 0 (REAP section, caveat paragraph)."""
    wl, x, d, b, st = _tiny()
    cache = layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()})
    r = layer.layer_forward(x, d, b, cache, wl.shape, eps=0.0, keep=True)
    c = np.array([0.5, 2.0, 3.0, 0.25, 1.0, 4.0, 0.7, 1.3])[:, None]
    y2 = layer.combine(r["Y_pair"], r["weights"] * c)
    out2 = layer.up_proj(layer.rmsnorm(y2, d["gamma"], eps=0.0), d["w_up"]) + r["shared"]
    rms = np.sqrt(np.mean(r["out"] ** 2))
    assert np.abs(out2 - r["out"]).max() < 1e-12 * rms
    # without the norm the same scaling is plainly visible
    assert np.abs(y2 - r["y"]).max() > 0.1 * np.abs(r["y"]).max()
    # with eps > 0 the norm's scale is 1/sqrt(mean(y^2) + eps): check that closed form
    y = r["y"]
    ms = np.mean(y * y, axis=1, keepdims=True)
    np.testing.assert_allclose(layer.rmsnorm(y, d["gamma"], 1e-6) * np.sqrt(ms + 1e-6), y, rtol=1e-13)


def test_pruning_equivalence_and_rotated_router_detected():
    """A pruned layer (experts renumbered: new i = old keep[i], router rows and bias
    reordered) equals the full layer with the dropped experts' bias at -inf;
    a router whose rows are rotated is caught (REAP section)."""
    wl, x, d, b, st = _tiny()
    sh = wl.shape
    E = sh.n_experts
    rng = np.random.default_rng(11)
    keep = np.sort(rng.choice(E, 20, replace=False))
    b_inf = b.copy()
    b_inf[np.setdiff1d(np.arange(E), keep)] = -np.inf
    full = layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()})
    r_full = layer.layer_forward(x, d, b_inf, full, sh)
    sub = {k: v[keep] for k, v in st.items()}
    d_sub = dict(d)
    d_sub["w_router"] = d["w_router"][keep]
    sh_sub = synth.LayerShape(sh.hidden, sh.latent, len(keep), sh.top_k, sh.inter, sh.n_shared, sh.shared_inter)
    cache_sub = layer.ExpertCache(lambda e: {k: v[e] for k, v in sub.items()})
    r_sub = layer.layer_forward(x, d_sub, b[keep], cache_sub, sh_sub)
    assert (keep[r_sub["ids"]] == r_full["ids"]).all()
    assert (r_sub["out"] == r_full["out"]).all()
    # identity prune is a bitwise no-op
    r_id = layer.layer_forward(x, d, b, full, sh)
    ident = np.arange(E)
    d_id = dict(d)
    d_id["w_router"] = d["w_router"][ident]
    r_id2 = layer.layer_forward(x, d_id, b[ident], layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()}), sh)
    assert (r_id["out"] == r_id2["out"]).all()
    # rotating the router rows (bias not rotated) changes the routing
    d_rot = dict(d_sub)
    d_rot["w_router"] = np.roll(d_sub["w_router"], 1, axis=0)
    r_rot = layer.layer_forward(x, d_rot, b[keep], cache_sub, sh_sub)
    assert not (r_rot["ids"] == r_sub["ids"]).all()


def test_zero_codes_leave_only_shared():
    wl, x, d, b, st = _tiny()
    zero = {k: (np.zeros_like(v) if k.endswith("packed") else v) for k, v in st.items()}
    cache = layer.ExpertCache(lambda e: {k: v[e] for k, v in zero.items()})
    r = layer.layer_forward(x, d, b, cache, wl.shape)
    assert (r["routed"] == 0).all()
    assert (r["out"] == r["shared"]).all()
    assert np.abs(r["shared"]).max() > 0


def test_shared_experts_concatenated_glu_identity():
    """Two GLUs of width Is summed == one GLU over the concatenated rows/columns."""
    wl = synth.workload("decode")
    sh = wl.shape
    rng = np.random.default_rng(2)
    H, Is, S = 64, 32, sh.n_shared
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, H)).astype(np.float32))
    g = synth.f32_to_bf16_bits(rng.standard_normal((S * Is, H)).astype(np.float32) * 0.1)
    u = synth.f32_to_bf16_bits(rng.standard_normal((S * Is, H)).astype(np.float32) * 0.1)
    dn = synth.f32_to_bf16_bits(rng.standard_normal((H, S * Is)).astype(np.float32) * 0.1)
    ref = layer.shared_experts(x, g, u, dn, S, Is)
    xf = layer.bf16_to_f64(x)
    one = layer.situ_glu(xf @ layer.bf16_to_f64(g).T, xf @ layer.bf16_to_f64(u).T) @ layer.bf16_to_f64(dn).T
    np.testing.assert_allclose(one, ref, rtol=1e-12, atol=1e-12)
    # and it is not a single expert's output
    single = layer.shared_experts(x, g[:Is], u[:Is], dn[:, :Is], 1, Is)
    assert np.abs(single - ref).max() > 1e-3


def test_threaded_expert_map_and_pair_layout():
    """The per-expert step may run under a thread pool's map: same result bit for
    bit as the serial loop.  H_pair / Y_pair hold each pair's rows in pair order,
    the rows H_sorted / Y_sorted hold at that pair's sorted position."""
    from concurrent.futures import ThreadPoolExecutor
    wl, x, d, b, st = _tiny()
    sh = wl.shape
    cache = layer.ExpertCache(lambda e: {k: v[e] for k, v in st.items()})
    r = layer.layer_forward(x, d, b, cache, sh, keep=True)
    with ThreadPoolExecutor(4) as ex:
        r2 = layer.layer_forward(x, d, b, cache, sh, keep=True, map_fn=ex.map)
    for key in ("out", "H_sorted", "Y_sorted", "H_pair", "Y_pair"):
        assert np.array_equal(r[key], r2[key]), key
    pos = r["perm"]["pair_pos"]
    k = sh.top_k
    assert np.array_equal(r["H_pair"].reshape(-1, sh.inter), r["H_sorted"][pos])
    assert np.array_equal(r["Y_pair"].reshape(-1, sh.latent), r["Y_sorted"][pos])
    # the pair order is p = t*k + j: token t's slot j
    t, j = 5, 2
    assert np.array_equal(r["H_pair"][t, j], r["H_sorted"][pos[t * k + j]])
