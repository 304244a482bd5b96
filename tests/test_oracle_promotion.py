"""Pins of the capped-promotion oracle (moe_k_hi; Kimi-K3-Alis-MLX-Dynamic
card, Build recipe: at most 4 promoted experts per token of the 16 routed, the
5th and later promoted expert's contribution dropped; about 1.7% of tokens per
layer at Binom(16, 0.1)).

Pinned by a hand-worked case, identities, and the drop rate under uniformly
random routing against the exact hypergeometric tail (a random 16-subset of
896 experts with 90 promoted), which the card's binomial figure approximates.
"""
import numpy as np
import pytest
from scipy.stats import binom, hypergeom

from oracle import layer
from oracle.promotion import cap_promoted


def _one_token(b, k):
    b = np.asarray([b], np.float32)
    scores = np.full_like(b, 0.5, dtype=np.float64)  # weights equal: the cap alone changes them
    r = layer.select_topk(scores, np.asarray(b[0]) - np.float32(0.5), k)
    return r["ids"], r["weights"], r["biased32"]


def test_hand_worked_case():
    # decision values of experts 0..9; the top 6 are 0, 2, 3, 5, 6, 9 (ascending slots)
    ids, w, b = _one_token([0.9, 0.1, 0.8, 0.7, 0.2, 0.6, 0.5, 0.3, 0.05, 0.4], 6)
    assert ids.tolist() == [[0, 2, 3, 5, 6, 9]]
    promoted = np.zeros(10, bool)
    promoted[[1, 2, 3, 6, 9]] = True  # 1 is promoted but not selected
    # routing order of the selected promoted experts: 2 (0.8), 3 (0.7), 6 (0.5), 9 (0.4)
    got = cap_promoted(ids, w, b, promoted, 2)
    assert np.array_equal(got[0] == 0, [False, False, False, False, True, True])  # 6 and 9 dropped
    assert np.allclose(got[0, :4], 1 / 6)  # the rest keep their weights: nothing re-normalised
    got = cap_promoted(ids, w, b, promoted, 3)
    assert np.array_equal(got[0] == 0, [False, False, False, False, False, True])  # only 9


def test_ties_go_to_the_lower_index():
    ids, w, b = _one_token([0.9, 0.1, 0.8, 0.7, 0.2, 0.7, 0.5, 0.3, 0.05, 0.4], 6)
    assert ids.tolist() == [[0, 2, 3, 5, 6, 9]]
    promoted = np.zeros(10, bool)
    promoted[[3, 5]] = True
    got = cap_promoted(ids, w, b, promoted, 1)
    assert got[0, 1] != 0 and got[0, 2] != 0 and got[0, 3] == 0  # 3 kept, 5 (same value) dropped


def test_identities():
    rng = np.random.default_rng(5)
    T, E, k = 64, 40, 8
    r = layer.select_topk(rng.random((T, E)), np.zeros(E, np.float32), k)
    promoted = rng.random(E) < 0.3
    assert np.array_equal(cap_promoted(r["ids"], r["weights"], r["biased32"], promoted, k), r["weights"])
    assert np.array_equal(cap_promoted(r["ids"], r["weights"], r["biased32"], np.zeros(E, bool), 0), r["weights"])
    none = cap_promoted(r["ids"], r["weights"], r["biased32"], promoted, 0)
    assert np.array_equal(none == 0, promoted[r["ids"]])


def test_drop_rate_matches_the_hypergeometric_tail():
    """Uniformly random routing (iid scores, no bias) picks a uniform 16-subset
    of 896; with 90 promoted experts the promoted count is Hypergeom(896, 90,
    16), so a token loses a contribution with probability P(X >= 5) and loses
    max(X - 4, 0) of them."""
    rng = np.random.default_rng(11)
    T, E, k, n_prom, k_hi = 20000, 896, 16, 90, 4
    r = layer.select_topk(rng.random((T, E)), np.zeros(E, np.float32), k)
    promoted = np.zeros(E, bool)
    promoted[rng.choice(E, n_prom, replace=False)] = True
    w = cap_promoted(r["ids"], r["weights"], r["biased32"], promoted, k_hi)
    X = promoted[r["ids"]].sum(axis=1)
    dropped = (w == 0).sum(axis=1)
    assert np.array_equal(dropped, np.maximum(X - k_hi, 0))
    kept_prom = ((w != 0) & promoted[r["ids"]]).sum(axis=1)
    assert np.array_equal(kept_prom, np.minimum(X, k_hi))
    hg = hypergeom(E, n_prom, k)
    p = hg.sf(k_hi)
    rate = (dropped > 0).mean()
    assert abs(rate - p) < 4 * np.sqrt(p * (1 - p) / T), (rate, p)
    xs = np.arange(k + 1)
    mean_dropped = (np.maximum(xs - k_hi, 0) * hg.pmf(xs)).sum()
    assert abs(dropped.mean() - mean_dropped) < 4 * np.sqrt(((np.maximum(xs - k_hi, 0) ** 2) * hg.pmf(xs)).sum() / T)
    # the card's figure is the binomial approximation of the same tail
    assert binom(k, 0.1).sf(k_hi) == pytest.approx(0.0170, abs=5e-5)
    assert abs(binom(k, 0.1).sf(k_hi) - p) < 1e-3
