"""Pins of the REAP saliency oracle against what the formula fixes (CPU)."""
import math

import numpy as np

from oracle import reap


def _loop_saliency(Y_pair, ids, weights, E):
    """Brute force: one pair at a time, the norm as an explicit square root of a sum."""
    T, k, L = Y_pair.shape
    sums = [0.0] * E
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            sq = 0.0
            for v in Y_pair[t, j]:
                sq += float(v) * float(v)
            sums[ids[t, j]] += float(weights[t, j]) * math.sqrt(sq)
            counts[ids[t, j]] += 1
    return np.array(sums), np.array(counts)


def _case(seed=0, T=9, k=3, L=5, E=7):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    w = rng.random((T, k))
    w /= w.sum(axis=1, keepdims=True)
    Y = rng.standard_normal((T, k, L))
    return Y, ids, w, E


def test_matches_brute_force():
    Y, ids, w, E = _case()
    r = reap.reap_saliency(Y, ids, w, E)
    s, c = _loop_saliency(Y, ids, w, E)
    np.testing.assert_allclose(r["sum"], s, rtol=1e-13, atol=1e-15)
    assert (r["count"] == c).all()
    np.testing.assert_allclose(r["S"], s / Y.shape[0], rtol=1e-13)


def test_closed_form_norms():
    """Expert outputs c * (a unit vector): g * ||e|| = g * |c| exactly."""
    T, k, L, E = 4, 2, 6, 3
    ids = np.array([[0, 1], [1, 2], [0, 2], [2, 1]])
    w = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, 0.0], [0.125, 0.875]])
    c = np.array([[2.0, -3.0], [4.0, 1.0], [-1.0, 5.0], [8.0, 0.5]])
    Y = np.zeros((T, k, L))
    for t in range(T):
        for j in range(k):
            Y[t, j, (t + j) % L] = c[t, j]
    r = reap.reap_saliency(Y, ids, w, E)
    want = np.zeros(E)
    for t in range(T):
        for j in range(k):
            want[ids[t, j]] += w[t, j] * abs(c[t, j])
    assert (r["sum"] == want).all()
    assert list(r["count"]) == [2, 3, 3]


def test_unrouted_expert_scores_zero_and_counts_sum():
    Y, ids, w, E = _case(seed=3, E=12)
    ids = ids % 6  # experts 6..11 never selected
    r = reap.reap_saliency(Y, ids, w, E)
    assert (r["sum"][6:] == 0).all() and (r["count"][6:] == 0).all()
    assert r["count"].sum() == ids.size


def test_scale_equivariance_and_token_order():
    Y, ids, w, E = _case(seed=5)
    r = reap.reap_saliency(Y, ids, w, E)
    r2 = reap.reap_saliency(-2.5 * Y, ids, w, E)
    np.testing.assert_allclose(r2["sum"], 2.5 * r["sum"], rtol=1e-13)
    p = np.random.default_rng(1).permutation(Y.shape[0])
    r3 = reap.reap_saliency(Y[p], ids[p], w[p], E)
    np.testing.assert_allclose(r3["sum"], r["sum"], rtol=1e-13)
    assert (r3["count"] == r["count"]).all()
