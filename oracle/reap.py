"""REAP expert saliency over a calibration batch (TEST INFRASTRUCTURE ONLY).

kimi-k3-mlx README, REAP section: each expert j is scored on a calibration
set C by S_j = (1/|C|) * sum over x in C of g_j(x) * ||e_j(x)||_2, where g_j(x)
is the router's gate for j on token x (zero when j is not among the token's
top-k) and e_j(x) the expert's output for x.  The section also notes that the
score of a layer depends only on that layer's input, router gates and expert
outputs, so a calibration pass streams one layer at a time.

Readings taken here (the pages print only the formula):
  * g_j(x) is the routing weight the layer combines the expert's output with
    (the selected sigmoid scores normalised to sum 1);
  * e_j(x) is the expert's un-weighted output in the latent (before the
    weighted combine and the RMSNorm);
  * |C| is the number of calibration tokens, as printed; the per-expert token
    counts are returned too, so the normalisation by the tokens routed to j
    (the REAP paper's form) is one division away.

The sums are float64.
"""
from __future__ import annotations

import numpy as np


def reap_saliency(Y_pair: np.ndarray, ids: np.ndarray, weights: np.ndarray, n_experts: int) -> dict:
    """Y_pair [T, k, L] un-weighted expert outputs, ids [T, k], weights [T, k] ->
    {"sum": [E] sum of g * ||e||, "count": [E] tokens routed to each expert, "S": sum / T}."""
    T, k, _ = Y_pair.shape
    norms = np.sqrt(np.sum(np.asarray(Y_pair, np.float64) ** 2, axis=2))  # [T, k]
    contrib = np.asarray(weights, np.float64) * norms
    sums = np.zeros(n_experts)
    counts = np.zeros(n_experts, np.int64)
    np.add.at(sums, ids.reshape(-1), contrib.reshape(-1))
    np.add.at(counts, ids.reshape(-1), 1)
    return {"sum": sums, "count": counts, "S": sums / T}
