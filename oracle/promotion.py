"""Capped promotion (moe_k_hi), float64 CPU oracle (test infrastructure only).

avlp12 Kimi-K3-Alis-MLX-Dynamic card, Build recipe: the experts that matter
are kept in their original MXFP4 format ("promoted"), and the serving
configuration caps that path at moe_k_hi = 4 promoted experts per token of the
16 routed; a token's 5th and later promoted expert has its contribution
dropped rather than downgraded.

Readings where the card is silent (listed with their reasons in the design
notes of this repository):
  * "5th and later" is in routing order: the larger float32 biased decision
    value first, ties to the lower expert index (the order of the top-k);
  * dropping a contribution sets that pair's routing weight to 0; the other
    weights keep their normalisation over all k selected experts (nothing is
    re-weighted);
  * ids are unchanged, so the dropped pair is still routed (its product is
    multiplied by 0).
"""
from __future__ import annotations

import numpy as np


def cap_promoted(ids: np.ndarray, weights: np.ndarray, biased32: np.ndarray, promoted: np.ndarray,
                 k_hi: int) -> np.ndarray:
    """Routing weights with every token's promoted experts past the first k_hi
    (in routing order) set to zero.

    ids [T, k] selected experts (ascending), weights [T, k] their routing
    weights, biased32 [T, E] the float32 decision values the selection used,
    promoted [E] bool.  Returns a new weights array."""
    ids = np.asarray(ids)
    out = np.array(weights, dtype=np.float64, copy=True)
    T, k = ids.shape
    for t in range(T):
        prom = [j for j in range(k) if promoted[ids[t, j]]]
        prom.sort(key=lambda j: (-float(biased32[t, ids[t, j]]), int(ids[t, j])))
        for j in prom[k_hi:]:
            out[t, j] = 0.0
    return out
