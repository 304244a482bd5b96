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
