"""moe_permute through the C ABI against the oracle's stable counting sort
(kimi-k3-mlx README, REAP section, two-bank paragraph: pairs sorted by expert
index give each expert a contiguous slice).

Token counts on both sides of the single-workgroup path (T <= 64) and the
three-kernel path, the largest pair count the single-workgroup path holds
(64 tokens x top-32), and a degenerate routing where every token picks the
same experts.  Every output is unique, so all are compared exactly.
"""
import numpy as np
import pytest
import torch

from synth.device import to_dev
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


def _run(mx, E, k, ids):
    from mxfp4_latent_moe_amd import ops
    T = ids.shape[0]
    s = mx.shape_of(LayerShape(256, 128, E, k, 128, 0, 0))
    ws = torch.empty(ops.workspace_bytes(s, ops.MOE_FN_PERMUTE, T), dtype=torch.uint8, device=DEV)
    P = T * k
    out = {"offsets": torch.empty(E + 1, dtype=torch.int32, device=DEV),
           "sorted_pair": torch.empty(P, dtype=torch.int32, device=DEV),
           "pair_pos": torch.empty(P, dtype=torch.int32, device=DEV),
           "active": torch.empty(E + 1, dtype=torch.int32, device=DEV)}
    ops.permute(s, to_dev(ids, DEV), out["offsets"], out["sorted_pair"], out["pair_pos"], out["active"], ws)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in out.items()}


def _check(g, ref):
    assert np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["sorted_pair"], ref["sorted_pair"])
    assert np.array_equal(g["pair_pos"], ref["pair_pos"])
    n = int(g["active"][0])
    assert n == ref["active"].size and np.array_equal(g["active"][1:1 + n], ref["active"])


@pytest.mark.parametrize("E,k", [(896, 16), (1024, 32), (32, 4)])
@pytest.mark.parametrize("T", [1, 37, 63, 64, 65, 128, 300])
def test_permute_matches_oracle(mx, E, k, T):
    rng = np.random.default_rng(31 * T + E + k)
    say(f"case: moe_permute E={E} k={k} T={T}")
    ids = np.sort(np.argsort(rng.random((T, E)), axis=1)[:, :k], axis=1).astype(np.int32)
    _check(_run(mx, E, k, ids), layer.permute(ids, E))


@pytest.mark.parametrize("T", [64, 65])
def test_permute_all_tokens_same_experts(mx, T):
    E, k = 896, 16
    say(f"case: moe_permute, every token on experts 0..15, T={T}")
    ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    _check(_run(mx, E, k, ids), layer.permute(ids, E))
