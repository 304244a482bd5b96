"""moe_route_noalloc against moe_route through the C ABI, on one GPU.

The allocation-free variant runs the same kernels on a fixed per-device
scratch array instead of a caller workspace, so its ids, weights, latent and
gaps must equal moe_route's bit for bit.  Two calls in a row, the second with
fewer tokens, so the second finds the first call's contents in the scratch.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from synth.device import to_dev, to_dev_bf16
from gpu_common import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _p(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


@pytest.mark.parametrize("wl_name", ["decode", "tiny"])
def test_route_noalloc_matches_route(wl_name):
    from mxfp4_latent_moe_amd import _lib, ops
    lib = _lib.load()
    wl = synth.workload(wl_name)
    sh = wl.shape
    s = ops.shape_of(sh)
    d = synth.gen_dense(wl)
    w_router = to_dev_bf16(d["w_router"], DEV)
    w_down = to_dev_bf16(d["w_down"], DEV)
    bias = to_dev(synth.gen_bias(wl), DEV)
    x_all = synth.gen_tokens(wl, 64)
    stream = torch.cuda.current_stream().cuda_stream
    for T in (16, 5):
        say(f"case: {wl_name} moe_route_noalloc vs moe_route, T={T}")
        x = to_dev_bf16(x_all[:T], DEV)
        outs = []
        for noalloc in (False, True):
            ids = torch.full((T, sh.top_k), -1, dtype=torch.int32, device=DEV)
            w = torch.full((T, sh.top_k), -1.0, dtype=torch.float32, device=DEV)
            z = torch.full((T, sh.latent), -1.0, dtype=torch.float32, device=DEV)
            gap = torch.full((T,), -1.0, dtype=torch.float32, device=DEV)
            if noalloc:
                rc = lib.moe_route_noalloc(s, T, _p(x), _p(w_router), _p(bias), _p(w_down), _p(ids), _p(w), _p(z),
                                           _p(gap), ctypes.c_void_p(stream))
            else:
                ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_ROUTE, T), dtype=torch.uint8, device=DEV)
                rc = lib.moe_route(s, T, _p(x), _p(w_router), _p(bias), _p(w_down), _p(ids), _p(w), _p(z), _p(gap),
                                   _p(ws), ws.numel(), ctypes.c_void_p(stream))
            assert rc == _lib.MOE_OK, rc
            torch.cuda.synchronize()
            outs.append([t.cpu().numpy() for t in (ids, w, z, gap)])
        for a, b in zip(*outs):
            assert np.array_equal(a, b)
        assert (outs[1][0] >= 0).all()
