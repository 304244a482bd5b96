"""The first layer's dense FFN (H = 7168, intermediate 33792, bf16 weights, SiTU-GLU) through
shared_expert_ffn as one expert of that width: decode (T = 16, streaming kernels) and prefill
(T = 4096, tiled kernels), against the float64 oracle on sampled tokens."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from synth.device import to_dev_bf16
from oracle import layer
from gpu_common import rel_max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ffn():
    import mxfp4_latent_moe_amd as mx
    mx.load()
    wl = synth.workload("dense_ffn")
    say("fixture: generating the dense FFN weights (3 x 242M bf16)")
    d = synth.gen_dense(wl)
    dev = torch.device("cuda:0")
    w = {k: to_dev_bf16(d[k], dev) for k in ("sh_gate", "sh_up", "sh_down")}
    return mx, wl, w, d


@pytest.mark.parametrize("T,rows", [(16, [0, 7, 15]), (4096, [0, 1234, 2999, 4095])])
def test_dense_ffn_layer0(ffn, T, rows):
    from mxfp4_latent_moe_amd import _lib, ops
    mx, wl, w, d = ffn
    sh = wl.shape
    dev = torch.device("cuda:0")
    x_bits = synth.gen_tokens(wl, T)
    say(f"case: layer-0 dense FFN, T={T}, H={sh.hidden}, intermediate {sh.shared_inter}")
    s = mx.shape_of(sh)
    ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_SHARED_FFN, T), dtype=torch.uint8, device=dev)
    out = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
    ops.shared_ffn(s, to_dev_bf16(x_bits, dev), w["sh_gate"], w["sh_up"], w["sh_down"], out, 0, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[rows]
    ref = layer.shared_experts(x_bits[np.asarray(rows)], d["sh_gate"], d["sh_up"], d["sh_down"],
                               sh.n_shared, sh.shared_inter)
    err = rel_max_err(got, ref)
    say(f"dense FFN T={T}: max|gpu-oracle|/rms over rows {rows} = {err:.3e}")
    assert err <= 1e-4
