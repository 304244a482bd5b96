"""Upload of the seeded synthetic inputs to a torch device (plumbing only).

Expert stacks are generated and copied in slices so that host memory stays at
a few GB even for the 15.7 GB full-shape stack.
"""
from __future__ import annotations

import numpy as np
import torch

from .inputs import Workload, gen_bias, gen_dense, gen_expert_stack, gen_tokens


def to_dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device` (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_experts(wl: Workload, device, slice_experts: int = 32) -> dict:
    sh = wl.shape
    E = sh.n_experts
    dims = {"w1": (sh.inter, sh.latent), "w3": (sh.inter, sh.latent), "w2": (sh.latent, sh.inter)}
    out = {}
    for w, (N, K) in dims.items():
        out[w + "_packed"] = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
        out[w + "_scale"] = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device)
    for e0 in range(0, E, slice_experts):
        ids = range(e0, min(E, e0 + slice_experts))
        st = gen_expert_stack(wl, ids)
        for k, v in st.items():
            out[k][e0:e0 + len(ids)].copy_(torch.from_numpy(v))
    return out


def upload_weights(wl: Workload, device, zipf_bias_path: str | None = None, experts: bool = True) -> dict:
    """Every weight of the layer on `device`; bf16 tensors carry the exact generated bits."""
    d = gen_dense(wl)
    w = {k: to_dev_bf16(v, device) for k, v in d.items()}
    w["bias"] = to_dev(gen_bias(wl, zipf_bias_path), device)
    if experts:
        w.update(upload_experts(wl, device))
    return w


def upload_tokens(wl: Workload, device, tokens: int | None = None) -> torch.Tensor:
    return to_dev_bf16(gen_tokens(wl, tokens), device)
