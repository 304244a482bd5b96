"""Benchmark: one forward pass of the Stable LatentMoE layer per step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill] [--no-cpu-baseline]

A step is one pass of the whole layer (moe_route, moe_permute, gate/up and
down grouped MXFP4 GEMMs, combine + RMSNorm + up_proj, shared experts) over
one batch of seeded synthetic tokens at full Kimi K3 shapes; inputs and
weights are resident in HBM before timing starts.  Prints one JSON line.

Fields beyond the headline: `roofline` for the dominant kernel (the gate/up
grouped GEMM: HBM-bound at decode, MFMA-bound at prefill), its duration taken
from HIP events recorded on the launch stream around that call in every timed
step; `cpu_baseline` = the CPU oracle timed on a bounded sample of the same
workload on this host; `secondary` = the prefill (T=4096) line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def _expert_gateup_bytes(sh) -> int:
    """w1 + w3 checkpoint bytes of one expert (packed + scales)."""
    return 2 * (sh.inter * sh.latent // 2 + sh.inter * sh.latent // 32)


def _expert_bytes(sh) -> int:
    return _expert_gateup_bytes(sh) + sh.latent * sh.inter // 2 + sh.latent * sh.inter // 32


def run_workload(mx, torch, synth, w, wl, steps, warmup):
    from synth.device import upload_tokens
    dev = torch.device("cuda:0")
    sh = wl.shape
    moe = mx.LatentMoE(mx.shape_of(sh), w, dev)
    x = upload_tokens(wl, dev)
    for _ in range(warmup):
        moe.forward(x)
    torch.cuda.synchronize()
    marks_all = []
    t0 = time.perf_counter()
    for _ in range(steps):
        marks = []
        moe.forward(x, marks=marks)
        marks_all.append(marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call durations from the events recorded on the launch stream
    names = [n for n, _ in marks_all[0][1:]]
    per_call = {n: 0.0 for n in names}
    for marks in marks_all:
        for (n0, e0), (n1, e1) in zip(marks[:-1], marks[1:]):
            per_call[n1] += e0.elapsed_time(e1) / steps
    b = moe.buffers(wl.tokens)
    e_act = int(b["active"][0].item())
    return {"wall_s": wall, "per_call_ms": per_call, "e_act": e_act, "T": wl.tokens}


def cpu_baseline(synth, wl, n_tokens):
    """The float64 oracle as it stands, on the first n_tokens tokens of the workload."""
    from oracle import layer
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    x_bits = synth.gen_tokens(wl, n_tokens)
    d = synth.gen_dense(wl)
    bias = synth.gen_bias(wl)

    def fetch(e):
        out = {}
        for m in ("w1", "w3", "w2"):
            p, s = synth.gen_expert(wl, e, m)
            out[m + "_packed"], out[m + "_scale"] = p, s
        return out

    cache = layer.ExpertCache(fetch, max_items=4 * wl.shape.top_k)
    t0 = time.perf_counter()
    layer.layer_forward(x_bits, d, bias, cache, wl.shape)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_tokens} of the {wl.tokens} tokens of the {wl.name} workload, float64 numpy "
                      f"oracle (expert dequantisation included), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU expert parallelism "
              "is not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp4_latent_moe_amd as mx
    import synth
    from synth.device import upload_weights

    mx.load()
    print("bench: uploading the full K3 weight set", file=sys.stderr, flush=True)
    wl = synth.workload(args.workload)
    sh = wl.shape
    w = upload_weights(wl, torch.device("cuda:0"))
    torch.cuda.synchronize()
    print("bench: timing", wl.name, file=sys.stderr, flush=True)
    r = run_workload(mx, torch, synth, w, wl, args.steps, args.warmup)
    ms = 1e3 * r["wall_s"] / args.steps
    value = wl.tokens * args.steps / r["wall_s"]

    gu_ms = r["per_call_ms"]["grouped_gemm_gateup"]
    P = wl.tokens * sh.top_k
    if args.workload == "decode":
        # algorithmic bytes of the gate/up grouped GEMM: w1+w3 of every active
        # expert, the latent rows read once, H written once
        traffic = r["e_act"] * _expert_gateup_bytes(sh) + wl.tokens * sh.latent * 4 + P * sh.inter * 4
        achieved = traffic / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "mxfp4_grouped_gemm gate/up (+SiTU-GLU)", "algorithmic_bytes": int(traffic),
                "avg_ms": round(gu_ms, 4), "active_experts": r["e_act"]}
    else:
        flops = 2.0 * P * sh.latent * sh.inter * 2
        achieved = flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "mxfp4_grouped_gemm gate/up (+SiTU-GLU)", "algorithmic_flops": flops,
                "avg_ms": round(gu_ms, 4)}

    line = {
        "metric": "MoE-layer tokens/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: one Stable LatentMoE layer forward, T={wl.tokens} tokens, "
                        f"H={sh.hidden}, L={sh.latent}, E={sh.n_experts}, top-{sh.top_k}, I={sh.inter}, "
                        f"{sh.n_shared} shared experts of {sh.shared_inter}",
            "tokens": wl.tokens,
            "operands": "MXFP4 expert weights (checkpoint bytes), bf16 dense weights, "
                        "bf16 hi+lo split activations, fp32 accumulate, fp32 output",
            "parallelism": "single GPU",
        },
        "per_call_ms": {k: round(v, 4) for k, v in r["per_call_ms"].items()},
        "roofline": roof,
    }
    if args.workload == "decode":
        line["expert_weight_bytes_per_step"] = r["e_act"] * _expert_bytes(sh)
        line["expert_hbm_frac_layer"] = round(
            r["e_act"] * _expert_bytes(sh) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    if not args.no_secondary and args.workload == "decode":
        pf = synth.workload("prefill")
        print("bench: timing prefill", file=sys.stderr, flush=True)
        rp = run_workload(mx, torch, synth, w, pf, max(2, args.steps // 5), 2)
        pms = 1e3 * rp["wall_s"] / max(2, args.steps // 5)
        layer_flops = 2.0 * pf.tokens * (sh.top_k * 3 * sh.latent * sh.inter + sh.n_experts * sh.hidden
                                         + 2 * sh.latent * sh.hidden
                                         + 3 * sh.n_shared * sh.shared_inter * sh.hidden)
        gu = rp["per_call_ms"]["grouped_gemm_gateup"]
        gu_flops = 2.0 * pf.tokens * sh.top_k * sh.latent * sh.inter * 2
        line["secondary"] = {
            "workload": "prefill T=4096, same shapes and weights",
            "tokens_per_s": round(pf.tokens / (pms * 1e-3), 1),
            "ms_per_step": round(pms, 3),
            "layer_tflops_algorithmic": round(layer_flops / (pms * 1e-3) / 1e12, 1),
            "layer_mfma_frac_algorithmic": round(layer_flops / (pms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "gateup_tflops": round(gu_flops / (gu * 1e-3) / 1e12, 1),
            "per_call_ms": {k: round(v, 4) for k, v in rp["per_call_ms"].items()},
        }

    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(synth, wl, 8 if args.workload == "decode" else 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
