"""Benchmark: one forward pass of the Stable LatentMoE layer per step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill] [--no-cpu-baseline]
    python bench.py --summarize-trace DIR            # rocprofv3 --kernel-trace --stats csv -> text
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR  # two --pmc runs -> traffic summary

A step is one pass of the whole layer (moe_route, moe_permute, gate/up and
down grouped MXFP4 GEMMs, combine + RMSNorm + up_proj, shared experts) over
one batch of seeded synthetic tokens at full Kimi K3 shapes; inputs and
weights are resident in HBM before timing starts.  The steps rotate through
--layers device copies of the weights (default 4, 64 GB), like consecutive
layers of the model.  Prints one JSON line.

Fields beyond the headline: `roofline` for the dominant kernel (the gate/up
grouped GEMM: HBM-bound at decode, MFMA-bound at prefill), its duration taken
from HIP events recorded on the launch stream around that call in every timed
step (the only events in the timed loop); `per_call_ms` from a separate loop
with events around every call; `cpu_baseline` = the CPU oracle timed on a bounded sample of the same
workload on this host; `secondary` = the prefill (T=4096) line; `cold_cache`
= the same layer timed with a 512 MiB write before every step, so that no
weight is served from the 256 MB last-level cache.

`roofline.traffic` is the HBM traffic of one launch of the dominant kernel as
read by the FETCH_SIZE and WRITE_SIZE counters (two rocprofv3 --pmc runs of
this script with --calibrate-copy), each scaled by what the same counter reads
for a plain copy of known size in the same run.  It is taken from the text
summary under profiles/ and reported only while the kernel's sources still
hash to the value recorded there.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FLUSH_BYTES = 512 << 20         # > the 256 MB last-level (MALL) cache
COPY_BYTES = 1 << 30            # calibration copy: reads and writes this many bytes

# Sources of the decode gate/up kernel: the traffic figure is valid only for them.
DECODE_GATEUP_SOURCES = ["mxfp4_latent_moe_amd/csrc/grouped_stream.hip", "mxfp4_latent_moe_amd/csrc/common.h",
                         "mxfp4_latent_moe_amd/csrc/kernels.h"]
DECODE_GATEUP_KERNEL = "grouped_stream_kernel<1, true"
PMC_SUMMARY = "profiles/grouped_gemm_gateup_decode_T16_traffic.txt"


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_summary(path) -> dict:
    out = {}
    full = os.path.join(ROOT, path)
    if not os.path.exists(full):
        return out
    for line in open(full):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def measured_traffic():
    """HBM bytes per launch of the decode gate/up kernel from the committed
    counter summary, or None when the kernel changed since it was taken."""
    d = read_summary(PMC_SUMMARY)
    if not d or d.get("source_sha256") != sources_sha256(DECODE_GATEUP_SOURCES):
        return None
    return int(float(d["traffic_bytes_per_launch"]))


def _expert_gateup_bytes(sh) -> int:
    """w1 + w3 checkpoint bytes of one expert (packed + scales)."""
    return 2 * (sh.inter * sh.latent // 2 + sh.inter * sh.latent // 32)


def _expert_bytes(sh) -> int:
    return _expert_gateup_bytes(sh) + sh.latent * sh.inter // 2 + sh.latent * sh.inter // 32


def _span(marks):
    """Milliseconds from the first call's start to the last call's end."""
    first = marks[0][1]
    return max(first.elapsed_time(e1) for _, _, e1 in marks)


def _pct(v, q):
    return round(float(np.percentile(np.asarray(v), q)), 4)


DOMINANT = "grouped_gemm_gateup"


def run_workload(mx, torch, synth, layers, wl, steps, warmup, cold_steps=0, breakdown_steps=10, operand_mode=0):
    """Step i runs layer i % len(layers): consecutive steps read different
    weight copies, as consecutive layers of the model do, so no step finds the
    previous step's weights in the last-level cache.

    The timed loop records HIP events only around the dominant call (on its
    stream), so timing adds almost nothing to the step; the per-call
    breakdown comes from a separate loop with events around every call."""
    from synth.device import upload_tokens
    dev = torch.device("cuda:0")
    sh = wl.shape
    moes = [mx.LatentMoE(mx.shape_of(sh, operand_mode), w, dev) for w in layers]
    x = upload_tokens(wl, dev)
    for i in range(warmup):
        moes[i % len(moes)].forward(x)
    torch.cuda.synchronize()
    dom = []
    t0 = time.perf_counter()
    for i in range(steps):
        moes[i % len(moes)].forward(x, marks=dom, mark_names=(DOMINANT,))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = [e0.elapsed_time(e1) for _, e0, e1 in dom]

    # per-call breakdown (events around every call; a little slower than the timed loop)
    marks_all = []
    for i in range(breakdown_steps):
        marks = []
        moes[i % len(moes)].forward(x, marks=marks)
        marks_all.append(marks)
    torch.cuda.synchronize()
    per_call = {n: 0.0 for n, _, _ in marks_all[0]}
    spans = []
    for marks in marks_all:
        for n, e0, e1 in marks:
            per_call[n] += e0.elapsed_time(e1) / len(marks_all)
        spans.append(_span(marks))
    b = moes[0].buffers(wl.tokens)
    e_act = int(b["active"][0].item())
    r = {"wall_s": wall, "per_call_ms": per_call, "e_act": e_act, "T": wl.tokens,
         "dominant_ms": float(np.mean(dom_ms)),
         "step_ms": {"median": _pct(spans, 50), "p10": _pct(spans, 10), "p90": _pct(spans, 90)}}
    if cold_steps > 0:
        # every step after a write of FLUSH_BYTES: nothing is left in the last-level cache
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        cold = []
        for i in range(cold_steps):
            scratch.fill_(float(i))
            marks = []
            moes[0].forward(x, marks=marks)
            cold.append(marks)
        torch.cuda.synchronize()
        cspans = [_span(m) for m in cold]
        r["cold_cache"] = {"flush_bytes": FLUSH_BYTES, "steps": cold_steps, "median_ms": _pct(cspans, 50),
                           "p10_ms": _pct(cspans, 10), "p90_ms": _pct(cspans, 90),
                           "tokens_per_s": round(wl.tokens / (float(np.median(cspans)) * 1e-3), 1)}
        del scratch
    return r


def calibration_copy(torch):
    """A plain elementwise copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES),
    run three times so the counters of a known-size transfer sit beside the
    layer's kernels in the same profile."""
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _short(name: str) -> str:
    return name.replace("moe::(anonymous namespace)::", "").replace("(moe::GemmArgs)", "").replace("void ", "")


def summarize_trace(d):
    """Kernel-trace --stats csv of one rocprofv3 run -> short text table."""
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        sys.exit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(f[0])))
    print(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in rows:
        print(f"{_short(r['Name'])[:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
              f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")


def _pmc_per_kernel(d, counter):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        sys.exit(f"no counter_collection.csv under {d}")
    acc = {}
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def summarize_pmc(fetch_dir, write_dir):
    """Two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) -> traffic summary.
    The scale of each counter is the copy's known byte count over what the
    counter read for it."""
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")

    def pick(acc, key):
        ks = [k for k in acc if key in k]
        if not ks:
            sys.exit(f"no dispatch of {key!r}")
        v = [x for k in ks for x in acc[k]]
        return sum(v) / len(v), len(v), _short(ks[0])

    copy_key = "elementwise"  # torch's mul kernel (the calibration copy)
    cf = [v for k in fetch if copy_key in k for v in fetch[k] if v * 1024 > COPY_BYTES / 4]
    cw = [v for k in write if copy_key in k for v in write[k] if v * 1024 > COPY_BYTES / 4]
    if not cf or not cw:
        sys.exit("calibration copy not found (run bench.py with --calibrate-copy)")
    f_scale = COPY_BYTES / (1024.0 * sum(cf) / len(cf))
    w_scale = COPY_BYTES / (1024.0 * sum(cw) / len(cw))
    kf, nf, kname = pick(fetch, DECODE_GATEUP_KERNEL)
    kw, nw, _ = pick(write, DECODE_GATEUP_KERNEL)
    traffic = kf * 1024 * f_scale + kw * 1024 * w_scale
    print("# HBM traffic of the decode gate/up grouped GEMM kernel (T=16, full K3 shapes)")
    print("# made by:")
    print("#   cd /tmp && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o run -- "
          "python3 <repo>/bench.py --steps 3 --warmup 1 --no-secondary --no-cpu-baseline --calibrate-copy")
    print("#   cd /tmp && timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o run -- "
          "python3 <repo>/bench.py --steps 3 --warmup 1 --no-secondary --no-cpu-baseline --calibrate-copy")
    print("#   python3 bench.py --summarize-pmc <F> <W>")
    print(f"kernel: {kname}")
    print(f"source_sha256: {sources_sha256(DECODE_GATEUP_SOURCES)}")
    print(f"copy_bytes: {COPY_BYTES}")
    print(f"copy_fetch_kib_per_dispatch: {sum(cf) / len(cf):.1f}")
    print(f"copy_write_kib_per_dispatch: {sum(cw) / len(cw):.1f}")
    print(f"fetch_scale: {f_scale:.4f}")
    print(f"write_scale: {w_scale:.4f}")
    print(f"kernel_fetch_kib_per_dispatch: {kf:.1f}  (n={nf})")
    print(f"kernel_write_kib_per_dispatch: {kw:.1f}  (n={nw})")
    print(f"traffic_bytes_per_launch: {traffic:.0f}")


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


def run_dense_ffn(mx, torch, synth):
    """The first layer's dense FFN (H = 7168, intermediate 33792, bf16) through shared_expert_ffn:
    decode T = 16 against HBM (its 1.45 GB of weights stream once per call, far more than the
    last-level cache holds) and prefill T = 4096 against bf16 MFMA."""
    from synth.device import to_dev_bf16
    from mxfp4_latent_moe_amd import _lib, ops
    dev = torch.device("cuda:0")
    wl = synth.workload("dense_ffn")
    sh = wl.shape
    d = synth.gen_dense(wl)
    w = {k: to_dev_bf16(d[k], dev) for k in ("sh_gate", "sh_up", "sh_down")}
    del d
    s = mx.shape_of(sh)
    wbytes = 3 * sh.shared_inter * sh.hidden * 2
    res = {"workload": "layer-0 dense FFN, H=7168, intermediate 33792, bf16 weights, SiTU-GLU"}
    for T, steps in ((16, 20), (4096, 5)):
        x = to_dev_bf16(synth.gen_tokens(wl, T), dev)
        ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_SHARED_FFN, T), dtype=torch.uint8, device=dev)
        out = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
        for _ in range(3):
            ops.shared_ffn(s, x, w["sh_gate"], w["sh_up"], w["sh_down"], out, 0, ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            ops.shared_ffn(s, x, w["sh_gate"], w["sh_up"], w["sh_down"], out, 0, ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        if T == 16:
            gbs = wbytes / (ms * 1e-3) / 1e9
            res["decode_T16"] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                                 "weight_bytes": wbytes, "gb_per_s": round(gbs, 1),
                                 "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            tf = 2.0 * T * sh.hidden * sh.shared_inter * 3 / (ms * 1e-3) / 1e12
            res["prefill_T4096"] = {"ms": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
                                    "tflops": round(tf, 1), "mfma_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}
        del x, ws, out
    return res


def run_reap(mx, torch, synth):
    """REAP saliency over one prefill batch (4096 tokens x top-16, L = 3584): the pass reads every
    expert-output row once (940 MB), so it is timed against HBM."""
    from mxfp4_latent_moe_amd import _lib, ops
    dev = torch.device("cuda:0")
    sh = synth.K3_SHAPE
    T, k, E, L = 4096, sh.top_k, sh.n_experts, sh.latent
    P = T * k
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    ids = torch.randint(0, E, (P,), device=dev, generator=g, dtype=torch.int32)
    sorted_pair = torch.sort(ids, stable=True).indices.to(torch.int32)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    offsets[1:] = torch.cumsum(torch.bincount(ids, minlength=E), 0).to(torch.int32)
    Y = torch.randn((P, L), device=dev, generator=g, dtype=torch.float32)
    w = torch.rand((P,), device=dev, generator=g, dtype=torch.float32)
    s = mx.shape_of(sh)
    ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_REAP_SALIENCY, P), dtype=torch.uint8, device=dev)
    sal = torch.zeros(E, dtype=torch.float64, device=dev)
    cnt = torch.zeros(E, dtype=torch.int64, device=dev)
    for _ in range(3):
        ops.reap_saliency(s, P, offsets, Y, w, sorted_pair, sal, cnt, 1, ws)
    steps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ops.reap_saliency(s, P, offsets, Y, w, sorted_pair, sal, cnt, 1, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = P * L * 4 + P * 16 + E * 20
    gbs = nbytes / (ms * 1e-3) / 1e9

    # the same sums fused into the combine (moe_combine_norm_up_reap), timed
    # against the plain combine + RMSNorm + up_proj over the same batch
    pair_pos = torch.empty_like(sorted_pair)
    pair_pos[sorted_pair.long()] = torch.arange(P, device=dev, dtype=torch.int32)
    gamma = torch.ones(L, device=dev, dtype=torch.bfloat16)
    w_up = (torch.randn((sh.hidden, L), device=dev, generator=g) * L ** -0.5).to(torch.bfloat16)
    out = torch.empty((T, sh.hidden), device=dev, dtype=torch.float32)
    wsc = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP_REAP, T), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    plain_ms = timed(lambda: ops.combine_norm_up(s, T, Y, pair_pos, w, gamma, w_up, out, 0, wsc))
    fused_ms = timed(lambda: ops.combine_norm_up_reap(s, T, Y, pair_pos, w, gamma, w_up, out, 0, offsets, sal,
                                                      cnt, 1, wsc))
    return {"workload": "REAP saliency, 4096 tokens x top-16 over 896 experts, L=3584, synthetic rows",
            "ms": round(ms, 4), "bytes": nbytes, "gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "fused_into_combine": {"combine_norm_up_ms": round(plain_ms, 4), "with_reap_ms": round(fused_ms, 4),
                                   "reap_extra_ms": round(fused_ms - plain_ms, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill"])
    ap.add_argument("--operand-mode", default="bf16x2", choices=["bf16x2", "mx8x3", "mx6x3"],
                    help="operand mode of the timed workload (the decode line's prefill extras cover all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--layers", type=int, default=4,
                    help="weight copies the steps rotate through (16 GB each at full shape)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps of one layer timed after a cache flush (0: none)")
    ap.add_argument("--calibrate-copy", action="store_true", help="run a known-size copy for counter scaling")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU expert parallelism "
              "is not implemented", file=sys.stderr)
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
    layers = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(max(1, args.layers) - 1)]
    torch.cuda.synchronize()
    print("bench: timing", wl.name, file=sys.stderr, flush=True)
    opnd = {"bf16x2": mx.MOE_OPND_BF16X2, "mx8x3": mx.MOE_OPND_MX8X3, "mx6x3": mx.MOE_OPND_MX6X3}[args.operand_mode]
    r = run_workload(mx, torch, synth, layers, wl, args.steps, args.warmup, args.cold_steps, operand_mode=opnd)
    ms = 1e3 * r["wall_s"] / args.steps
    value = wl.tokens * args.steps / r["wall_s"]

    gu_ms = r["dominant_ms"]  # events around the gate/up call in every timed step
    P = wl.tokens * sh.top_k
    if args.workload == "decode":
        # algorithmic bytes of the gate/up grouped GEMM: w1+w3 of every active
        # expert, the latent rows read once, H written once
        traffic = r["e_act"] * _expert_gateup_bytes(sh) + wl.tokens * sh.latent * 4 + P * sh.inter * 4
        achieved = traffic / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
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
                        + {"bf16x2": "bf16 hi+lo split activations",
                           "mx8x3": "expert GEMM activations as three e4m3 terms, other activations bf16 hi+lo",
                           "mx6x3": "expert GEMM activations as three e2m3 terms, other activations bf16 hi+lo"}[
                            args.operand_mode] + ", fp32 accumulate, fp32 output",
            "parallelism": "single GPU",
            "layers_rotated": len(layers),
        },
        "per_call_ms": {k: round(v, 4) for k, v in r["per_call_ms"].items()},
        "step_ms_with_call_events": r["step_ms"],
        "roofline": roof,
    }
    if "cold_cache" in r:
        line["cold_cache"] = r["cold_cache"]
    if args.workload == "decode":
        line["expert_weight_bytes_per_step"] = r["e_act"] * _expert_bytes(sh)
        line["expert_hbm_frac_layer"] = round(
            r["e_act"] * _expert_bytes(sh) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    if not args.no_secondary and args.workload == "decode":
        pf = synth.workload("prefill")
        print("bench: timing prefill", file=sys.stderr, flush=True)
        rp = run_workload(mx, torch, synth, layers, pf, max(2, args.steps // 5), 2, breakdown_steps=2)
        pms = 1e3 * rp["wall_s"] / max(2, args.steps // 5)
        layer_flops = 2.0 * pf.tokens * (sh.top_k * 3 * sh.latent * sh.inter + sh.n_experts * sh.hidden
                                         + 2 * sh.latent * sh.hidden
                                         + 3 * sh.n_shared * sh.shared_inter * sh.hidden)
        gu = rp["dominant_ms"]
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
        # the same prefill with the MX-scaled expert GEMMs (three fp8 activation terms)
        print("bench: timing prefill, MX fp8 operand mode", file=sys.stderr, flush=True)
        rm = run_workload(mx, torch, synth, layers, pf, max(2, args.steps // 5), 2, breakdown_steps=2,
                          operand_mode=mx.MOE_OPND_MX8X3)
        mms = 1e3 * rm["wall_s"] / max(2, args.steps // 5)
        line["secondary_mx8x3"] = {
            "workload": "prefill T=4096, expert GEMM activations as three e4m3 terms (operand mode MX8X3)",
            "tokens_per_s": round(pf.tokens / (mms * 1e-3), 1),
            "ms_per_step": round(mms, 3),
            "layer_tflops_algorithmic": round(layer_flops / (mms * 1e-3) / 1e12, 1),
            "layer_mfma_frac_algorithmic": round(layer_flops / (mms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "gateup_tflops": round(gu_flops / (rm["dominant_ms"] * 1e-3) / 1e12, 1),
            "per_call_ms": {k: round(v, 4) for k, v in rm["per_call_ms"].items()},
        }

        # and with three fp6 (e2m3) activation terms, which the MX MFMA runs at the fp4 rate
        print("bench: timing prefill, MX fp6 operand mode", file=sys.stderr, flush=True)
        r6 = run_workload(mx, torch, synth, layers, pf, max(2, args.steps // 5), 2, breakdown_steps=2,
                          operand_mode=mx.MOE_OPND_MX6X3)
        m6 = 1e3 * r6["wall_s"] / max(2, args.steps // 5)
        line["secondary_mx6x3"] = {
            "workload": "prefill T=4096, expert GEMM activations as three e2m3 terms (operand mode MX6X3)",
            "tokens_per_s": round(pf.tokens / (m6 * 1e-3), 1),
            "ms_per_step": round(m6, 3),
            "layer_tflops_algorithmic": round(layer_flops / (m6 * 1e-3) / 1e12, 1),
            "layer_mfma_frac_algorithmic": round(layer_flops / (m6 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "gateup_tflops": round(gu_flops / (r6["dominant_ms"] * 1e-3) / 1e12, 1),
            "per_call_ms": {k: round(v, 4) for k, v in r6["per_call_ms"].items()},
        }

        print("bench: timing the layer-0 dense FFN", file=sys.stderr, flush=True)
        line["secondary_dense_ffn"] = run_dense_ffn(mx, torch, synth)
        print("bench: timing the REAP saliency pass", file=sys.stderr, flush=True)
        line["secondary_reap"] = run_reap(mx, torch, synth)

    if args.calibrate_copy:
        calibration_copy(torch)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(synth, wl, 8 if args.workload == "decode" else 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
