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
FP8_MFMA_PEAK_TFLOPS = 5000.0   # dense fp8 (the fp4 x fp8 MX MFMA runs at this rate)
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense fp6 / fp4 (the fp4 x fp6 MX MFMA runs at this rate)
PREFILL_STEPS = 10              # timed steps of each prefill line
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


def run_workload(mx, torch, synth, layers, wl, steps, warmup, cold_steps=0, breakdown_steps=10, operand_mode=0,
                 bank_bs=None):
    """Step i runs layer i % len(layers): consecutive steps read different
    weight copies, as consecutive layers of the model do, so no step finds the
    previous step's weights in the last-level cache.

    The timed loop records no events (each HIP event record costs about 5 us
    of a decode step).  The same number of steps then runs again with HIP
    events around the dominant call and the down call (on their stream), for
    the kernels' average durations; the per-call breakdown comes from a third
    loop with events around every call."""
    from synth.device import upload_tokens
    dev = torch.device("cuda:0")
    sh = wl.shape
    if bank_bs is None:
        moes = [mx.LatentMoE(mx.shape_of(sh, operand_mode), w, dev) for w in layers]
    else:
        # two-bank layers: the MXFP4 tensors of the first E - n_b experts, then bank B
        n_a = sh.n_experts - int(bank_bs[0]["n_experts"])
        moes = [mx.LatentMoE(mx.shape_of(sh, operand_mode),
                             {k: (v[:n_a] if k[:2] in ("w1", "w3", "w2") else v) for k, v in w.items()}, dev,
                             bank_b=bb) for w, bb in zip(layers, bank_bs)]
    x = upload_tokens(wl, dev)
    for i in range(warmup):
        moes[i % len(moes)].forward(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moes[i % len(moes)].forward(x)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom = []
    t1 = time.perf_counter()
    for i in range(steps):
        moes[i % len(moes)].forward(x, marks=dom, mark_names=(DOMINANT, "grouped_gemm_down"))
    torch.cuda.synchronize()
    wall_marked = time.perf_counter() - t1
    dom_ms = [e0.elapsed_time(e1) for n, e0, e1 in dom if n == DOMINANT]
    down_ms = [e0.elapsed_time(e1) for n, e0, e1 in dom if n != DOMINANT]

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
    active_ids = b["active"][1:1 + e_act].cpu().numpy()
    r = {"wall_s": wall, "wall_marked_s": wall_marked, "per_call_ms": per_call, "e_act": e_act, "T": wl.tokens, "active_ids": active_ids,
         "dominant_ms": float(np.mean(dom_ms)), "down_ms": float(np.mean(down_ms)),
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

    # torch's elementwise multiply kernel is the calibration copy (the fills of
    # the cache-flush steps are elementwise kernels too, with other byte counts)
    copy_key = "MulFunctor"
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
    print(f"copy_fetch_kib_per_dispatch: {sum(cf) / len(cf):.1f}  (each: {', '.join(f'{v:.0f}' for v in cf)})")
    print(f"copy_write_kib_per_dispatch: {sum(cw) / len(cw):.1f}  (each: {', '.join(f'{v:.0f}' for v in cw)})")
    print(f"fetch_scale: {f_scale:.4f}")
    print(f"write_scale: {w_scale:.4f}")
    print(f"kernel_fetch_kib_per_dispatch: {kf:.1f}  (n={nf})")
    print(f"kernel_write_kib_per_dispatch: {kw:.1f}  (n={nw})")
    print(f"traffic_bytes_per_launch: {traffic:.0f}")


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_BUSY_CU_CYCLES TCC_HIT TCC_MISS")
SIMDS = 1024   # 256 CUs x 4 SIMDs
XCDS = 8


def summarize_mfma(d, cmd):
    """One --pmc run with MFMA_COUNTERS -> per-kernel MFMA work and utilisation.

    Per dispatch, averaged over the kernel's dispatches: duration from the
    dispatch timestamps; executed MFMA FLOPs = 512 x the MOPS counters (the
    counters count MFMA math operations in units of 512); MFMA busy = the SIMDs'
    MFMA-busy cycles over (GPU-active cycles of one XCD x 1024 SIMDs), the
    counter's summed-over-XCD GRBM_GUI_ACTIVE divided by 8; L2 hit rate."""
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        sys.exit(f"no counter_collection.csv under {d}")
    per = {}
    for r in csv.DictReader(open(f[0])):
        k = _short(r["Kernel_Name"])
        disp = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
        disp[r["Counter_Name"]] = float(r["Counter_Value"])
        disp["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    print("# MFMA work and utilisation per kernel, prefill T=4096 at full K3 shapes")
    print("# made by:")
    print(f"#   cd /tmp && timeout -s KILL 180 rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d <D> -o run -- "
          f"python3 <repo>/bench.py {cmd}")
    print("#   python3 bench.py --summarize-mfma <D> --summary-cmd '<the bench.py arguments>'")
    print("# exec_tflop: executed MFMA FLOPs per dispatch (512 x MOPS, all types); mfma_busy: MFMA-busy SIMD cycles / "
          "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs)")
    print("# clk_ghz: GRBM_GUI_ACTIVE / 8 per microsecond of the dispatch (the engine clock the counters saw)")
    print(f"{'kernel':56s} {'calls':>5s} {'avg_us':>9s} {'exec_tflop':>10s} {'exec_tf/s':>9s} {'mfma_busy':>9s} "
          f"{'l2_hit':>7s} {'clk_ghz':>7s}")
    for k, disps in per.items():
        ds = list(disps.values())
        n = len(ds)
        if n == 0 or "SQ_VALU_MFMA_BUSY_CYCLES" not in ds[0]:
            continue
        avg = lambda key: sum(x.get(key, 0.0) for x in ds) / n  # noqa: E731
        us = avg("_us")
        flop = 512.0 * (avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") + avg("SQ_INSTS_VALU_MFMA_MOPS_F8")
                        + avg("SQ_INSTS_VALU_MFMA_MOPS_F6F4"))
        if flop == 0:
            continue
        active = avg("GRBM_GUI_ACTIVE") / XCDS
        busy = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (active * SIMDS) if active else 0.0
        hit, miss = avg("TCC_HIT"), avg("TCC_MISS")
        print(f"{k[:56]:56s} {n:5d} {us:9.1f} {flop / 1e12:10.4f} {flop / (us * 1e-6) / 1e12:9.1f} "
              f"{100 * busy:8.1f}% {100 * hit / max(1.0, hit + miss):6.1f}% {active / us / 1e3:7.2f}")


def cpu_baseline(synth, wl, n_tokens, bias=None):
    """The float64 oracle as it stands, on the first n_tokens tokens of the workload.

    Only the oracle's arithmetic is timed: the seeded fixtures (tokens, dense
    weights and the raw checkpoint bytes of every expert the sample routes to)
    are generated before the clock starts; dequantisation stays inside, as it
    is part of the oracle's forward.  BLAS runs on every core this process may
    use; the per-expert steps run one after another, as the oracle has them."""
    from oracle import layer
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    x_bits = synth.gen_tokens(wl, n_tokens)
    d = synth.gen_dense(wl)
    bias = synth.gen_bias(wl) if bias is None else bias
    ids = layer.route(x_bits, d["w_router"], bias, wl.shape.top_k)["ids"]
    raw = {}
    for e in sorted(set(ids.reshape(-1).tolist())):
        raw[e] = {}
        for m in ("w1", "w3", "w2"):
            raw[e][m + "_packed"], raw[e][m + "_scale"] = synth.gen_expert(wl, e, m)
    cache = layer.ExpertCache(lambda e: raw[e], max_items=4 * wl.shape.top_k)
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        limit = None
    t0 = time.perf_counter()
    layer.layer_forward(x_bits, d, bias, cache, wl.shape)
    dt = time.perf_counter() - t0
    if limit is not None:
        limit.restore_original_limits()
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_tokens} of the {wl.tokens} tokens of the {wl.name} workload ({len(raw)} experts), "
                      f"float64 numpy oracle, expert dequantisation included, fixtures generated beforehand; "
                      f"BLAS on {cores} threads, the rest single-threaded; {dt:.1f} s"}


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


PEAK_OF_MODE = {"bf16x2": ("bf16", BF16_MFMA_PEAK_TFLOPS), "bf16": ("bf16", BF16_MFMA_PEAK_TFLOPS),
                "mx8x3": ("fp8", FP8_MFMA_PEAK_TFLOPS),
                "mx6x3": ("fp6/fp4", FP4_MFMA_PEAK_TFLOPS)}
# MFMA products executed per algorithmic product in each operand mode's expert
# GEMMs (gate/up with z, down with H): hi + lo planes, or three MX terms
EXEC_PER_ALG = {"bf16x2": 2, "bf16": 1, "mx8x3": 3, "mx6x3": 3}


def _layer_flops(sh, T):
    """Algorithmic FLOPs of one layer forward over T tokens: routed experts
    (gate, up, down), router, latent down and up projections, shared experts."""
    return 2.0 * T * (sh.top_k * 3 * sh.latent * sh.inter + sh.n_experts * sh.hidden
                      + 2 * sh.latent * sh.hidden + 3 * sh.n_shared * sh.shared_inter * sh.hidden)


TWO_BANK_A = 504  # MXFP4 experts of the two-bank layer; the other 392 are affine 2-bit (82% of the expert bytes)


def _affine_expert_bytes(sh) -> int:
    """Codes plus bf16 scales and biases of one affine 2-bit expert (w1, w3, w2)."""
    per = lambda n, k: n * k // 4 + 2 * n * (k // 64) * 2  # noqa: E731
    return 2 * per(sh.inter, sh.latent) + per(sh.latent, sh.inter)


def run_two_bank(mx, torch, synth, layers):
    """The two-bank layer (experts 0..503 MXFP4, 504..895 affine 2-bit with
    seeded codes, scales and biases) against the single MXFP4 bank, at decode
    T = 16 and prefill T = 4096, each pair of runs back to back on the same
    rotated weight copies; the split point stays on the device."""
    from mxfp4_latent_moe_amd import _lib
    dev = torch.device("cuda:0")
    sh = synth.K3_SHAPE
    n_b = sh.n_experts - TWO_BANK_A
    wl = synth.workload("decode")
    aff = synth.gen_expert_affine2_stack(wl, range(TWO_BANK_A, sh.n_experts))
    b0 = {k: torch.from_numpy(v).to(dev) for k, v in aff.items()}
    del aff
    banks = [dict(b0, format=_lib.MOE_WF_AFFINE2, n_experts=n_b)]
    banks += [dict({k: v.clone() for k, v in b0.items()}, format=_lib.MOE_WF_AFFINE2, n_experts=n_b)
              for _ in range(len(layers) - 1)]
    eb_a, eb_b = _expert_bytes(sh), _affine_expert_bytes(sh)
    out = {"workload": f"two-bank layer, experts 0..{TWO_BANK_A - 1} MXFP4 and {TWO_BANK_A}..{sh.n_experts - 1} "
                       f"affine 2-bit (group 64, bf16 scale and bias), full K3 shapes",
           "expert_bytes_ratio_all_experts": round((TWO_BANK_A * eb_a + n_b * eb_b) / (sh.n_experts * eb_a), 4)}
    for name, steps in (("decode", 100), ("prefill", PREFILL_STEPS)):
        w_l = synth.workload(name)
        r1 = run_workload(mx, torch, synth, layers, w_l, steps, 5, breakdown_steps=5)
        r2 = run_workload(mx, torch, synth, layers, w_l, steps, 5, breakdown_steps=5, bank_bs=banks)
        ms1, ms2 = 1e3 * r1["wall_s"] / steps, 1e3 * r2["wall_s"] / steps
        ids = r2["active_ids"]
        bytes2 = int((ids < TWO_BANK_A).sum()) * eb_a + int((ids >= TWO_BANK_A).sum()) * eb_b
        bytes1 = r1["e_act"] * eb_a
        g1, g2 = r1["dominant_ms"] + r1["down_ms"], r2["dominant_ms"] + r2["down_ms"]
        out[name] = {"tokens": w_l.tokens, "steps": steps,
                     "single_bank_ms": round(ms1, 4), "two_bank_ms": round(ms2, 4),
                     "two_bank_over_single": round(ms2 / ms1, 4),
                     "grouped_gemm_ms_single": round(g1, 4), "grouped_gemm_ms_two_bank": round(g2, 4),
                     "expert_bytes_single": bytes1, "expert_bytes_two_bank": bytes2,
                     "expert_gb_per_s_single": round(bytes1 / (g1 * 1e-3) / 1e9, 1),
                     "expert_gb_per_s_two_bank": round(bytes2 / (g2 * 1e-3) / 1e9, 1)}
    del banks, b0
    return out


def prefill_line(mx, torch, synth, layers, pf, mode, label):
    """Prefill T=4096 in one operand mode: tokens/s, the layer's algorithmic
    TFLOP/s against bf16 peak, and the expert GEMMs against the peak of the
    MFMA type they run (bf16, or fp8 / fp6 for the MX modes), algorithmic and
    executed (hi + lo planes or three MX terms)."""
    sh = pf.shape
    r = run_workload(mx, torch, synth, layers, pf, PREFILL_STEPS, 2, breakdown_steps=2, operand_mode=mode)
    ms = 1e3 * r["wall_s"] / PREFILL_STEPS
    P = pf.tokens * sh.top_k
    gu_flops = 2.0 * P * sh.latent * sh.inter * 2
    dn_flops = 2.0 * P * sh.inter * sh.latent
    dt_name, dt_peak = PEAK_OF_MODE[label]
    gu_tf = gu_flops / (r["dominant_ms"] * 1e-3) / 1e12
    dn_tf = dn_flops / (r["down_ms"] * 1e-3) / 1e12
    lt = _layer_flops(sh, pf.tokens) / (ms * 1e-3) / 1e12
    return {
        "workload": f"prefill T={pf.tokens}, full K3 shapes, operand mode {label}",
        "steps": PREFILL_STEPS,
        "tokens_per_s": round(pf.tokens / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 3),
        "layer_tflops_algorithmic": round(lt, 1),
        "layer_mfma_frac_algorithmic": round(lt / BF16_MFMA_PEAK_TFLOPS, 4),
        "gateup_ms": round(r["dominant_ms"], 4), "down_ms": round(r["down_ms"], 4),
        "gateup_tflops": round(gu_tf, 1), "down_tflops": round(dn_tf, 1),
        "expert_gemm_mfma_type": dt_name, "expert_gemm_type_peak_tflops": dt_peak,
        "gateup_frac_of_type_peak": round(gu_tf / dt_peak, 4),
        "gateup_frac_of_type_peak_executed": round(gu_tf * EXEC_PER_ALG[label] / dt_peak, 4),
        "gateup_frac_of_bf16_peak": round(gu_tf / BF16_MFMA_PEAK_TFLOPS, 4),
        "per_call_ms": {k: round(v, 4) for k, v in r["per_call_ms"].items()},
    }


def run_batched_decode(mx, torch, synth, layers, steps):
    """Batched decode T=256 with the Zipf-calibrated correction bias: tokens/s
    and the grouped GEMMs' expert-weight bytes over their event-timed time."""
    wl = synth.workload("batched_decode")
    sh = wl.shape
    bias = synth.gen_bias(wl, os.path.join(ROOT, "tests", "golden", "zipf_bias_T256.txt"))
    bias_d = torch.from_numpy(bias).to("cuda:0")
    zl = [dict(w, bias=bias_d) for w in layers]
    r = run_workload(mx, torch, synth, zl, wl, steps, 5, breakdown_steps=5)
    ms = 1e3 * r["wall_s"] / steps
    eb = r["e_act"] * _expert_bytes(sh)
    g_ms = r["dominant_ms"] + r["down_ms"]
    gbs = eb / (g_ms * 1e-3) / 1e9
    return {"workload": f"batched decode T={wl.tokens}, full K3 shapes, Zipf(1.1)-calibrated expert load",
            "steps": steps, "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "active_experts": r["e_act"], "expert_weight_bytes": eb,
            "grouped_gemm_ms": round(g_ms, 4), "gateup_ms": round(r["dominant_ms"], 4),
            "down_ms": round(r["down_ms"], 4),
            "expert_gb_per_s": round(gbs, 1), "expert_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "expert_hbm_frac_layer": round(eb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "per_call_ms": {k: round(v, 4) for k, v in r["per_call_ms"].items()}}


def run_microbench(mx, torch, synth, w, steps=10):
    """Isolated grouped GEMM: segments ~ Multinomial(65536, Zipf(1.1)) over the
    896 experts, A = bf16 N(0, 1) rows already in expert order; gate/up +
    SiTU-GLU then down, in the default and the MX fp6 operand modes."""
    from synth.device import to_dev
    from mxfp4_latent_moe_amd import _lib, ops
    dev = torch.device("cuda:0")
    wl = synth.workload("microbench")
    sh = wl.shape
    counts = synth.gen_microbench_counts(wl)
    P = int(counts.sum())
    offsets = np.zeros(sh.n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    A = torch.from_numpy(synth.gen_microbench_activations(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    off_d = to_dev(offsets, dev)
    H = torch.empty((P, sh.inter), dtype=torch.float32, device=dev)
    Y = torch.empty((P, sh.latent), dtype=torch.float32, device=dev)
    gu_flops = 2.0 * P * sh.latent * sh.inter * 2
    dn_flops = 2.0 * P * sh.inter * sh.latent
    out = {"workload": f"isolated grouped GEMM, {P} rows over {sh.n_experts} experts (Multinomial(65536, "
                       f"Zipf(1.1)) segments, largest {int(counts.max())}), A bf16 already permuted",
           "steps": steps, "weight_bytes": sh.n_experts * _expert_bytes(sh)}
    for label, mode in (("bf16x2", _lib.MOE_OPND_BF16X2), ("mx6x3", _lib.MOE_OPND_MX6X3)):
        s = mx.shape_of(sh, mode)
        ws = torch.empty(ops.workspace_bytes(s, _lib.MOE_FN_GROUPED_GEMM, P), dtype=torch.uint8, device=dev)

        def gu():
            ops.grouped_gemm(s, _lib.MOE_OP_GATEUP_SITU, P, off_d, None, A, w["w1_packed"], w["w1_scale"],
                             w["w3_packed"], w["w3_scale"], None, H, ws)

        def dn():
            ops.grouped_gemm(s, _lib.MOE_OP_DOWN, P, off_d, None, H, w["w2_packed"], w["w2_scale"], None, None,
                             None, Y, ws)
        for _ in range(2):
            gu()
            dn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1, e2 in ev:
            e0.record()
            gu()
            e1.record()
            dn()
            e2.record()
        torch.cuda.synchronize()
        gu_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
        dn_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
        tf = (gu_flops + dn_flops) / ((gu_ms + dn_ms) * 1e-3) / 1e12
        # gate/up takes the exact bf16 rows with one MFMA (or as MX terms); down takes H as hi + lo
        dt_name, dt_peak = PEAK_OF_MODE[label]
        out[label] = {"gateup_ms": round(gu_ms, 4), "down_ms": round(dn_ms, 4),
                      "gateup_tflops": round(gu_flops / (gu_ms * 1e-3) / 1e12, 1),
                      "down_tflops": round(dn_flops / (dn_ms * 1e-3) / 1e12, 1),
                      "tflops": round(tf, 1), "mfma_frac_bf16_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                      "expert_gemm_mfma_type": dt_name, "frac_of_type_peak": round(tf / dt_peak, 4),
                      "weight_gb_per_s": round(out["weight_bytes"] / ((gu_ms + dn_ms) * 1e-3) / 1e9, 1)}
        if label == "bf16x2":
            out["roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                               "kernel": "mxfp4_grouped_gemm gate/up + down", "algorithmic_flops": gu_flops + dn_flops}
        del ws
    del A, H, Y
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill"])
    ap.add_argument("--operand-mode", default="bf16x2", choices=["bf16x2", "bf16", "mx8x3", "mx6x3"],
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
    ap.add_argument("--summarize-mfma", metavar="DIR")
    ap.add_argument("--summary-cmd", default="", help="the profiled bench.py arguments, for the summary header")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.summary_cmd)
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
    opnd = {"bf16x2": mx.MOE_OPND_BF16X2, "bf16": mx.MOE_OPND_BF16, "mx8x3": mx.MOE_OPND_MX8X3, "mx6x3": mx.MOE_OPND_MX6X3}[args.operand_mode]
    r = run_workload(mx, torch, synth, layers, wl, args.steps, args.warmup, args.cold_steps, operand_mode=opnd)
    ms = 1e3 * r["wall_s"] / args.steps
    value = wl.tokens * args.steps / r["wall_s"]

    gu_ms = r["dominant_ms"]  # events around the gate/up call in every step of the event-timed pass
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
                           "bf16": "activations rounded once to bf16",
                           "mx8x3": "expert GEMM activations as three e4m3 terms, other activations bf16 hi+lo",
                           "mx6x3": "expert GEMM activations as three e2m3 terms, other activations bf16 hi+lo"}[
                            args.operand_mode] + ", fp32 accumulate, fp32 output",
            "parallelism": "single GPU",
            "layers_rotated": len(layers),
        },
        "per_call_ms": {k: round(v, 4) for k, v in r["per_call_ms"].items()},
        # the same steps with HIP events around the gate/up and down calls (the pass the roofline's avg_ms is from)
        "ms_per_step_with_kernel_events": round(1e3 * r["wall_marked_s"] / args.steps, 4),
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
        print("bench: timing batched decode T=256 (Zipf load)", file=sys.stderr, flush=True)
        line["secondary_batched_decode"] = run_batched_decode(mx, torch, synth, layers, args.steps)
        pf = synth.workload("prefill")
        for key, mode, label in (("secondary", mx.MOE_OPND_BF16X2, "bf16x2"),
                                 ("secondary_mx8x3", mx.MOE_OPND_MX8X3, "mx8x3"),
                                 ("secondary_mx6x3", mx.MOE_OPND_MX6X3, "mx6x3")):
            print(f"bench: timing prefill, operand mode {label}", file=sys.stderr, flush=True)
            line[key] = prefill_line(mx, torch, synth, layers, pf, mode, label)
        print("bench: timing the grouped-GEMM microbenchmark", file=sys.stderr, flush=True)
        line["secondary_microbench"] = run_microbench(mx, torch, synth, layers[0])
        print("bench: timing the two-bank layer", file=sys.stderr, flush=True)
        line["secondary_two_bank"] = run_two_bank(mx, torch, synth, layers)
        print("bench: timing the layer-0 dense FFN", file=sys.stderr, flush=True)
        line["secondary_dense_ffn"] = run_dense_ffn(mx, torch, synth)
        print("bench: timing the REAP saliency pass", file=sys.stderr, flush=True)
        line["secondary_reap"] = run_reap(mx, torch, synth)

    if args.calibrate_copy:
        calibration_copy(torch)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(synth, wl, 8 if args.workload == "decode" else 4)
        if "secondary" in line:
            line["secondary"]["cpu_baseline"] = cpu_baseline(synth, synth.workload("prefill"), 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
