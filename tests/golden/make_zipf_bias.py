"""Write zipf_bias_T256.txt: the correction bias of the batched-decode workload
(full K3 shapes, T = 256), calibrated so that expert load follows Zipf(1.1)
over a seeded permutation of the experts.

The pages give no procedure for such a bias; this script's reading:
  1. target load of Zipf rank r: T*k*p_r with p_r = r^-1.1 / sum_j j^-1.1,
     capped at T (an expert can take each token at most once) and
     water-filled so the targets still sum to T*k; expert perm[r-1] has rank r;
  2. start from b = 0 and the workload's own router scores (oracle);
  3. 512 steps of b_e += 1e-3 * sign(target_e - load_e), load_e counted from
     the oracle's top-k selection (the usual aux-loss-free update rule);
  4. store b as float32, one value per line, with the realised load
     statistics in the header.
Only oracle/ and synth/ are used.  Run from the repository root:
    python tests/golden/make_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import layer  # noqa: E402

STEPS = 512
STEP = 1e-3


def water_fill(p, total, cap):
    t = total * p
    capped = np.zeros(p.size, bool)
    while (t > cap + 1e-9).any():
        capped |= t > cap
        rest = total - cap * capped.sum()
        t = np.where(capped, cap, rest * p / p[~capped].sum())
    return t


def gini(v):
    v = np.sort(v.astype(np.float64))
    n = v.size
    return float((2 * np.arange(1, n + 1) - n - 1).dot(v) / (n * v.sum()))


def main():
    wl = synth.workload("batched_decode")
    sh = wl.shape
    T, k, E = wl.tokens, sh.top_k, sh.n_experts
    x = synth.gen_tokens(wl)
    d = synth.gen_dense(wl)
    _, scores = layer.router_scores(x, d["w_router"])
    perm = synth.zipf_permutation(wl)
    p_rank = synth.zipf_probabilities(E, wl.zipf_s)
    target = np.empty(E)
    target[perm] = water_fill(p_rank, T * k, T)
    b = np.zeros(E, np.float32)
    for _ in range(STEPS):
        ids = layer.select_topk(scores, b, k)["ids"]
        load = np.bincount(ids.reshape(-1), minlength=E)
        b = (b + np.float32(STEP) * np.sign(target - load).astype(np.float32)).astype(np.float32)
    r = layer.select_topk(scores, b, k)
    load = np.bincount(r["ids"].reshape(-1), minlength=E)
    ranked = load[perm]
    nz = ranked > 0
    rr = np.arange(1, E + 1)[nz]
    slope = np.polyfit(np.log(rr[:64]), np.log(ranked[nz][:64]), 1)[0]
    hdr = [
        "correction bias, batched-decode workload (T=256, full K3 shapes), Zipf(1.1)-calibrated",
        "written by tests/golden/make_zipf_bias.py (oracle routing only)",
        f"realised: max load {load.max()}, active experts {int((load > 0).sum())}, zero-load {int((load == 0).sum())}, "
        f"CV {load.std() / load.mean():.3f}, Gini {gini(load):.3f}, log-log slope (top 64 ranks) {slope:.3f}, "
        f"L1 distance to target {np.abs(load - target).sum():.0f} of {T * k}, "
        f"tokens with gap < 1e-5: {int((r['gap'] < 1e-5).sum())}",
    ]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_T256.txt")
    np.savetxt(out, b.astype(np.float64), fmt="%.9g", header="\n".join(hdr))
    print("\n".join(hdr))


if __name__ == "__main__":
    main()
