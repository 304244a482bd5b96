"""Helpers shared by the GPU parity tests: oracle references for sampled tokens
and the acceptance metrics (expert ids and permutation exact outside the
near-tie tokens, max|gpu - oracle| / rms(oracle) on outputs)."""
from __future__ import annotations

import os
import sys

import numpy as np

import synth
from oracle import layer

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ZIPF_BIAS = os.path.join(GOLDEN, "zipf_bias_T256.txt")
GAP_EXCLUDE = 1e-5
TOL = 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2)))
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / rms)


def raw_expert(wl, e):
    """One expert's checkpoint-layout tensors from the seeded generator."""
    return {
        **dict(zip(("w1_packed", "w1_scale"), synth.gen_expert(wl, e, "w1"))),
        **dict(zip(("w3_packed", "w3_scale"), synth.gen_expert(wl, e, "w3"))),
        **dict(zip(("w2_packed", "w2_scale"), synth.gen_expert(wl, e, "w2"))),
    }


def expert_cache(wl):
    return layer.ExpertCache(lambda e: raw_expert(wl, e), max_items=80)


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_layer_threaded(wl, x_bits, dense, bias):
    """The oracle's layer forward over the given token rows, with its per-expert
    step mapped over a thread pool (experts dequantised on demand, not kept:
    one full-shape expert is 264 MB in float64)."""
    from concurrent.futures import ThreadPoolExecutor
    get = lambda e: layer.dequant_expert(raw_expert(wl, e))  # noqa: E731
    with ThreadPoolExecutor(oracle_threads()) as ex:
        return layer.layer_forward(x_bits, dense, bias, get, wl.shape, keep=True, map_fn=ex.map)


def pick_tokens(ids, gap, n_experts, chunk_rows, n_tokens, seed=0):
    """Tokens whose pairs cover the grouped kernels' work-item shapes, from the
    oracle's own permutation: for every count 1..chunk_rows/16 of active 16-row
    tiles, a token in the last tile of a chunk with that count; tokens in the
    second and the last chunk of the longest segment; the first and last token;
    then tokens that add the fewest new experts (to bound the oracle's work),
    up to n_tokens.  Near-tie tokens (gap < 1e-5) are never picked, so every
    picked token's expert set is exact on both sides."""
    T, k = ids.shape
    ok = gap >= GAP_EXCLUDE
    perm = layer.permute(ids, n_experts)
    offs, sp = perm["offsets"], perm["sorted_pair"]
    chosen = []

    def add(t):
        t = int(t)
        if ok[t] and t not in chosen:
            chosen.append(t)
            return True
        return False

    for c in range(1, chunk_rows // 16 + 1):
        for e in range(n_experts):
            n = int(offs[e + 1] - offs[e])
            if n == 0:
                continue
            last = n - (n - 1) // chunk_rows * chunk_rows  # rows of the segment's last chunk
            if (last + 15) // 16 != c:
                continue
            if any(add(sp[int(offs[e + 1]) - 1 - i] // k) for i in range(min(last, 4))):
                break
    e_long = int(np.argmax(np.diff(offs)))
    if offs[e_long + 1] - offs[e_long] > chunk_rows:
        add(sp[int(offs[e_long]) + chunk_rows] // k)
        add(sp[int(offs[e_long + 1]) - 1] // k)
    add(0)
    add(T - 1)
    experts = set(ids[chosen].reshape(-1).tolist())
    rng = np.random.default_rng(seed)
    cand = [t for t in rng.permutation(T) if ok[t] and t not in chosen]
    while len(chosen) < min(n_tokens, int(ok.sum())):
        new = [len(set(ids[t].tolist()) - experts) for t in cand]
        i = int(np.argmin(new))
        t = cand.pop(i)
        chosen.append(int(t))
        experts |= set(ids[t].tolist())
    return np.array(sorted(chosen))


def check_routing(gpu_ids: np.ndarray, gpu_w: np.ndarray, ref: dict):
    """ids exact for tokens whose k-th/(k+1)-th gap is >= 1e-5; returns the excluded set."""
    excl = np.nonzero(ref["gap"] < GAP_EXCLUDE)[0]
    keep = np.setdiff1d(np.arange(gpu_ids.shape[0]), excl)
    bad = keep[(gpu_ids[keep] != ref["ids"][keep]).any(axis=1)]
    assert bad.size == 0, f"expert ids differ for tokens {bad[:10]}"
    np.testing.assert_allclose(gpu_w[keep], ref["weights"][keep], rtol=2e-5, atol=1e-7)
    return excl


def check_permutation(gpu: dict, ids_ref: np.ndarray, E: int, excl: np.ndarray):
    """Per-expert token lists identical once the excluded tokens' pairs are removed."""
    T, k = ids_ref.shape
    g_off = gpu["offsets"]
    g_sp = gpu["sorted_pair"]
    g_ids = gpu["topk_ids"]
    # the GPU's own permutation must be a valid stable sort of its own ids
    assert g_off[0] == 0 and g_off[E] == T * k and (np.diff(g_off) >= 0).all()
    assert (gpu["pair_pos"][g_sp] == np.arange(T * k)).all()
    flat = g_ids.reshape(-1)
    for e in range(E):
        seg = g_sp[g_off[e]:g_off[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()
    # against the oracle, without the excluded tokens
    ex = set(excl.tolist())
    ref = layer.permute(ids_ref, E)
    r_off, r_sp = ref["offsets"], ref["sorted_pair"]
    for e in range(E):
        a = [p // k for p in g_sp[g_off[e]:g_off[e + 1]] if p // k not in ex]
        b = [p // k for p in r_sp[r_off[e]:r_off[e + 1]] if p // k not in ex]
        assert a == b, f"expert {e}: token lists differ"
    act = gpu["active"]
    assert act[0] == np.count_nonzero(np.diff(g_off)) and (act[1:1 + act[0]] == np.nonzero(np.diff(g_off))[0]).all()
