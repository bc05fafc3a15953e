#!/usr/bin/env python3
"""Benchmark of the Flash-Cache per-layer denoising step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
slot map -> fused QKV + RoPE + cache write -> scheduled attention with the
formula-(2) column mass, layer by layer, then the top-k of the tracked set.

Default workload (the headline): the 32-layer LLaDA-8B-shaped sweep (d_model
4096, 32 heads x 128, bf16) at batch 32, context 2048 (prompt 1536 + gen 512),
with denoising steps alternating between a full refresh (2048 rows per
sequence and layer) and a cache-phase step (32 masked window + 8 new + 32
tracked rows per sequence and layer); one top-32 per step after the last
layer.  Timed steps alternate the two kinds.

Metric: refreshed tokens/s per layer = rows refreshed per layer over the timed
steps / (their time / layers).  Inputs are resident in HBM before timing
starts; the batch-32 caches and weights (38 GB) are far larger than the
256 MB Infinity Cache.  The single-layer workloads reported beside it (batch
1, the mixed batch of 8, the batch-4 verify step) rotate over enough
independent copies of weights, caches and inputs to span >= 1 GiB.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "refreshed tokens/s per layer (cache-update+attention)"
SINGLE = ("llada_b1", "mixed_b8", "verify_b4")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llada_b32", choices=["llada_b32", *SINGLE])
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="only the headline workload (no other workloads, variants or decode side)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--probe", default=None,
                   help="profiling aid: launch one kernel a few times and print no bench line; "
                        "attn_full_b32 | attn_cache_b32 (batch-32 attention, full refresh or cache phase) | "
                        "qkv:<rows>[:<shape>] (the projection of <rows> LLaDA-8B-shaped rows, optionally forcing "
                        "a tile shape such as g256x128o2)")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode-side reductions (logits -> confidence, threshold rule, verify scan)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run a plain device copy of this size (counter calibration)")
    return p.parse_args()


def pct(vals):
    import numpy as np
    a = np.asarray(vals, dtype=np.float64)
    return {"mean": float(a.mean()), "p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90))}


def layer_work(sh, rows, cache_el=2):
    """Algorithmic bytes and flops of one layer of a step: the projection
    (W_qkv once; per row x in, q out, K and V rows into the cache) and the
    attention (per key of a sequence its K and V row; per row q in, o out;
    4 n flops per visible (row, key) pair), each kernel's bound, their sum
    (the step's roofline) and the stricter overlap bound."""
    import numpy as np
    n = sh.n_heads * sh.head_dim
    d = sh.d_model
    el = 2 if sh.dtype == "bf16" else 4
    kel = cache_el if el == 2 else el
    R = rows.n_rows
    qkv_bytes = 3 * n * d * el + R * d * el + R * n * el + 2 * R * n * kel
    qkv_flops = 2 * R * d * 3 * n
    kv = rows.kv_len.astype(np.int64)
    attn_bytes = int(kv.sum()) * 2 * n * kel + 2 * R * n * el
    attn_flops = 0
    for b in range(len(kv)):
        rb = int(rows.cu_q[b + 1] - rows.cu_q[b])
        vis = rows.visible[b].sum() if rows.visible is not None else rb * int(kv[b])
        attn_flops += 4 * int(vis) * n
    bw, pk = HBM_PEAK_GBS * 1e9, MFMA_BF16_PEAK_TFLOPS * 1e12
    b_qkv = max(qkv_bytes / bw, qkv_flops / pk) * 1e6
    b_att = max(attn_bytes / bw, attn_flops / pk) * 1e6
    return {"qkv_bytes": qkv_bytes, "qkv_flops": qkv_flops, "attn_bytes": attn_bytes, "attn_flops": attn_flops,
            "qkv_bound_us": b_qkv, "qkv_bound": "hbm" if qkv_bytes / bw >= qkv_flops / pk else "mfma",
            "attn_bound_us": b_att, "attn_bound": "hbm" if attn_bytes / bw >= attn_flops / pk else "mfma",
            "sum_of_bounds_us": b_qkv + b_att,
            "overlap_bound_us": max((qkv_bytes + attn_bytes) / bw, (qkv_flops + attn_flops) / pk) * 1e6}


def counter_traffic(name):
    """Counter-measured HBM bytes per launch of a profiled kernel
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy calibration), from a
    profiles/ record; None once the kernel's source differs from the one
    profiled."""
    import hashlib
    tfile = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(tfile):
        return None
    tj = json.load(open(tfile))
    src = open(os.path.join(ROOT, tj["source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != tj["source_sha256"]:
        return None
    return tj["bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from io_aware_kv_amd import dllm

    dllm.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.probe:
        probe(args.probe, dev)
        if args.copy_probe_mib:
            copy_probe(args.copy_probe_mib, dev)
        return
    if args.workload == "llada_b32":
        out = bench_layers(args, dev)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        if not args.no_extras:
            out["other_workloads"] = {}
            for name in SINGLE:
                out["other_workloads"][name] = bench_single(args, dev, name, detail=name == "llada_b1")
                torch.cuda.empty_cache()
    else:
        out = bench_single(args, dev, args.workload, detail=not args.no_extras)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)
    if not args.no_decode and not args.no_graph and not args.no_extras:
        out["decode_side"] = bench_decode(args, dev)
    if not args.no_extras:
        out["achievable"] = achievable_probes(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_b32() if args.workload == "llada_b32"
                               else cpu_baseline(args.workload, args.cpu_seconds))
        # the oracle beside each single-layer line too, on a shorter budget
        for name, line in out.get("other_workloads", {}).items():
            line["cpu_baseline"] = cpu_baseline(name, min(2.0, args.cpu_seconds))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# the headline: 32 layers, batch 32
# ---------------------------------------------------------------------------

def bench_layers(args, dev):
    """32-layer batch-32 sweep.  Timed: K denoising steps alternating full
    refresh (2048 rows per sequence per layer) and cache phase (72 rows per
    sequence per layer), each with per-layer HIP events around the projection
    and the attention on the launch stream, plus the step's top-k.  Variants
    (score from the middle layers only, E4M3 caches, block-freeze row sets,
    the unfused arm) are timed after it on the same layers."""
    import numpy as np
    import torch
    from io_aware_kv_amd import workloads as W
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = W.make_workload("llada_b32")
    sh = wl.shape
    L = sh.layers
    run = FlashCacheRunner(wl, device=dev)
    Ws = [W.device_weights(wl, l, dev) for l in range(L)]
    rows = {"full": W.full_refresh_rows(wl)}
    sts = {"full": run.upload_step(rows["full"])}
    xs = {"full": [W.device_activations(wl, rows["full"], 0, l, dev) for l in range(L)]}
    stream = torch.cuda.current_stream()

    def step(kind, ev=None, unfused=False, topk_each=False):
        st = sts[kind]
        mass = kind in ("full", "cache", "cache_mid")    # block-cache steps have no formula-(2) rows
        run.map_slots(st)
        for l in range(L):
            if ev is not None:
                ev[l][0].record(stream)
            if unfused:
                run.cache_update_unfused(st, xs[kind][l], Ws[l], l)
            else:
                run.cache_update(st, xs[kind][l], Ws[l], l)
            if ev is not None:
                ev[l][1].record(stream)
            # cache_mid: the score only from the middle layers 5..20 (1-based); the
            # first scoring layer stores its term, the others add theirs
            first = 4 if kind == "cache_mid" else 0
            run.attention(st, l, with_mass=mass and (kind != "cache_mid" or 5 <= l + 1 <= 20),
                          mass_overwrite=l == first)
            if ev is not None:
                ev[l][2].record(stream)
            # the labelled per-layer variant: a selection after every layer over
            # the score accumulated so far (the last one feeds the next step)
            if topk_each and mass and l < L - 1:
                run.topk(clear_mass=False)
        if mass:
            run.topk(clear_mass=False)
        if ev is not None:
            ev[L][0].record(stream)

    step("full")
    idx = run.top_idx.cpu().numpy()
    rows["cache"] = W.config_step_rows(wl, [idx[b][idx[b] >= 0] for b in range(wl.n_seq)])
    sts["cache"] = run.upload_step(rows["cache"])
    xs["cache"] = [W.device_activations(wl, rows["cache"], 1, l, dev) for l in range(L)]
    kinds = ("full", "cache")
    for i in range(max(2, args.warmup)):
        step(kinds[i % 2])
    torch.cuda.synchronize()

    # ---- the timed region: K steps alternating full refresh and cache phase ----
    K = max(2, args.steps)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [[[ev() for _ in range(3)] for _ in range(L + 1)] for _ in range(K)]
    t_step = [(ev(), ev()) for _ in range(K)]
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        t_step[i][0].record(stream)
        step(kinds[i % 2], evs[i])
        t_step[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    res = {}
    for k, kind in enumerate(kinds):
        its = range(k, K, 2)
        qkv = [evs[i][l][0].elapsed_time(evs[i][l][1]) * 1e3 for i in its for l in range(L)]
        att = [evs[i][l][1].elapsed_time(evs[i][l][2]) * 1e3 for i in its for l in range(L)]
        tk = [evs[i][L - 1][2].elapsed_time(evs[i][L][0]) * 1e3 for i in its]
        stp = [t_step[i][0].elapsed_time(t_step[i][1]) for i in its]
        wk = layer_work(sh, rows[kind])
        ms = float(np.mean(stp))
        q, a = pct(qkv), pct(att)
        res[kind] = {"rows_per_layer": rows[kind].n_rows, "steps_timed": len(stp),
                     "ms_per_step": ms, "ms_per_step_pct": pct(stp), "us_per_layer": ms * 1e3 / L,
                     "tokens_per_s_per_layer": rows[kind].n_rows / (ms * 1e-3 / L),
                     "qkv_us": q["mean"], "qkv_us_pct": q, "qkv_bound_us": wk["qkv_bound_us"],
                     "qkv_bound": wk["qkv_bound"], "qkv_frac": wk["qkv_bound_us"] / q["mean"],
                     "attn_us": a["mean"], "attn_us_pct": a, "attn_bound_us": wk["attn_bound_us"],
                     "attn_bound": wk["attn_bound"], "attn_frac": wk["attn_bound_us"] / a["mean"],
                     "topk_us": float(np.mean(tk)), "topk_us_per_layer": float(np.mean(tk)) / L,
                     "layer_sum_of_bounds_us": wk["sum_of_bounds_us"],
                     "layer_overlap_bound_us": wk["overlap_bound_us"],
                     "layer_roofline_frac": wk["sum_of_bounds_us"] / (ms * 1e3 / L),
                     "layer_overlap_frac": wk["overlap_bound_us"] / (ms * 1e3 / L),
                     "alg_bytes_per_layer": wk["qkv_bytes"] + wk["attn_bytes"],
                     "alg_flops_per_layer": wk["qkv_flops"] + wk["attn_flops"]}
        eprint(f"[bench] llada_b32 {kind}: {ms:.2f} ms/step, {ms * 1e3 / L:.1f} us/layer "
               f"(projection {q['mean']:.1f} us = {res[kind]['qkv_frac']:.3f} of its bound, "
               f"attention {a['mean']:.1f} us = {res[kind]['attn_frac']:.3f})")
    # the same steps replayed from one captured hipGraph each (labelled beside
    # the stream-launch figures; `value` stays the stream-launch measurement)
    if not args.no_graph:
        for kind in kinds:
            gms = _graph_time(lambda _c, kind=kind: step(kind), 1, 3, 1, stream)
            res[kind]["graph_ms_per_step"] = gms
            res[kind]["graph_us_per_layer"] = gms * 1e3 / L
            eprint(f"[bench] llada_b32 {kind}: {gms:.2f} ms/step replayed from a hipGraph")
    tot_rows = sum(rows[kinds[i % 2]].n_rows for i in range(K))
    value = tot_rows / (total_ms * 1e-3 / L)
    dom = res["full"]
    dom_work = layer_work(sh, rows["full"])
    achieved = dom_work["qkv_flops"] / (dom["qkv_us"] * 1e-6) / 1e12
    out = {
        "metric": METRIC,
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": total_ms / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LLaDA-8B-shaped 32-layer sweep (d_model 4096, 32x128 heads, bf16), batch 32, "
                               "context 2048 (prompt 1536 + gen 512); denoising steps alternating full refresh "
                               "(2048 rows/seq/layer) and cache phase (72 rows/seq/layer: 32 window + 8 new + "
                               "32 tracked), top-32 once per step",
                   "layers": L, "batch": wl.n_seq, "d_model": sh.d_model, "heads": sh.n_heads,
                   "head_dim": sh.head_dim, "parallelism": "single GPU",
                   "timing": "stream launches (hipGraph replays of each step kind beside them in steps_detail)",
                   "steps_alternate": list(kinds)},
        "steps_detail": res,
        "step_roofline_frac": sum(res[k]["layer_sum_of_bounds_us"] * res[k]["steps_timed"] for k in kinds) * L
                              / (total_ms * 1e3),
        "step_overlap_frac": sum(res[k]["layer_overlap_bound_us"] * res[k]["steps_timed"] for k in kinds) * L
                             / (total_ms * 1e3),
        "roofline": {"bound": "mfma", "kernel": "qkv_rope_cachewrite (full refresh, 65536 rows per layer)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": counter_traffic("qkv_rope_cachewrite_llada_b32_full_traffic.json"),
                     "alg_flops_per_launch": dom_work["qkv_flops"],
                     "alg_bytes_per_launch": dom_work["qkv_bytes"]},
    }
    if args.no_extras:
        return out

    # ---- variants on the same layers ----
    rows["cache_mid"], sts["cache_mid"], xs["cache_mid"] = rows["cache"], sts["cache"], xs["cache"]
    for mode in W.BLOCK_CACHE_MODES:
        rows[mode] = W.block_cache_rows(wl, mode)
        sts[mode] = run.upload_step(rows[mode])
        xs[mode] = [W.device_activations(wl, rows[mode], 2, l, dev) for l in range(L)]
    run8 = FlashCacheRunner(wl, device=dev, kv_format="e4m3")
    st8 = {"full": run8.upload_step(rows["full"]), "cache": run8.upload_step(rows["cache"])}

    def step8(kind, ev=None):
        st = st8[kind]
        run8.map_slots(st)
        for l in range(L):
            if ev is not None:
                ev[l][0].record(stream)
            run8.cache_update(st, xs[kind][l], Ws[l], l)
            if ev is not None:
                ev[l][1].record(stream)
            run8.attention(st, l, mass_overwrite=l == 0)
            if ev is not None:
                ev[l][2].record(stream)
        run8.topk(clear_mass=False)

    step8("full")
    step8("cache")
    torch.cuda.synchronize()
    KV = max(2, min(5, K // 2))
    var = {}
    for kind in ("cache_mid", "cache_e4m3", "cache_unfused", "cache_topk_each") + W.BLOCK_CACHE_MODES:
        vevs = [[[ev() for _ in range(3)] for _ in range(L + 1)] for _ in range(KV)]
        a0, a1 = ev(), ev()
        a0.record(stream)
        for i in range(KV):
            if kind == "cache_e4m3":
                step8("cache", vevs[i])
            elif kind == "cache_unfused":
                step("cache", vevs[i], unfused=True)
            elif kind == "cache_topk_each":
                step("cache", vevs[i], topk_each=True)
            else:
                step(kind, vevs[i])
        a1.record(stream)
        torch.cuda.synchronize()
        ms = a0.elapsed_time(a1) / KV
        rk = rows["cache"] if kind in ("cache_e4m3", "cache_unfused", "cache_topk_each") else rows[kind]
        wk = layer_work(sh, rk, cache_el=1 if kind == "cache_e4m3" else 2)
        qkv_us = float(np.mean([vevs[i][l][0].elapsed_time(vevs[i][l][1]) for i in range(KV) for l in range(L)])) * 1e3
        att_us = float(np.mean([vevs[i][l][1].elapsed_time(vevs[i][l][2]) for i in range(KV) for l in range(L)])) * 1e3
        var[kind] = {"rows_per_layer": rk.n_rows, "ms_per_step": ms, "us_per_layer": ms * 1e3 / L,
                     "tokens_per_s_per_layer": rk.n_rows / (ms * 1e-3 / L),
                     "qkv_us": qkv_us, "qkv_bound_us": wk["qkv_bound_us"], "qkv_frac": wk["qkv_bound_us"] / qkv_us,
                     "qkv_bound": wk["qkv_bound"],
                     "attn_us": att_us, "attn_bound_us": wk["attn_bound_us"], "attn_frac": wk["attn_bound_us"] / att_us,
                     "attn_bound": wk["attn_bound"],
                     "layer_roofline_frac": wk["sum_of_bounds_us"] / (ms * 1e3 / L)}
        eprint(f"[bench] llada_b32 {kind}: {var[kind]}")
    var["cache_unfused"]["fused_speedup_per_layer"] = var["cache_unfused"]["ms_per_step"] / res["cache"]["ms_per_step"]
    var["cache_unfused"]["fused_update_speedup"] = var["cache_unfused"]["qkv_us"] / res["cache"]["qkv_us"]
    out["block_cache_steps"] = {k: var.pop(k) for k in W.BLOCK_CACHE_MODES}
    out["cache_phase_middle_layer_score"] = var.pop("cache_mid")
    out["cache_phase_e4m3_cache"] = var.pop("cache_e4m3")
    out["unfused_arm_cache_phase"] = var.pop("cache_unfused")
    te = var.pop("cache_topk_each")
    # each added selection's cost: the step's extra time over its L - 1 added launches
    te["topk_us_each"] = (te["ms_per_step"] - res["cache"]["ms_per_step"]) * 1e3 / (L - 1)
    te["note"] = ("the cache-phase step with the top-k after every layer over the score accumulated so far "
                  "(the once-per-step selection is the default line)")
    out["cache_phase_topk_each_layer"] = te
    del run8, st8, xs, sts, Ws, run
    return out


# ---------------------------------------------------------------------------
# single-layer workloads (batch 1, mixed batch 8, verify batch 4)
# ---------------------------------------------------------------------------

def describe(name):
    return {
        "llada_b1": "LLaDA-8B-shaped layer (d_model 4096, 32x128 heads, bf16), batch 1, context 512 "
                    "(prompt 256 + gen 256), cache-phase step: 32 window + 8 new + 32 tracked rows",
        "mixed_b8": "LLaDA-8B-shaped layer, batch 8 mixed: 6 cache-phase sequences (40-72 rows, context "
                    "512-1024) + 2 full refreshes (512, 1024 rows)",
        "verify_b4": "LLaDA-8B-shaped layer, batch 4, context 1024 + 32 view slots, verify step with "
                     "16 draft + 16 mask views + 40 ordinary rows per sequence under the verify mask",
    }[name]


def _graph_time(fn, copies, K, warmup, stream):
    """Per-call time of fn(copy) replayed from one captured graph per copy."""
    import torch
    graphs = []
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                fn(c)
            graphs.append(g)
    stream.wait_stream(cs)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(K):
        graphs[i % copies].replay()
    g1.record(stream)
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) / K


def bench_single(args, dev, name, detail=False):
    """One single-layer workload: step 0 (full refresh) on the GPU fills the
    cache and picks the tracked rows; its own step is then timed as plain
    launches (HIP events around every kernel) and as hipGraph replays over
    rotated copies (>= 1 GiB).  detail: also the unfused arm, the full
    refresh, the E4M3 cache and the block-freeze row sets on the same layer."""
    import numpy as np
    import torch
    from io_aware_kv_amd import dllm
    from io_aware_kv_amd import workloads as W
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = W.make_workload(name)
    sh = wl.shape
    n_out = sh.n_heads * sh.head_dim

    run = FlashCacheRunner(wl, device=dev, layers=1)
    w0 = run.to_device_array(W.weights(wl, 0))
    rows0 = W.full_refresh_rows(wl)
    st0 = run.upload_step(rows0)
    x0 = run.to_device_array(W.activations(wl, rows0, 0))
    run.layer_step(st0, x0, w0, 0)
    run.topk(clear_mass=True)
    idx = run.top_idx.cpu().numpy()
    rows1 = W.config_step_rows(wl, [idx[b][idx[b] >= 0] for b in range(wl.n_seq)])
    R = rows1.n_rows
    st = run.upload_step(rows1)
    x1 = run.to_device_array(W.activations(wl, rows1, 1))
    del st0, x0

    per_copy = (w0.numel() * w0.element_size() + 2 * run.k_cache[0].numel() * run.k_cache[0].element_size()
                + x1.numel() * x1.element_size())
    copies = max(1, int(np.ceil(args.rotate_gib * (1 << 30) / per_copy)))
    Ws, Ks, Vs, Xs = [w0], [run.k_cache[0]], [run.v_cache[0]], [x1]
    for _ in range(copies - 1):
        Ws.append(w0.clone()); Ks.append(run.k_cache[0].clone())
        Vs.append(run.v_cache[0].clone()); Xs.append(x1.clone())
    torch.cuda.synchronize()
    eprint(f"[bench] {name}: R={R} rows/step, {copies} copies x {per_copy / 2**20:.1f} MiB "
           f"= {copies * per_copy / 2**30:.2f} GiB rotated")

    def qkv(c, s=st, X=Xs):
        dllm.qkv_rope_cachewrite_paged(X[c], Ws[c], s.pos, s.cu_q, s.logical, run.page_table, wl.max_pages,
                                       s.slot, s.q, Ks[c], Vs[c], sh.n_heads, sh.head_dim, sh.rope_base, s.ws_qkv)

    def attn(c, s=st, mass=True):
        dllm.sched_attention(s.q, s.cu_q, Ks[c], Vs[c], run.page_table, wl.max_pages, s.kv_len, s.o,
                             s.ws_attn, sh.n_heads, sh.head_dim, s.max_kv, mask_bits=s.mask_bits,
                             mask_off=s.mask_off, mass_count=s.mass_count if mass else None,
                             max_mass_rows=s.max_mass if mass else 0, mass_accum=run.mass if mass else None,
                             n_cap=run.n_cap, mass_overwrite=mass)

    def step(c):
        qkv(c)
        attn(c)
        run.topk(clear_mass=False)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i % copies)
    torch.cuda.synchronize()

    # ---- plain stream launches, HIP events around every kernel ----
    K = max(20, args.steps * 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(K):
        c = i % copies
        e = evs[i]
        e[0].record(stream)
        qkv(c)
        e[1].record(stream)
        attn(c)
        e[2].record(stream)
        run.topk(clear_mass=False)
        e[3].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    plain_ms = t_start.elapsed_time(t_end) / K
    names = ["qkv_rope_cachewrite", "sched_attention", "topk_tracked"]
    per = {n: pct([evs[i][j].elapsed_time(evs[i][j + 1]) * 1e3 for i in range(K)]) for j, n in enumerate(names)}

    graph_ms = None if args.no_graph else _graph_time(step, copies, K, args.warmup, stream)
    step_ms = graph_ms if graph_ms is not None else plain_ms
    wk = layer_work(sh, rows1)
    # the dominant kernel alone: back-to-back launches (one per copy) in one
    # graph, so its per-launch time is the kernel plus the dispatch gap only
    qkv_us = per["qkv_rope_cachewrite"]["mean"]
    if not args.no_graph:
        qkv_us = _graph_time(lambda _c: [qkv(c) for c in range(copies)], 1, max(1, K // copies), 1,
                             stream) * 1e3 / copies
    kernels = {
        "qkv_rope_cachewrite": {"us": qkv_us, "us_events_pct": per["qkv_rope_cachewrite"],
                                "alg_bytes": wk["qkv_bytes"], "alg_flops": wk["qkv_flops"],
                                "bound": wk["qkv_bound"], "frac": wk["qkv_bound_us"] / qkv_us},
        "sched_attention": {"us": per["sched_attention"]["mean"], "us_pct": per["sched_attention"],
                            "alg_bytes": wk["attn_bytes"], "alg_flops": wk["attn_flops"],
                            "bound": wk["attn_bound"], "frac": wk["attn_bound_us"] / per["sched_attention"]["mean"]},
        "topk_tracked": {"us": per["topk_tracked"]["mean"], "us_pct": per["topk_tracked"]},
    }
    hbm = wk["qkv_bound"] == "hbm"
    out = {
        "metric": METRIC, "value": R / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.dtype, "data": "synthetic",
        "config": {"workload": describe(name), "rows_per_step": R, "layers": 1, "batch": wl.n_seq,
                   "d_model": sh.d_model, "heads": sh.n_heads, "head_dim": sh.head_dim,
                   "kv_len": [int(k) for k in rows1.kv_len], "parallelism": "single GPU",
                   "rotated_copies": copies, "timing": "hipGraph replay" if graph_ms else "stream launches"},
        "plain_launch_ms_per_step": plain_ms, "graph_ms_per_step": graph_ms,
        "step_sum_of_bounds_us": wk["sum_of_bounds_us"], "step_overlap_bound_us": wk["overlap_bound_us"],
        "step_roofline_frac": wk["sum_of_bounds_us"] / (step_ms * 1e3),
        "step_overlap_frac": wk["overlap_bound_us"] / (step_ms * 1e3),
        "kernels": kernels,
        "roofline": {"bound": wk["qkv_bound"], "kernel": "qkv_rope_cachewrite",
                     "achieved": (wk["qkv_bytes"] / 1e9 if hbm else wk["qkv_flops"] / 1e12) / (qkv_us * 1e-6),
                     "peak": HBM_PEAK_GBS if hbm else MFMA_BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if hbm else "TFLOP/s",
                     "frac": wk["qkv_bound_us"] / qkv_us,
                     "traffic": counter_traffic(f"qkv_rope_cachewrite_{name}_traffic.json")},
    }
    eprint(f"[bench] {name}: {step_ms * 1e3:.1f} us/step ({out['step_roofline_frac']:.3f} of the step bound), "
           f"kernels {({k: round(v['us'], 1) for k, v in kernels.items()})}")
    if not detail or args.no_graph:
        return out

    # ---- the unfused arm of the same step ----
    qkv_raw = torch.empty(R, 3 * n_out, dtype=st.q.dtype, device=dev)

    def step_unfused(c):
        run.map_slots(st)
        dllm.qkv_project(Xs[c], Ws[c], qkv_raw, sh.n_heads, sh.head_dim, st.ws_qkv)
        dllm.rope_apply(qkv_raw, st.pos, st.q, sh.n_heads, sh.head_dim, sh.rope_base)
        dllm.cache_write(qkv_raw, st.slot, Ks[c], Vs[c], sh.n_heads, sh.head_dim)
        attn(c)
        run.topk(clear_mass=False)
    if sh.dtype == "bf16":
        ums = _graph_time(step_unfused, copies, K, args.warmup, stream)
        out["unfused_arm"] = {"ms_per_step": ums, "fused_speedup": ums / step_ms,
                              "note": "slot mapping, projection to memory, rotary, cache write as separate "
                                      "launches; same attention and top-k"}

    # ---- the full refresh and the block-granular caching steps on the same layer ----
    block = {}
    for mode in W.BLOCK_CACHE_MODES + ("full",):
        rws = W.block_cache_rows(wl, mode) if mode != "full" else rows0
        stm = run.upload_step(rws)
        xm = run.to_device_array(W.activations(wl, rws, 2))
        Xm = [xm] + [xm.clone() for _ in range(copies - 1)]
        mass = mode == "full"     # the full refresh forms the score and runs the top-k

        def mstep(c, stm=stm, Xm=Xm, mass=mass):
            qkv(c, stm, Xm)
            attn(c, stm, mass)
            if mass:
                run.topk(clear_mass=False)
        mms = _graph_time(mstep, copies, K, args.warmup, stream)
        wm = layer_work(sh, rws)
        rec = {"rows": rws.n_rows, "kv_len": [int(k) for k in rws.kv_len], "us_per_step": mms * 1e3,
               "tokens_per_s": rws.n_rows / (mms * 1e-3), "step_sum_of_bounds_us": wm["sum_of_bounds_us"],
               "step_roofline_frac": wm["sum_of_bounds_us"] / (mms * 1e3)}
        if mode == "full":
            out["full_refresh_step"] = rec
        else:
            block[mode] = rec
        del Xm, xm, stm
    out["block_cache_steps"] = block

    # ---- the same step over one-byte E4M3 caches (filled by a full refresh in that format) ----
    if sh.dtype == "bf16":
        run8 = FlashCacheRunner(wl, device=dev, layers=1, kv_format="e4m3")
        st8_0 = run8.upload_step(rows0)
        run8.layer_step(st8_0, run8.to_device_array(W.activations(wl, rows0, 0)), w0, 0)
        run8.topk(clear_mass=True)
        st8 = run8.upload_step(rows1)
        K8 = [run8.k_cache[0]] + [run8.k_cache[0].clone() for _ in range(copies - 1)]
        V8 = [run8.v_cache[0]] + [run8.v_cache[0].clone() for _ in range(copies - 1)]

        def step8(c):
            dllm.qkv_rope_cachewrite_paged(Xs[c], Ws[c], st8.pos, st8.cu_q, st8.logical, run8.page_table,
                                           wl.max_pages, st8.slot, st8.q, K8[c], V8[c], sh.n_heads,
                                           sh.head_dim, sh.rope_base, st8.ws_qkv)
            dllm.sched_attention(st8.q, st8.cu_q, K8[c], V8[c], run8.page_table, wl.max_pages, st8.kv_len,
                                 st8.o, st8.ws_attn, sh.n_heads, sh.head_dim, st8.max_kv,
                                 mask_bits=st8.mask_bits, mask_off=st8.mask_off, mass_count=st8.mass_count,
                                 max_mass_rows=st8.max_mass, mass_accum=run8.mass, n_cap=run8.n_cap,
                                 mass_overwrite=True)
            run8.topk(clear_mass=False)
        lms = _graph_time(step8, copies, K, args.warmup, stream)
        out["e4m3_cache_step"] = {"cache_format": "E4M3 (one byte per K/V element)", "us_per_step": lms * 1e3,
                                  "tokens_per_s": R / (lms * 1e-3), "vs_bf16_cache": step_ms / lms}
        del K8, V8, run8
    return out


def achievable_probes(dev):
    """What this machine reaches on the two resources the roofline prices,
    measured beside the line (context for its fractions, not part of the
    path): a plain 1 GiB device copy (HBM read + write bytes per second), and
    torch's bf16 GEMM (hipBLASLt) on the full-refresh projection's shape,
    65536 x 4096 @ 4096 x 12288 (no rotary, no cache write)."""
    import torch
    res = {}
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b_ = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        b_.copy_(a)
    e0.record()
    for _ in range(5):
        b_.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    res["device_copy_GBs"] = 2 * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b_
    x = torch.randn(65536, 4096, device=dev).to(torch.bfloat16)
    w = torch.randn(12288, 4096, device=dev).mul_(4096 ** -0.5).to(torch.bfloat16)
    wt = w.t().contiguous()
    y = torch.empty(65536, 12288, dtype=torch.bfloat16, device=dev)
    best = None
    # W as stored (out x in: the Linear layer's 2-D product) and W^T laid out (a plain 2-D product)
    for gemm in (lambda: torch.nn.functional.linear(x, w), lambda: torch.matmul(x, wt, out=y)):
        for _ in range(2):
            gemm()
        e0.record()
        for _ in range(5):
            gemm()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        best = ms if best is None else min(best, ms)
    res["library_gemm_TFLOPs"] = 2 * 65536 * 4096 * 12288 / (best * 1e-3) / 1e12
    res["library_gemm_frac"] = res["library_gemm_TFLOPs"] / 2500.0
    res["note"] = ("torch's plain bf16 GEMM and device copy on this GPU, for context; the path's own kernels "
                   "are measured above")
    del x, w, wt, y
    torch.cuda.empty_cache()
    return res


def copy_probe(mib, dev):
    """A plain device copy of `mib` MiB, three times: what the HBM byte
    counters read for known bytes (their calibration)."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b_ = torch.empty_like(a)
    for _ in range(3):
        b_.copy_(a)
    torch.cuda.synchronize()
    eprint(f"[probe] device copy of {mib} MiB, 3 times")


def probe(what, dev, launches=3):
    """Launch one kernel a few times on a fixed shape (for rocprofv3 counter
    passes); inputs are random, outputs unused."""
    import torch
    from io_aware_kv_amd import dllm
    from io_aware_kv_amd import workloads as W
    from io_aware_kv_amd.runner import FlashCacheRunner
    if what.startswith("attn_"):
        wl = W.make_workload("llada_b32")
        run = FlashCacheRunner(wl, device=dev, layers=1)
        rows = W.full_refresh_rows(wl) if what == "attn_full_b32" else W.config_step_rows(wl, W.seeded_tracked(wl, 1))
        st = run.upload_step(rows)
        for c in (run.k_cache[0], run.v_cache[0], st.q):
            c.copy_(torch.randn(c.shape, device=dev).to(c.dtype))
        for _ in range(launches):
            run.attention(st, 0)
    elif what.startswith("qkv:"):
        parts = what.split(":")
        R = int(parts[1])
        if len(parts) > 2:
            dllm.set_tuning("qkv_kernel", parts[2])
        H, D, d = 32, 128, 4096
        w = torch.randn(3 * H * D, d, device=dev).mul_(d ** -0.5).to(torch.bfloat16)
        x = torch.randn(R, d, device=dev).to(torch.bfloat16)
        pos = torch.arange(R, dtype=torch.int32, device=dev)
        q = torch.empty(R, H * D, dtype=torch.bfloat16, device=dev)
        kc, vc = torch.empty_like(q), torch.empty_like(q)
        for _ in range(launches):
            dllm.qkv_rope_cachewrite(x, w, pos, pos, q, kc, vc, H, D, 5e5)
    else:
        raise SystemExit(f"unknown probe {what}")
    torch.cuda.synchronize()
    eprint(f"[probe] {what}: {launches} launches")


def bench_decode(args, dev):
    """Decode-side reductions over one logits row per masked window position,
    at the assumed LM-head width: batch 1 (32 rows) and batch 32 (32 x 32
    rows).  Each call is the two-launch logits pass + decision; calls run back
    to back in a captured graph over enough distinct logits copies (>= 1 GiB)
    that the Infinity Cache cannot serve them.  Algorithmic bytes per call:
    the logits (R x V bf16) plus the per-row outputs."""
    import numpy as np
    import torch
    from io_aware_kv_amd import dllm
    from io_aware_kv_amd import workloads as W
    V = W.VOCAB
    out = {"vocab_assumed": V, "eps": 0.9, "gamma": 0.8}
    stream = torch.cuda.current_stream()
    for name, lens in (("batch1", [32]), ("batch32", [32] * 32)):
        rows = W.decode_rows(21, lens, V, twin_frac=0.05)
        R = int(rows.cu[-1])
        per = R * V * 2
        copies = max(2, int(np.ceil((1 << 30) / per)))
        L = [W.decode_logits_device(21 + c, rows, V, dev) for c in range(copies)]
        cu = torch.from_numpy(rows.cu).to(dev)
        draft = torch.from_numpy(rows.draft).to(dev)
        tok = torch.empty(R, dtype=torch.int32, device=dev)
        conf = torch.empty(R, dtype=torch.float32, device=dev)
        flag = torch.empty(R, dtype=torch.uint8, device=dev)
        cnt = torch.empty(len(lens), dtype=torch.int32, device=dev)
        ws = torch.empty(dllm.confidence_workspace(R, V) // 4 + 4, dtype=torch.float32, device=dev)
        res = {"rows": R, "sequences": len(lens), "logits_bytes": per, "rotated_copies": copies}
        for kind in ("commit", "verify"):
            def call(c):
                if kind == "commit":
                    dllm.decode_commit(L[c], cu, 0.9, tok, conf, flag, cnt, ws)
                else:
                    dllm.decode_verify(L[c], cu, draft, 0.8, tok, conf, flag, cnt, ws)
            call(0)
            torch.cuda.synchronize()
            reps = max(2, min(50, args.steps * 40 // copies))
            us = _graph_time(lambda _c: [call(c) for c in range(copies)], 1, reps, 1, stream) * 1e3 / copies
            alg = per + R * (4 + 4 + 1) + len(lens) * 4 + (R * 4 if kind == "verify" else 0)
            gbs = alg / (us * 1e-6) / 1e9
            res[kind] = {"us_per_call": us, "alg_bytes": alg, "achieved_GBs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                         "rows_per_s": R / (us * 1e-6)}
        out[name] = res
        del L
        torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untouched, on this host's cores
# ---------------------------------------------------------------------------

def host_setup():
    """Set the BLAS pool to every core this process may run on (capped at the
    thread share the environment grants, OMP_NUM_THREADS, where set) and
    describe the host: cores, CPU model, BLAS library."""
    visible = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    cores = min(visible, share) if share > 0 else visible
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        blas = [f"{i.get('internal_api')} {i.get('version')} ({os.path.basename(i.get('filepath', ''))}, "
                f"{i.get('num_threads')} threads)" for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception as e:       # threadpoolctl missing
        blas = [f"unknown ({e.__class__.__name__})"]
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return limiter, {"cores": cores, "cores_visible": visible, "cpu_model": model, "blas": blas}


def cpu_baseline_b32():
    """The oracle on a bounded sample of the headline workload: one layer,
    two sequences of each step type (full refresh: 2048 rows over 2048 keys;
    cache phase: 72 rows over 2048 keys), each sequence a separate oracle
    call.  The oracle treats sequences and layers independently, so its
    refreshed tokens/s per layer for the whole batch follows by scaling the
    time linearly by sequences (32 / 2); labelled extrapolated."""
    import numpy as np
    import oracle as O
    from io_aware_kv_amd import workloads as W
    limiter, host = host_setup()
    wl = W.make_workload("llada_b32")
    sh = wl.shape
    n = sh.n_heads * sh.head_dim
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3 * n, sh.d_model)) / np.sqrt(sh.d_model)
    pages = wl.max_pages
    table = O.build_block_table([pages], list(range(pages)), pages, pages)
    kc = np.zeros((pages * W.PAGE, n))
    vc = np.zeros_like(kc)
    full = W.full_refresh_rows(wl)
    cache = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    t, meas, rows_sampled = {}, {}, {}
    for kind, rws in (("full", full), ("cache", cache)):
        el = 0.0
        nr = 0
        for b in (0, 1):
            r0, r1 = int(rws.cu_q[b]), int(rws.cu_q[b + 1])
            x = rng.standard_normal((r1 - r0, sh.d_model))
            t0 = time.perf_counter()
            O.layer_step(x, w, rws.pos[r0:r1], rws.logical[r0:r1], [0, r1 - r0], [int(rws.kv_len[b])],
                         [int(rws.mass_count[b])], kc, vc, table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
            el += time.perf_counter() - t0
            nr += r1 - r0
        meas[kind] = el
        t[kind] = el * wl.n_seq / 2          # per layer for the batch, extrapolated
        rows_sampled[kind] = nr
    value = (full.n_rows + cache.n_rows) / (t["full"] + t["cache"])
    del limiter
    return {"value": value, "unit": "tokens/s", **host, "kind": "oracle",
            "sample": f"extrapolated: one layer, 2 of the 32 sequences of each step type (full refresh "
                      f"{rows_sampled['full']} rows, cache phase {rows_sampled['cache']} rows, 2048 keys each), "
                      f"fp64 NumPy, measured {meas['full']:.1f} s + {meas['cache']:.1f} s and scaled by 16 to the "
                      f"batch; the same alternating mix of step types as the GPU figure"}


def cpu_baseline(name, seconds):
    """The oracle on the same single-layer step (projection, RoPE, scatter,
    attention, formula-(2) term, top-k), repeated for about `seconds`."""
    import numpy as np
    import oracle as O
    from io_aware_kv_amd import workloads as W
    limiter, host = host_setup()
    wl = W.make_workload(name)
    sh = wl.shape
    rows = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
    w = W.as_f64(wl, W.weights(wl, 0))
    x = W.as_f64(wl, W.activations(wl, rows, 1))
    n_out = sh.n_heads * sh.head_dim
    kc = np.zeros((wl.pool_pages * W.PAGE, n_out))
    vc = np.zeros_like(kc)
    elig = wl.eligible().astype(bool)
    reps = 0
    t0 = time.perf_counter()
    while True:
        out = O.layer_step(x, w, rows.pos, rows.logical, rows.cu_q, rows.kv_len, rows.mass_count, kc, vc,
                           table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE, visible=rows.visible)
        O.topk(out["mass"], elig, sh.top_k)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    del limiter
    return {"value": rows.n_rows * reps / el, "unit": "tokens/s", **host, "kind": "oracle",
            "sample": f"{reps} oracle steps of the same workload ({rows.n_rows} rows each, fp64 NumPy) "
                      f"in {el:.1f} s"}


if __name__ == "__main__":
    main()
