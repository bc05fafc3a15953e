#!/usr/bin/env python3
"""Benchmark of the Flash-Cache per-layer denoising step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
slot map -> fused QKV + RoPE + cache write -> scheduled attention with the
formula-(2) column mass -> top-k of the tracked set.  The default workload is
the LLaDA-8B-shaped layer (d_model 4096, 32 heads x 128, bf16) with one
sequence of 512 tokens in the cache phase: 72 refreshed rows (32 masked
window + 8 newly decoded + 32 tracked).

Metric: refreshed tokens/s per layer = rows refreshed per step / step time.
Inputs are resident in HBM before timing starts.  To keep the 256 MB
Infinity Cache from serving the weights and caches, the timed loop rotates
over enough independent copies (weights, caches, inputs) to span >= 1 GiB.

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


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llada_b1",
                   choices=["llada_b1", "mixed_b8", "verify_b4", "llada_b32"])
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--no-graph", action="store_true")
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from io_aware_kv_amd import dllm
    from io_aware_kv_amd import workloads as W
    from io_aware_kv_amd.runner import FlashCacheRunner

    dllm.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.probe:
        return probe(args.probe, dev)
    if args.workload == "llada_b32":
        return bench_layers(args, dev)
    wl = W.make_workload(args.workload)
    sh = wl.shape
    n_out = sh.n_heads * sh.head_dim

    # ---- step 0 (full refresh) on the GPU fills the cache and picks the tracked rows ----
    run = FlashCacheRunner(wl, device=dev, layers=1)
    w_raw = W.weights(wl, 0)
    w0 = run.to_device_array(w_raw)
    rows0 = W.full_refresh_rows(wl)
    st0 = run.upload_step(rows0)
    x0 = run.to_device_array(W.activations(wl, rows0, 0))
    run.layer_step(st0, x0, w0, 0)
    run.topk(clear_mass=True)
    idx = run.top_idx.cpu().numpy()
    tracked = [idx[b][idx[b] >= 0] for b in range(wl.n_seq)]
    rows1 = W.config_step_rows(wl, tracked)
    R = rows1.n_rows
    st = run.upload_step(rows1)
    x1 = run.to_device_array(W.activations(wl, rows1, 1))
    del st0, x0

    # ---- buffer rotation over independent copies ----
    per_copy = (w0.numel() * w0.element_size() + 2 * run.k_cache[0].numel() * run.k_cache[0].element_size()
                + x1.numel() * x1.element_size())
    copies = max(1, int(np.ceil(args.rotate_gib * (1 << 30) / per_copy)))
    Ws, Ks, Vs, Xs = [w0], [run.k_cache[0]], [run.v_cache[0]], [x1]
    for _ in range(copies - 1):
        Ws.append(w0.clone()); Ks.append(run.k_cache[0].clone())
        Vs.append(run.v_cache[0].clone()); Xs.append(x1.clone())
    torch.cuda.synchronize()
    eprint(f"[bench] {args.workload}: R={R} rows/step, {copies} copies x {per_copy / 2**20:.1f} MiB "
           f"= {copies * per_copy / 2**30:.2f} GiB rotated")

    def step(i):
        c = i % copies
        dllm.qkv_rope_cachewrite_paged(Xs[c], Ws[c], st.pos, st.cu_q, st.logical, run.page_table,
                                       wl.max_pages, st.slot, st.q, Ks[c], Vs[c], sh.n_heads,
                                       sh.head_dim, sh.rope_base, st.ws_qkv)
        dllm.sched_attention(st.q, st.cu_q, Ks[c], Vs[c], run.page_table, wl.max_pages, st.kv_len, st.o,
                             st.ws_attn, sh.n_heads, sh.head_dim, st.max_kv, mask_bits=st.mask_bits,
                             mask_off=st.mask_off, mass_count=st.mass_count, max_mass_rows=st.max_mass,
                             mass_accum=run.mass, n_cap=run.n_cap, mass_overwrite=True)
        run.topk(clear_mass=False)

    # the unfused comparison arm of the same step: slot mapping, projection to
    # memory, rotary, cache write as launches of their own, then attention, top-k
    qkv_raw = torch.empty(R, 3 * n_out, dtype=st.q.dtype, device=dev)

    def step_unfused(i):
        c = i % copies
        run.map_slots(st)
        dllm.qkv_project(Xs[c], Ws[c], qkv_raw, sh.n_heads, sh.head_dim, st.ws_qkv)
        dllm.rope_apply(qkv_raw, st.pos, st.q, sh.n_heads, sh.head_dim, sh.rope_base)
        dllm.cache_write(qkv_raw, st.slot, Ks[c], Vs[c], sh.n_heads, sh.head_dim)
        dllm.sched_attention(st.q, st.cu_q, Ks[c], Vs[c], run.page_table, wl.max_pages, st.kv_len, st.o,
                             st.ws_attn, sh.n_heads, sh.head_dim, st.max_kv, mask_bits=st.mask_bits,
                             mask_off=st.mask_off, mass_count=st.mass_count, max_mass_rows=st.max_mass,
                             mass_accum=run.mass, n_cap=run.n_cap, mass_overwrite=True)
        run.topk(clear_mass=False)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- plain stream launches, HIP events around every kernel ----
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        c = i % copies
        e = evs[i]
        e[0].record(stream)
        dllm.qkv_rope_cachewrite_paged(Xs[c], Ws[c], st.pos, st.cu_q, st.logical, run.page_table,
                                       wl.max_pages, st.slot, st.q, Ks[c], Vs[c], sh.n_heads,
                                       sh.head_dim, sh.rope_base, st.ws_qkv)
        e[1].record(stream)
        dllm.sched_attention(st.q, st.cu_q, Ks[c], Vs[c], run.page_table, wl.max_pages, st.kv_len, st.o,
                             st.ws_attn, sh.n_heads, sh.head_dim, st.max_kv, mask_bits=st.mask_bits,
                             mask_off=st.mask_off, mass_count=st.mass_count, max_mass_rows=st.max_mass,
                             mass_accum=run.mass, n_cap=run.n_cap, mass_overwrite=True)
        e[2].record(stream)
        run.topk(clear_mass=False)
        e[3].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    plain_ms = t_start.elapsed_time(t_end) / K
    names = ["qkv_rope_cachewrite", "sched_attention", "topk_tracked"]
    per = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)])) * 1e3
           for j, n in enumerate(names)}
    per_p50 = {n: float(np.median([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)])) * 1e3
               for j, n in enumerate(names)}

    # ---- captured hipGraph replay (one graph per copy) ----
    graph_ms = None
    if not args.no_graph:
        graphs = []
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    step(c)
                graphs.append(g)
        stream.wait_stream(cs)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for i in range(K):
            graphs[i % copies].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K

    # ---- the dominant kernel alone: back-to-back launches (one per copy) in a
    # graph, so the per-launch time is the kernel plus the dispatch gap only ----
    qkv_graph_us = None
    if not args.no_graph:
        qg = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cs):
            with torch.cuda.graph(qg, stream=cs):
                for c in range(copies):
                    dllm.qkv_rope_cachewrite_paged(Xs[c], Ws[c], st.pos, st.cu_q, st.logical, run.page_table,
                                                   wl.max_pages, st.slot, st.q, Ks[c], Vs[c], sh.n_heads,
                                                   sh.head_dim, sh.rope_base, st.ws_qkv)
        stream.wait_stream(cs)
        torch.cuda.synchronize()
        reps = max(1, K // copies)
        qg.replay()
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        for _ in range(reps):
            qg.replay()
        q1.record(stream)
        torch.cuda.synchronize()
        qkv_graph_us = q0.elapsed_time(q1) / (reps * copies) * 1e3

    # ---- the unfused arm, same replay scheme ----
    unfused_ms = None
    if not args.no_graph and sh.dtype == "bf16":
        ugraphs = []
        with torch.cuda.stream(cs):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    step_unfused(c)
                ugraphs.append(g)
        stream.wait_stream(cs)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            ugraphs[i % copies].replay()
        torch.cuda.synchronize()
        u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        u0.record(stream)
        for i in range(K):
            ugraphs[i % copies].replay()
        u1.record(stream)
        torch.cuda.synchronize()
        unfused_ms = u0.elapsed_time(u1) / K

    # ---- block-granular caching steps over the same layer, caches and kernels:
    # DualCache (the current block only) and the active window of PrefixCache /
    # FreeCache (the current block and every later block) ----
    block = None
    full = None
    if not args.no_graph:
        block = {}
        for mode in W.BLOCK_CACHE_MODES + ("full",):
            rws = W.block_cache_rows(wl, mode) if mode != "full" else rows0
            stm = run.upload_step(rws)
            xm = run.to_device_array(W.activations(wl, rws, 2))
            Xm = [xm] + [xm.clone() for _ in range(copies - 1)]
            mass = mode == "full"     # the full refresh forms the score and runs the top-k

            def mstep(c, stm=stm, Xm=Xm, mass=mass):
                dllm.qkv_rope_cachewrite_paged(Xm[c], Ws[c], stm.pos, stm.cu_q, stm.logical, run.page_table,
                                               wl.max_pages, stm.slot, stm.q, Ks[c], Vs[c], sh.n_heads,
                                               sh.head_dim, sh.rope_base, stm.ws_qkv)
                dllm.sched_attention(stm.q, stm.cu_q, Ks[c], Vs[c], run.page_table, wl.max_pages, stm.kv_len,
                                     stm.o, stm.ws_attn, sh.n_heads, sh.head_dim, stm.max_kv,
                                     mass_count=stm.mass_count if mass else None,
                                     max_mass_rows=stm.max_mass if mass else 0,
                                     mass_accum=run.mass if mass else None, n_cap=run.n_cap,
                                     mass_overwrite=mass)
                if mass:
                    run.topk(clear_mass=False)
            mg = []
            with torch.cuda.stream(cs):
                for c in range(copies):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=cs):
                        mstep(c)
                    mg.append(g)
            stream.wait_stream(cs)
            torch.cuda.synchronize()
            for i in range(args.warmup):
                mg[i % copies].replay()
            torch.cuda.synchronize()
            m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            m0.record(stream)
            for i in range(K):
                mg[i % copies].replay()
            m1.record(stream)
            torch.cuda.synchronize()
            mms = m0.elapsed_time(m1) / K
            rec = {"rows": rws.n_rows, "kv_len": [int(k) for k in rws.kv_len], "us_per_step": mms * 1e3,
                   "tokens_per_s": rws.n_rows / (mms * 1e-3)}
            if mode == "full":
                # step bound: projection max(W bytes, MFMA) + attention max(K/V bytes, MFMA), bf16 peaks
                Rf = rws.n_rows
                pb = max((3 * n_out * sh.d_model + 4 * Rf * n_out) * 2 / (HBM_PEAK_GBS * 1e9),
                         2 * Rf * sh.d_model * 3 * n_out / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                kv = rws.kv_len.astype(np.int64)
                cu = rws.cu_q.astype(np.int64)
                af = sum(4 * int(cu[b + 1] - cu[b]) * int(kv[b]) * n_out for b in range(wl.n_seq))
                ab = max((int(kv.sum()) * 2 + 2 * Rf) * n_out * 2 / (HBM_PEAK_GBS * 1e9),
                         af / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                rec["step_roofline_us"] = (pb + ab) * 1e6
                rec["step_roofline_frac"] = (pb + ab) * 1e6 / rec["us_per_step"]
                full = rec
            else:
                block[mode] = rec
            del mg, Xm, xm, stm
        torch.cuda.synchronize()

    # ---- the same step over one-byte E4M3 caches (filled by a full refresh in that format) ----
    lowbit = None
    if not args.no_graph and sh.dtype == "bf16":
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
        g8 = []
        with torch.cuda.stream(cs):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    step8(c)
                g8.append(g)
        stream.wait_stream(cs)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            g8[i % copies].replay()
        torch.cuda.synchronize()
        l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        l0.record(stream)
        for i in range(K):
            g8[i % copies].replay()
        l1.record(stream)
        torch.cuda.synchronize()
        lms = l0.elapsed_time(l1) / K
        lowbit = {"cache_format": "E4M3 (one byte per K/V element)", "us_per_step": lms * 1e3,
                  "tokens_per_s": R / (lms * 1e-3), "vs_bf16_cache": graph_ms / lms if graph_ms else None}
        del g8, K8, V8

    step_ms = graph_ms if graph_ms is not None else plain_ms
    value = R / (step_ms * 1e-3)

    # ---- roofline of the dominant kernel (the weight-streaming projection) ----
    d = sh.d_model
    el = 2 if sh.dtype == "bf16" else 4
    qkv_bytes = 3 * n_out * d * el + R * d * el + R * n_out * el + 2 * R * n_out * el
    # launch duration of the dominant kernel: back-to-back graph launches when
    # timed (closest to the kernel trace), else the events around each launch
    qkv_us = qkv_graph_us if qkv_graph_us is not None else per["qkv_rope_cachewrite"]
    achieved = qkv_bytes / (qkv_us * 1e-6) / 1e9
    kv_keys = int(rows1.kv_len.sum())
    attn_bytes = kv_keys * 2 * n_out * el + 2 * R * n_out * el
    attn_flops = 0
    for b in range(wl.n_seq):
        rb = int(rows1.cu_q[b + 1] - rows1.cu_q[b])
        vis = rows1.visible[b].sum() if rows1.visible is not None else rb * int(rows1.kv_len[b])
        attn_flops += 4 * int(vis) * n_out
    qkv_flops = 2 * R * d * 3 * n_out
    b_qkv = max(qkv_bytes / (HBM_PEAK_GBS * 1e9), qkv_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    b_att = max(attn_bytes / (HBM_PEAK_GBS * 1e9), attn_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    step_bound_us = (b_qkv + b_att) * 1e6
    kernels = {
        "qkv_rope_cachewrite": {"us": qkv_us, "us_events": per["qkv_rope_cachewrite"],
                                "us_events_p50": per_p50["qkv_rope_cachewrite"],
                                "alg_bytes": qkv_bytes, "alg_flops": qkv_flops,
                                "bound": "hbm" if qkv_bytes / 8e12 >= qkv_flops / 2.5e15 else "mfma",
                                "frac": b_qkv * 1e6 / qkv_us},
        "sched_attention": {"us": per["sched_attention"], "us_p50": per_p50["sched_attention"],
                            "alg_bytes": attn_bytes, "alg_flops": attn_flops,
                            "bound": "hbm" if attn_bytes / 8e12 >= attn_flops / 2.5e15 else "mfma",
                            "frac": b_att * 1e6 / per["sched_attention"]},
        "topk_tracked": {"us": per["topk_tracked"]},
    }
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "qkv_rope_cachewrite_llada_b1_traffic.json")
    if args.workload == "llada_b1" and os.path.exists(tfile):
        # counter-measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by
        # a plain-copy calibration); only valid for the kernel source profiled
        import hashlib
        tj = json.load(open(tfile))
        src = open(os.path.join(ROOT, tj["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() == tj["source_sha256"]:
            traffic = tj["bytes_per_launch"]

    # ---- optional plain copy (calibrates the HBM byte counters) ----
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()

    # ---- decode side (after the model head), timed on its own ----
    decode = None
    if not args.no_decode and not args.no_graph:
        decode = bench_decode(args, dev)

    # ---- CPU baseline: the oracle on host cores, bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, rows1, args.cpu_seconds)

    out = {
        "metric": "refreshed tokens/s per layer (cache-update+attention)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": describe(args.workload), "rows_per_step": R, "layers": 1,
                   "batch": wl.n_seq, "d_model": sh.d_model, "heads": sh.n_heads, "head_dim": sh.head_dim,
                   "kv_len": [int(k) for k in rows1.kv_len], "parallelism": "single GPU",
                   "rotated_copies": copies, "timing": "hipGraph replay" if graph_ms else "stream launches"},
        "plain_launch_ms_per_step": plain_ms,
        "graph_ms_per_step": graph_ms,
        "step_roofline_us": step_bound_us,
        "step_roofline_frac": step_bound_us / (step_ms * 1e3),
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": "qkv_rope_cachewrite", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic},
        "unfused_arm": None if unfused_ms is None else {
            "ms_per_step": unfused_ms, "fused_speedup": unfused_ms / step_ms,
            "note": "slot mapping, projection to memory, rotary, cache write as separate launches; same attention and top-k"},
        "full_refresh_step": full,
        "e4m3_cache_step": lowbit,
        "block_cache_steps": block,
        "decode_side": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


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
            os.environ["DLLM_QKV_KERNEL"] = parts[2]
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
            cs = torch.cuda.Stream()
            cs.wait_stream(stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cs):
                with torch.cuda.graph(g, stream=cs):
                    for c in range(copies):
                        call(c)
            stream.wait_stream(cs)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            reps = max(2, min(50, args.steps * 4 // copies))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / (reps * copies) * 1e3
            alg = per + R * (4 + 4 + 1) + len(lens) * 4 + (R * 4 if kind == "verify" else 0)
            gbs = alg / (us * 1e-6) / 1e9
            res[kind] = {"us_per_call": us, "alg_bytes": alg, "achieved_GBs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                         "rows_per_s": R / (us * 1e-6)}
        out[name] = res
        del L
        torch.cuda.synchronize()
    return out


def bench_layers(args, dev):
    """32-layer batch-32 sweep: alternating full-refresh steps (2048 rows per
    sequence per layer) and cache-phase steps (72 rows per sequence per layer),
    one top-k per step after the last layer."""
    import numpy as np
    import torch
    from io_aware_kv_amd import dllm
    from io_aware_kv_amd import workloads as W
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = W.make_workload("llada_b32")
    sh = wl.shape
    L, n = sh.layers, sh.n_heads * sh.head_dim
    run = FlashCacheRunner(wl, device=dev)
    Ws = [W.device_weights(wl, l, dev) for l in range(L)]
    rows = {"full": W.full_refresh_rows(wl)}
    sts = {"full": run.upload_step(rows["full"])}
    xs = {"full": [W.device_activations(wl, rows["full"], 0, l, dev) for l in range(L)]}

    def step(kind, ev=None, unfused=False):
        st = sts[kind]
        mass = kind in ("full", "cache", "cache_mid")    # block-cache steps have no formula-(2) rows
        run.map_slots(st)
        for l in range(L):
            if ev is not None:
                ev[l][0].record()
            if unfused:
                run.cache_update_unfused(st, xs[kind][l], Ws[l], l)
            else:
                run.cache_update(st, xs[kind][l], Ws[l], l)
            if ev is not None:
                ev[l][1].record()
            # cache_mid: the score only from the middle layers 5..20 (1-based); the
            # first scoring layer stores its term, the others add theirs
            first = 4 if kind == "cache_mid" else 0
            run.attention(st, l, with_mass=mass and (kind != "cache_mid" or 5 <= l + 1 <= 20),
                          mass_overwrite=l == first)
            if ev is not None:
                ev[l][2].record()
        if mass:
            run.topk(clear_mass=False)

    step("full")
    idx = run.top_idx.cpu().numpy()
    rows["cache"] = W.config_step_rows(wl, [idx[b][idx[b] >= 0] for b in range(wl.n_seq)])
    sts["cache"] = run.upload_step(rows["cache"])
    xs["cache"] = [W.device_activations(wl, rows["cache"], 1, l, dev) for l in range(L)]
    rows["cache_mid"], sts["cache_mid"], xs["cache_mid"] = rows["cache"], sts["cache"], xs["cache"]
    for mode in W.BLOCK_CACHE_MODES:
        rows[mode] = W.block_cache_rows(wl, mode)
        sts[mode] = run.upload_step(rows[mode])
        xs[mode] = [W.device_activations(wl, rows[mode], 2, l, dev) for l in range(L)]
    # the same cache-phase step over one-byte E4M3 caches (a second set of
    # caches, filled by a full refresh in that format)
    run8 = FlashCacheRunner(wl, device=dev, kv_format="e4m3")
    st8 = {"full": run8.upload_step(rows["full"]), "cache": run8.upload_step(rows["cache"])}

    def step8(kind, ev=None):
        st = st8[kind]
        run8.map_slots(st)
        for l in range(L):
            if ev is not None:
                ev[l][0].record()
            run8.cache_update(st, xs[kind][l], Ws[l], l)
            if ev is not None:
                ev[l][1].record()
            run8.attention(st, l, mass_overwrite=l == 0)
            if ev is not None:
                ev[l][2].record()
        run8.topk(clear_mass=False)

    step8("full")
    for _ in range(max(1, args.warmup // 10)):
        step("cache")
        step("full")
        step8("cache")
    torch.cuda.synchronize()
    K = max(2, min(args.steps, 10))
    res = {}
    for kind in ("full", "cache", "cache_mid", "cache_e4m3") + W.BLOCK_CACHE_MODES:
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(L)] for _ in range(K)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(K):
            if kind == "cache_e4m3":
                step8("cache", evs[i])
            else:
                step(kind, evs[i])
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / K
        qkv_us = float(np.mean([evs[i][l][0].elapsed_time(evs[i][l][1]) for i in range(K) for l in range(L)])) * 1e3
        att_us = float(np.mean([evs[i][l][1].elapsed_time(evs[i][l][2]) for i in range(K) for l in range(L)])) * 1e3
        rk = rows["cache"] if kind == "cache_e4m3" else rows[kind]
        R = rk.n_rows
        kv = rk.kv_len.astype(np.int64)
        cu = rk.cu_q.astype(np.int64)
        cache_el = 1 if kind == "cache_e4m3" else 2        # bytes per cached K/V element
        qkv_flops = 2 * R * sh.d_model * 3 * n
        qkv_bytes = 3 * n * sh.d_model * 2 + R * (16 + 8 * cache_el) * 1024
        att_flops = int(sum(4 * (cu[b + 1] - cu[b]) * kv[b] * n for b in range(wl.n_seq)))
        att_bytes = int(kv.sum()) * 2 * n * cache_el + 2 * R * n * 2
        b_qkv = max(qkv_bytes / (HBM_PEAK_GBS * 1e9), qkv_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
        b_att = max(att_bytes / (HBM_PEAK_GBS * 1e9), att_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
        res[kind] = {"rows_per_layer": R, "ms_per_step": ms, "us_per_layer": ms * 1e3 / L,
                     "tokens_per_s_per_layer": R / (ms * 1e-3 / L),
                     "qkv_us": qkv_us, "qkv_bound_us": b_qkv, "qkv_frac": b_qkv / qkv_us,
                     "qkv_bound": "mfma" if qkv_flops / 2.5e15 > qkv_bytes / 8e12 else "hbm",
                     "attn_us": att_us, "attn_bound_us": b_att, "attn_frac": b_att / att_us,
                     "attn_bound": "mfma" if att_flops / 2.5e15 > att_bytes / 8e12 else "hbm",
                     "layer_roofline_frac": (b_qkv + b_att) / (ms * 1e3 / L)}
        eprint(f"[bench] llada_b32 {kind}: {res[kind]}")
    # the unfused comparison arm on the cache-phase step (per-layer projection,
    # rotary and cache write as three launches with q|k|v in memory)
    step("cache", unfused=True)
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(L)] for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(K):
        step("cache", evs[i], unfused=True)
    t1.record()
    torch.cuda.synchronize()
    ums = t0.elapsed_time(t1) / K
    unfused = {"us_per_layer": ums * 1e3 / L,
               "update_us": float(np.mean([evs[i][l][0].elapsed_time(evs[i][l][1]) for i in range(K) for l in range(L)])) * 1e3,
               "fused_speedup_per_layer": ums / res["cache"]["ms_per_step"],
               "fused_update_speedup": float(np.mean([evs[i][l][0].elapsed_time(evs[i][l][1]) for i in range(K) for l in range(L)])) * 1e3 / res["cache"]["qkv_us"]}
    eprint(f"[bench] llada_b32 cache, unfused arm: {unfused}")
    tot_rows = sum(res[k]["rows_per_layer"] for k in ("full", "cache"))
    tot_ms = sum(res[k]["ms_per_step"] for k in ("full", "cache"))
    block = {k: res.pop(k) for k in W.BLOCK_CACHE_MODES}
    mid = res.pop("cache_mid")
    e4m3 = res.pop("cache_e4m3")
    value = tot_rows / (tot_ms * 1e-3 / L)
    dom = res["full"]
    out = {
        "metric": "refreshed tokens/s per layer (cache-update+attention)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": 2 * K, "warmup": args.warmup,
        "ms_per_step": tot_ms / 2, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LLaDA-8B-shaped 32-layer sweep (d_model 4096, 32x128 heads, bf16), batch 32, "
                               "context 2048 (prompt 1536 + gen 512); alternating full-refresh (2048 rows/seq) and "
                               "cache-phase (72 rows/seq) steps, top-32 once per step",
                   "layers": L, "batch": wl.n_seq, "parallelism": "single GPU", "timing": "stream launches"},
        "steps_detail": res,
        "block_cache_steps": block,
        "cache_phase_middle_layer_score": mid,
        "cache_phase_e4m3_cache": e4m3,
        "unfused_arm_cache_phase": unfused,
        "roofline": {"bound": "mfma", "kernel": "qkv_rope_cachewrite (full refresh)",
                     "achieved": 2 * dom["rows_per_layer"] * sh.d_model * 3 * n / (dom["qkv_us"] * 1e-6) / 1e12,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": dom["qkv_frac"], "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_b32(wl, rows["cache"], args.cpu_seconds),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_b32(wl, rows, seconds):
    """The oracle on one sequence's cache-phase rows of one layer (72 rows over
    2048 keys), repeated for about `seconds`; tokens/s scales linearly with
    rows, sequences and layers, so this is the batch figure too."""
    import numpy as np
    import oracle as O
    from io_aware_kv_amd import workloads as W
    sh = wl.shape
    n = sh.n_heads * sh.head_dim
    r0, r1 = int(rows.cu_q[0]), int(rows.cu_q[1])
    kv = int(rows.kv_len[0])
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3 * n, sh.d_model)) / np.sqrt(sh.d_model)
    x = rng.standard_normal((r1 - r0, sh.d_model))
    pages = (kv + W.PAGE - 1) // W.PAGE
    table = O.build_block_table([pages], list(range(pages)), pages, pages)
    kc = np.zeros((pages * W.PAGE, n))
    vc = np.zeros_like(kc)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.layer_step(x, w, rows.pos[r0:r1], rows.logical[r0:r1], [0, r1 - r0], [kv], [int(rows.mass_count[0])],
                     kc, vc, table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": (r1 - r0) * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} oracle layer steps of one sequence's cache-phase rows ({r1 - r0} rows, {kv} keys, "
                      f"fp64 NumPy) in {el:.1f} s; extrapolated linearly to the batch"}


def describe(name):
    return {
        "llada_b1": "LLaDA-8B-shaped layer (d_model 4096, 32x128 heads, bf16), batch 1, context 512 "
                    "(prompt 256 + gen 256), cache-phase step: 32 window + 8 new + 32 tracked rows",
        "mixed_b8": "LLaDA-8B-shaped layer, batch 8 mixed: 6 cache-phase sequences (40-72 rows, context "
                    "512-1024) + 2 full refreshes (512, 1024 rows)",
        "verify_b4": "LLaDA-8B-shaped layer, batch 4, context 1024 + 32 view slots, verify step with "
                     "16 draft + 16 mask views + 40 ordinary rows per sequence under the verify mask",
    }[name]


def cpu_baseline(wl, rows, seconds):
    """The oracle, untouched, on this host's cores: the same step (projection,
    RoPE, scatter, attention, formula-(2) term, top-k) on the same rows,
    repeated for about `seconds`."""
    import numpy as np
    import oracle as O
    from io_aware_kv_amd import workloads as W
    sh = wl.shape
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
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
    return {"value": rows.n_rows * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} oracle steps of the same workload ({rows.n_rows} rows each, fp64 NumPy) "
                      f"in {el:.1f} s"}


if __name__ == "__main__":
    main()
