"""Full-size parity of the 32-layer LLaDA-8B-shaped workload (batch 32,
context 2048): a full-refresh step (65536 rows per layer) and a cache-phase
step (2304 rows per layer), every layer accumulating the formula (2) score and
one top-k after the last layer.

The GPU runs everything at full size.  The oracle checks sampled (layer,
sequence, head) triples: sequences and heads are independent in these
kernels, so the oracle only needs that sequence's rows projected onto that
head's Q/K/V columns.  Top-k selection is checked exactly on the GPU's own
scores for all 32 sequences.  The cache-phase row set is a seeded draw (it
must not come from either side's top-k); per-step isolation loads the
oracle's step-0 K/V of each sampled head, rounded to bf16, into the GPU cache
before step 1.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, TOL, close, log
from test_gpu_parity import head_sum

pytestmark = pytest.mark.gpu

SAMPLES = [(0, 3, 0), (0, 20, 13), (17, 3, 31), (17, 29, 5), (31, 11, 22), (31, 20, 7)]   # (layer, seq, head)
P = W.PAGE


def _bf16_to_f64(t):
    import torch
    return W.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _oracle_head(x_b, w_head, pos, logical, kv, mass_count, k_prev, v_prev, D, base):
    """One sequence, one head: project, rotate, write into that head's cache
    column block (logical order), attend over kv keys, formula (2) term."""
    table = O.build_block_table([(kv + P - 1) // P], list(range((kv + P - 1) // P)),
                                (kv + P - 1) // P, (kv + P - 1) // P)
    out = O.layer_step(x_b, w_head, pos, logical, [0, len(logical)], [kv], [mass_count], k_prev, v_prev,
                       table, 1, D, base, P)
    return out


@pytest.fixture(scope="module")
def b32(gpu):
    import torch
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = W.make_workload("llada_b32")
    run = FlashCacheRunner(wl, device=gpu)
    log(f"[gpu] llada_b32: {run.layers} layers, caches {2 * run.layers * run.k_cache[0].numel() * 2 / 2**30:.1f} GiB")
    return wl, run


def _slots_of(run, wl, b, positions):
    table = run.page_table.cpu().numpy().reshape(wl.n_seq, wl.max_pages)
    positions = np.asarray(positions)
    return table[b, positions // P] * P + positions % P


def test_llada_b32_full_refresh_then_cache_phase(b32, gpu):
    import torch
    wl, run = b32
    sh = wl.shape
    H, D, n = sh.n_heads, sh.head_dim, sh.n_heads * sh.head_dim
    layers = sorted({l for l, _, _ in SAMPLES})
    atol, rtol = TOL["bf16"]
    ma, mr = MASS_TOL["bf16"]
    oracle_cache = {}

    for step in (0, 1):
        rows = W.full_refresh_rows(wl) if step == 0 else W.config_step_rows(wl, W.seeded_tracked(wl, 1))
        st = run.upload_step(rows)
        run.map_slots(st)
        run.mass.zero_()
        log(f"[gpu] llada_b32 step {step}: {rows.n_rows} rows per layer")
        for l in range(run.layers):
            w = W.device_weights(wl, l, gpu)
            x = W.device_activations(wl, rows, step, l, gpu)
            if step == 1 and l in layers:
                # isolation: the sampled heads start from the oracle's step-0 cache (bf16)
                for (ls, b, h) in SAMPLES:
                    if ls != l:
                        continue
                    kv = int(rows.kv_len[b])
                    sl = torch.from_numpy(_slots_of(run, wl, b, np.arange(kv)).astype(np.int64)).to(gpu)
                    kc, vc = oracle_cache[(l, b, h)]
                    for cache, src in ((run.k_cache[l], kc), (run.v_cache[l], vc)):
                        vals = torch.from_numpy(W.round_bf16_bits(src.astype(np.float32)).view(np.int16)).to(gpu)
                        cache.view(torch.int16)[sl, h * D:(h + 1) * D] = vals
            before = run.mass.clone() if l in layers else None
            run.cache_update(st, x, w, l)
            run.attention(st, l)
            if l not in layers:
                continue
            torch.cuda.synchronize()
            term = (run.mass - before).cpu().numpy()
            wq = W.bf16_bits_to_f64(w.view(torch.int16).cpu().numpy().view(np.uint16))
            for (ls, b, h) in SAMPLES:
                if ls != l:
                    continue
                r0, r1 = int(rows.cu_q[b]), int(rows.cu_q[b + 1])
                kv = int(rows.kv_len[b])
                x_b = _bf16_to_f64(x[r0:r1])
                w_head = np.concatenate([wq[p * n + h * D:p * n + (h + 1) * D] for p in range(3)])
                if step == 0:
                    k_prev = np.zeros((kv, D)); v_prev = np.zeros((kv, D))
                else:
                    k_prev, v_prev = oracle_cache[(l, b, h)]
                    k_prev = W.bf16_bits_to_f64(W.round_bf16_bits(k_prev.astype(np.float32)))
                    v_prev = W.bf16_bits_to_f64(W.round_bf16_bits(v_prev.astype(np.float32)))
                out = _oracle_head(x_b, w_head, rows.pos[r0:r1], rows.logical[r0:r1], kv,
                                   int(rows.mass_count[b]), k_prev, v_prev, D, sh.rope_base)
                if step == 0:
                    oracle_cache[(l, b, h)] = (out["k_cache"][:kv], out["v_cache"][:kv])
                cols = slice(h * D, (h + 1) * D)
                slots = _slots_of(run, wl, b, rows.logical[r0:r1])
                tag = f"llada_b32 step{step} layer{l} seq{b} head{h}"
                close(_bf16_to_f64(st.q[r0:r1, cols]), out["q"], atol, rtol, tag + " q")
                kc = _bf16_to_f64(run.k_cache[l][torch.from_numpy(slots.astype(np.int64)).to(gpu)][:, cols])
                vc = _bf16_to_f64(run.v_cache[l][torch.from_numpy(slots.astype(np.int64)).to(gpu)][:, cols])
                close(kc, out["k"], atol, rtol, tag + " K rows")
                close(vc, out["v"], atol, rtol, tag + " V rows")
                close(_bf16_to_f64(st.o[r0:r1, cols]), out["o"], atol, rtol, tag + " o")
                # the GPU's per-head term carries 1/(H |M|); the one-head oracle carries 1/|M|
                info = close(term[b, h, :kv], out["mass"][0, :kv] / H, ma, mr, tag + " mass")
                log(f"   {tag}: mass max_abs {info['max_abs']:.2e}")
        torch.cuda.synchronize()
        score = head_sum(run.mass.cpu().numpy())
        run.topk(clear_mass=True)
        idx = run.top_idx.cpu().numpy()
        cnt = run.top_cnt.cpu().numpy()
        elig = wl.eligible().astype(bool)
        o_idx, _, o_cnt = O.topk(score.astype(np.float64), elig, sh.top_k)
        assert np.array_equal(idx, o_idx) and np.array_equal(cnt, o_cnt)
        log(f"[gpu] llada_b32 step {step}: top-k selection identical for {wl.n_seq} sequences")
