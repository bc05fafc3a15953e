"""Shared machinery of the GPU parity tests: run a workload's step 0 (full
refresh) and its own step (step 1) through the HIP path and through the
oracle on identical inputs, with per-step isolation (the GPU cache is loaded
with the oracle's post-step-0 cache, rounded to the path dtype, before step 1).
"""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle as O
from io_aware_kv_amd import workloads as W

# Tolerances.  bf16: |g - o| <= 2e-2 + 1e-2 |o| on q, written K/V and o;
# fp32: 1e-4 + 1e-4 |o|.  Formula-(2) mass: the GPU rounds q and k to bf16
# (relative 2^-9 each) before the scores, so a score moves by up to ~2^-8 of
# sum_d |q_d k_d| / sqrt(D); averaged over rows and heads the per-key mass
# moves well under 1%: gate at 1e-2 relative + 1e-7 absolute (bf16) and
# 1e-4 relative + 1e-8 absolute (fp32).
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
MASS_TOL = {"bf16": (1e-7, 1e-2), "f32": (1e-8, 1e-4)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def measure(got: np.ndarray, want: np.ndarray, atol: float, rtol: float, what: str) -> dict:
    """The error statistics of close() without the assertion: max error,
    max error / rms(oracle), elements beyond atol + rtol |want|, and the
    largest ratio err / (atol + rtol |want|) (above 1 = outside the gate)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    return {"what": what, "max_abs": float(err.max()) if err.size else 0.0,
            "max_over_rms": float(err.max() / rms) if err.size and rms else 0.0,
            "n_bad": int((err > lim).sum()), "worst_ratio": float((err / lim).max()) if err.size else 0.0}


def close(got: np.ndarray, want: np.ndarray, atol: float, rtol: float, what: str) -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    # diagnostic beside the gate: elements further than 30 bf16 spacings from
    # the oracle (the spacing of a bf16 value v is 2^(floor(log2 |v|) - 7);
    # zero and subnormal references take the smallest normal spacing)
    ex = np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126)))
    ulp = np.exp2(ex - 7.0)
    info = {"what": what, "max_abs": float(err.max()) if err.size else 0.0,
            "max_over_rms": float(err.max() / rms) if err.size and rms else 0.0,
            "n_over_30ulp_bf16": int((err > 30.0 * ulp).sum()),
            "n_bad": int(bad.sum())}
    assert not bad.any(), f"{what}: {info}, first bad at {np.argwhere(bad)[:5].tolist()}"
    return info


def bf16_round(a: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f64(W.round_bf16_bits(np.asarray(a, dtype=np.float32)))


class Case:
    """Inputs and oracle results of one workload (steps 0 and 1)."""

    def __init__(self, name: str, heavy: bool = False):
        t0 = time.time()
        self.wl = wl = W.make_workload(name, heavy=heavy)
        sh = wl.shape
        self.kind = sh.dtype
        self.n_out = sh.n_heads * sh.head_dim
        self.table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
        self.w_raw = W.weights(wl, 0)
        w64 = W.as_f64(wl, self.w_raw)
        rows_cache = wl.pool_pages * W.PAGE
        self.k_init_raw = W.sentinel_cache(wl, rows_cache, self.n_out, 1)
        self.v_init_raw = W.sentinel_cache(wl, rows_cache, self.n_out, 2)
        kc = W.as_f64(wl, self.k_init_raw)
        vc = W.as_f64(wl, self.v_init_raw)
        # step 0: full refresh
        self.rows0 = W.full_refresh_rows(wl)
        self.x0_raw = W.activations(wl, self.rows0, 0)
        self.out0 = O.layer_step(W.as_f64(wl, self.x0_raw), w64, self.rows0.pos, self.rows0.logical,
                                 self.rows0.cu_q, self.rows0.kv_len, self.rows0.mass_count, kc, vc,
                                 self.table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
        self.top0 = O.topk(self.out0["mass"], wl.eligible().astype(bool), sh.top_k)
        # the same step with the path's bf16 stores of q, K and V modelled (the
        # attention reads the stored values): the reference for o where the
        # planted rows' large scores magnify the storage rounding
        self.out0_store = None
        if heavy and self.kind == "bf16":
            self.out0_store = O.layer_step(W.as_f64(wl, self.x0_raw), w64, self.rows0.pos, self.rows0.logical,
                                           self.rows0.cu_q, self.rows0.kv_len, self.rows0.mass_count, kc, vc,
                                           self.table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE,
                                           store="bf16")
        # step 1 starts from the step-0 cache rounded to the path dtype
        rnd = bf16_round if self.kind == "bf16" else (lambda a: np.asarray(a, np.float32).astype(np.float64))
        self.k1_in = rnd(self.out0["k_cache"])
        self.v1_in = rnd(self.out0["v_cache"])
        tracked = [self.top0[0][b][self.top0[0][b] >= 0] for b in range(wl.n_seq)]
        self.rows1 = W.config_step_rows(wl, tracked)
        self.x1_raw = W.activations(wl, self.rows1, 1)
        self.out1 = O.layer_step(W.as_f64(wl, self.x1_raw), w64, self.rows1.pos, self.rows1.logical,
                                 self.rows1.cu_q, self.rows1.kv_len, self.rows1.mass_count, self.k1_in,
                                 self.v1_in, self.table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE,
                                 visible=self.rows1.visible)
        self.top1 = O.topk(self.out1["mass"], wl.eligible().astype(bool), sh.top_k)
        log(f"[parity] oracle for {name}{' (heavy)' if heavy else ''} ready in {time.time() - t0:.1f}s "
            f"(R0={self.rows0.n_rows}, R1={self.rows1.n_rows})")

    def to_cache_raw(self, a64: np.ndarray) -> np.ndarray:
        if self.kind == "bf16":
            return W.round_bf16_bits(a64.astype(np.float32))
        return a64.astype(np.float32)


def device_values(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> float64 numpy."""
    import torch
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy().astype(np.float64)


def device_bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def check_topk(case: Case, mass_gpu: np.ndarray, idx: np.ndarray, val: np.ndarray, cnt: np.ndarray,
               mass_oracle: np.ndarray, exact_set: bool = False) -> None:
    """(1) The selection itself, decided on the GPU's own fp32 scores, equals
    the oracle's top-k on those scores, bit for bit.  (2) Against the oracle's
    scores: positions clearly above the k-th oracle score are selected and
    positions clearly below are not; 'clearly' is outside a window of
    max(1e-3 * a_k, mass tolerance) around the k-th score (or exact sets for
    well-separated planted scores)."""
    wl = case.wl
    k = wl.shape.top_k
    elig = wl.eligible().astype(bool)
    o_idx, o_val, o_cnt = O.topk(mass_gpu.astype(np.float64), elig, k)
    assert np.array_equal(idx, o_idx), (idx, o_idx)
    assert np.array_equal(cnt, o_cnt)
    for b in range(wl.n_seq):
        n = int(cnt[b])
        assert np.array_equal(val[b, :n], mass_gpu[b, idx[b, :n]].astype(np.float32))
    r_idx, _, r_cnt = O.topk(mass_oracle, elig, k)
    assert np.array_equal(cnt, r_cnt)
    atol, rtol = MASS_TOL[case.kind]
    for b in range(wl.n_seq):
        n = int(r_cnt[b])
        if n == 0:
            continue
        sel_g = set(idx[b, :n].tolist())
        if exact_set:
            assert sel_g == set(r_idx[b, :n].tolist()), b
            continue
        ak = mass_oracle[b, r_idx[b, n - 1]]
        win = max(1e-3 * ak, atol + rtol * ak)
        cand = np.flatnonzero(elig[b])
        for i in cand:
            a = mass_oracle[b, i]
            if a > ak + win:
                assert i in sel_g, (b, i, a, ak)
            elif a < ak - win:
                assert i not in sel_g, (b, i, a, ak)
