"""The low-bit cache on the GPU: bf16 layers whose K and V caches hold E4M3
codes (DLLM_BF16_E4M3KV), against the oracle's layer step in the same format
(oracle/lowbit.py; [FD] paper summary page, 未来方向 item (3)).

Each workload runs its full refresh (step 0) from a cache of seeded codes and
then its own step (step 1) from the oracle's step-0 cache, through the same
entry points as the bf16 path: the paged projection (rotate, encode, write),
the scheduled attention (decode while staging, formula (2)) and the top-k.

Bars: written cache rows decode to the oracle's stored values (the kernel
rounds its fp32 value, the oracle its fp64 value, so a value at a rounding
tie may land one code apart: at most 1 in 1000 entries, each within one step
of the format); rows the step must not write keep their codes bit for bit;
q, o and the score with the bf16 tolerances; the top-k by the usual rule.
"""
import types

import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, TOL, check_topk, close, device_values, log

pytestmark = pytest.mark.gpu

_CASES = {}


def _seeded_codes(rows, width, salt):
    r = np.random.default_rng(9000 + salt)
    mag = r.integers(0, 0x7F, size=(rows, width))
    return (mag | (r.integers(0, 2, size=(rows, width)) << 7)).astype(np.uint8)


class LowbitCase:
    def __init__(self, name):
        self.wl = wl = W.make_workload(name)
        sh = wl.shape
        self.table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
        self.w_raw = W.weights(wl, 0)
        w64 = W.as_f64(wl, self.w_raw)
        n = sh.n_heads * sh.head_dim
        rows_cache = wl.pool_pages * W.PAGE
        self.k0_codes = _seeded_codes(rows_cache, n, 1)
        self.v0_codes = _seeded_codes(rows_cache, n, 2)
        self.rows = [W.full_refresh_rows(wl), None]
        self.x_raw = [W.activations(wl, self.rows[0], 0), None]
        args = dict(n_heads=sh.n_heads, head_dim=sh.head_dim, rope_base=sh.rope_base, page_size=W.PAGE,
                    kv_format="e4m3")
        r0 = self.rows[0]
        self.out = [O.layer_step(W.as_f64(wl, self.x_raw[0]), w64, r0.pos, r0.logical, r0.cu_q, r0.kv_len,
                                 r0.mass_count, O.e4m3_decode(self.k0_codes), O.e4m3_decode(self.v0_codes),
                                 self.table, **args), None]
        top0 = O.topk(self.out[0]["mass"], wl.eligible().astype(bool), sh.top_k)
        self.rows[1] = W.config_step_rows(wl, [top0[0][b][top0[0][b] >= 0] for b in range(wl.n_seq)])
        r1 = self.rows[1]
        self.x_raw[1] = W.activations(wl, r1, 1)
        self.k1_codes = O.e4m3_encode(self.out[0]["k_cache"])
        self.v1_codes = O.e4m3_encode(self.out[0]["v_cache"])
        self.out[1] = O.layer_step(W.as_f64(wl, self.x_raw[1]), w64, r1.pos, r1.logical, r1.cu_q, r1.kv_len,
                                   r1.mass_count, self.out[0]["k_cache"], self.out[0]["v_cache"], self.table,
                                   visible=r1.visible, **args)


def _case(name):
    if name not in _CASES:
        _CASES[name] = LowbitCase(name)
    return _CASES[name]


def _codes_close(got_codes, want_values, what):
    got = O.e4m3_decode(got_codes)
    same = (got == want_values) | ((got == 0) & (want_values == 0))
    frac = 1.0 - same.mean()
    step = np.abs(got - want_values) <= 2.0 ** -3 * np.abs(want_values) + 2.0 ** -9
    assert step.all(), f"{what}: {np.count_nonzero(~step)} entries more than one step apart"
    assert frac <= 1e-3, f"{what}: {frac:.2e} of the entries differ"
    return frac


@pytest.mark.parametrize("name", ["tiny_bf16", "llada_b1", "mixed_b8", "verify_b4"])
@pytest.mark.parametrize("step", [0, 1])
def test_lowbit_cache_step(name, step, gpu):
    import torch
    import test_gpu_parity as T
    from io_aware_kv_amd.runner import FlashCacheRunner
    c = _case(name)
    wl = c.wl
    rows, out = c.rows[step], c.out[step]
    print(f"[gpu] e4m3 cache {name} step {step}: R={rows.n_rows}", flush=True)
    run = FlashCacheRunner(wl, device=gpu, layers=1, kv_format="e4m3")
    k_init, v_init = (c.k0_codes, c.v0_codes) if step == 0 else (c.k1_codes, c.v1_codes)
    run.k_cache[0].copy_(torch.from_numpy(k_init).to(gpu))
    run.v_cache[0].copy_(torch.from_numpy(v_init).to(gpu))
    st = run.upload_step(rows)
    run.layer_step(st, run.to_device_array(c.x_raw[step]), run.to_device_array(c.w_raw), 0)
    torch.cuda.synchronize()
    mass = T.head_sum(run.mass.cpu().numpy())
    run.topk(clear_mass=True)
    torch.cuda.synchronize()
    k_codes, v_codes = run.k_cache[0].cpu().numpy(), run.v_cache[0].cpu().numpy()
    slots = out["slots"]
    assert np.array_equal(st.slot.cpu().numpy(), slots.astype(np.int32))
    written = np.zeros(k_codes.shape[0], dtype=bool)
    written[slots] = True
    assert np.array_equal(k_codes[~written], k_init[~written]), "unwritten K rows changed"
    assert np.array_equal(v_codes[~written], v_init[~written]), "unwritten V rows changed"
    fk = _codes_close(k_codes[slots], out["k"], f"{name} step{step} K rows")
    fv = _codes_close(v_codes[slots], out["v"], f"{name} step{step} V rows")
    atol, rtol = TOL["bf16"]
    infos = [close(device_values(st.q), out["q"], atol, rtol, "q_out"),
             close(device_values(st.o), out["o"], atol, rtol, "o"),
             close(mass, out["mass"], *MASS_TOL["bf16"], "mass")]
    log(f"   {name} step{step} e4m3: K/V codes differing {fk:.1e}/{fv:.1e}; " +
        "; ".join(f"{i['what']} max_abs={i['max_abs']:.2e}" for i in infos))
    case = types.SimpleNamespace(wl=wl, kind="bf16")
    check_topk(case, mass, run.top_idx.cpu().numpy(), run.top_val.cpu().numpy(), run.top_cnt.cpu().numpy(),
               out["mass"])
