"""Block-granular caching steps on the GPU against the oracle: DualCache
(only the current block is queried and written; the prefix and the masked
suffix come from the cache) and the active window of PrefixCache / FreeCache
(the current block and every later block are queried and written; the prompt
and the finished blocks are frozen).  Same kernels and entry points as the
Flash-Cache step; no formula-(2) rows.

[FST] Fast-dLLM article (senqingzn.com), block-wise KV cache section;
[FDLM] FlashDLM notes (papernotes.org), FreeCache.

Each case starts from the oracle's step-0 cache (the full refresh), rounded to
the path dtype, and compares q, the written K/V rows and o with the same
tolerances as the Flash-Cache step; cache rows the step must not write are
compared bit for bit.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import TOL, close, device_bits, device_values, log

pytestmark = pytest.mark.gpu

_ORACLE = {}


def _oracle(c, mode):
    key = (c.wl.name, mode)
    if key not in _ORACLE:
        wl, sh = c.wl, c.wl.shape
        rows = W.block_cache_rows(wl, mode)
        x_raw = W.activations(wl, rows, 2)
        out = O.layer_step(W.as_f64(wl, x_raw), W.as_f64(wl, c.w_raw), rows.pos, rows.logical, rows.cu_q,
                           rows.kv_len, rows.mass_count, c.k1_in, c.v1_in, c.table, sh.n_heads, sh.head_dim,
                           sh.rope_base, W.PAGE)
        _ORACLE[key] = (rows, x_raw, out)
    return _ORACLE[key]


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16", "llada_b1", "mixed_b8"])
@pytest.mark.parametrize("mode", W.BLOCK_CACHE_MODES)
def test_block_cache_step_parity(name, mode, gpu):
    import torch
    import test_gpu_parity as T
    from io_aware_kv_amd.runner import FlashCacheRunner
    c = T.case(name)
    rows, x_raw, out = _oracle(c, mode)
    print(f"[gpu] block-cache {mode} {name}: R={rows.n_rows}", flush=True)
    run = FlashCacheRunner(c.wl, device=gpu, layers=1)
    run.k_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.k1_in)))
    run.v_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.v1_in)))
    k_before, v_before = device_bits(run.k_cache[0]), device_bits(run.v_cache[0])
    st = run.upload_step(rows)
    run.layer_step(st, run.to_device_array(x_raw), run.to_device_array(c.w_raw), 0, with_mass=False)
    torch.cuda.synchronize()
    assert np.array_equal(st.slot.cpu().numpy(), out["slots"].astype(np.int32))
    k_bits, v_bits = device_bits(run.k_cache[0]), device_bits(run.v_cache[0])
    written = np.zeros(k_bits.shape[0], dtype=bool)
    written[out["slots"]] = True
    assert np.array_equal(k_bits[~written], k_before[~written]), "frozen K rows changed"
    assert np.array_equal(v_bits[~written], v_before[~written]), "frozen V rows changed"
    atol, rtol = TOL[c.kind]
    infos = [close(device_values(st.q), out["q"], atol, rtol, "q_out"),
             close(device_values(run.k_cache[0])[out["slots"]], out["k"], atol, rtol, "K rows"),
             close(device_values(run.v_cache[0])[out["slots"]], out["v"], atol, rtol, "V rows"),
             close(device_values(st.o), out["o"], atol, rtol, "o")]
    assert not run.mass.cpu().numpy().any(), "a step without formula-(2) rows wrote scores"
    for i in infos:
        log(f"   {name} {mode} {i['what']}: max_abs={i['max_abs']:.3e} max/rms={i['max_over_rms']:.3e} "
            f"beyond 30 bf16 ulps: {i['n_over_30ulp_bf16']}")
