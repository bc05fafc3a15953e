"""bf16 projection with 64-wide heads on every kernel that takes them.

Rotate-half RoPE pairs columns (i, i + D/2) of each head ([FD] 研究动机 and
核心方法 name RoPE as the projection's fused second stage); with D = 64 a
head holds 32 pairs, so the weight-streaming kernels' 8-pair output pieces
and their pair groups must map onto heads of half the usual width.  The
workloads all use D = 128, so these cases run H = 8 heads of 64 (n = 512)
through the cache-phase streaming kernel (100 rows), the mid-size kernel in
two shapes and the LDS-tiled kernel (300 rows), and compare q and the K/V
rows written to shuffled cache slots with the oracle's projection and
rotation; cache rows no slot names stay untouched.
"""
import numpy as np
import pytest

import oracle as O
from parity import TOL, close, log

pytestmark = pytest.mark.gpu

H, D, DM = 8, 64, 512
N_OUT = H * D
BASE = 1e4


@pytest.mark.parametrize("rows,kernel", [(100, None), (300, "mid10x6"), (300, "mid4x12"), (300, "tiled"),
                                         (300, None)])
def test_head_dim_64(rows, kernel, gpu):
    import torch
    from io_aware_kv_amd import dllm
    log(f"[gpu] head_dim 64: {rows} rows, kernel {kernel or 'planner'}")
    rng = np.random.default_rng(9700 + rows)
    x = torch.from_numpy(rng.standard_normal((rows, DM)).astype(np.float32)).to(torch.bfloat16).to(gpu)
    w = torch.from_numpy((rng.standard_normal((3 * N_OUT, DM)) / np.sqrt(DM)).astype(np.float32)).to(
        torch.bfloat16).to(gpu)
    pos = rng.integers(0, 4096, size=rows).astype(np.int32)
    cache_rows = rows + 29
    slot = rng.permutation(cache_rows)[:rows].astype(np.int32)
    q = torch.empty(rows, N_OUT, dtype=torch.bfloat16, device=gpu)
    kc = torch.full((cache_rows, N_OUT), 5.0, dtype=torch.bfloat16, device=gpu)
    vc = kc.clone()
    dllm.set_tuning("qkv_kernel", kernel)
    try:
        dllm.qkv_rope_cachewrite(x, w, torch.from_numpy(pos).to(gpu), torch.from_numpy(slot).to(gpu), q, kc, vc,
                                 H, D, BASE)
        torch.cuda.synchronize()
    finally:
        dllm.set_tuning("qkv_kernel", None)
    x64 = x.to(torch.float64).cpu().numpy()
    w64 = w.to(torch.float64).cpu().numpy()
    qo, ko, vo = O.project(x64, w64, N_OUT)
    qo = O.rope(qo.reshape(rows, H, D), pos, BASE).reshape(rows, N_OUT)
    ko = O.rope(ko.reshape(rows, H, D), pos, BASE).reshape(rows, N_OUT)
    g = lambda t: t.to(torch.float64).cpu().numpy()
    kcn, vcn = g(kc), g(vc)
    atol, rtol = TOL["bf16"]
    infos = [close(g(q), qo, atol, rtol, "q"), close(kcn[slot], ko, atol, rtol, "K rows"),
             close(vcn[slot], vo, atol, rtol, "V rows")]
    untouched = np.setdiff1d(np.arange(cache_rows), slot)
    assert np.all(kcn[untouched] == 5.0) and np.all(vcn[untouched] == 5.0)
    for i in infos:
        log(f"   {i['what']}: max_abs={i['max_abs']:.3e} max/rms={i['max_over_rms']:.3e}")
