"""The rotary embedding at large positions on every projection path.

The rotate-half rotation turns column pair (i, i + D/2) of q and k by the
angle pos * theta_i with theta_i = base^(-2i/D) ([FD] 研究动机 and 核心方法
name RoPE as the projection's second fused stage).  The kernels form the
angle in fp64, reduce it to at most half a turn and take the hardware sin/cos
of the remainder, so the rotation must stay accurate however large the
position: the workloads' positions stay below 4096, so these cases draw
positions over the whole int32 range (0, 1, 2^16, 2^20 + 7, 2^24 - 1,
2^30 + 123, 2^31 - 1 and random ones), for the weight-streaming kernel (at
most 128 rows), the mid-size streaming kernel (three shapes), the GEMM in two
tile shapes, the LDS-tiled kernel and the
fp32 kernel, and compare q and the K/V rows written to their (shuffled) cache
slots with the oracle's projection and rotation of the same inputs.  Cache
rows no slot names must stay untouched.  A contraction of 64 (two 32-deep
stages, fewer than the GEMM's ring holds) runs the GEMM's ring with every
refill past the last stage.
"""
import numpy as np
import pytest

import oracle as O
from parity import TOL, close, log

pytestmark = pytest.mark.gpu

H, D = 4, 128
N_OUT = H * D
BASE = 5e5
SPECIAL = (0, 1, 1 << 16, (1 << 20) + 7, (1 << 24) - 1, (1 << 30) + 123, (1 << 31) - 1)


@pytest.mark.parametrize("rows,kernel,dt,DM", [(100, None, "bf16", 512), (300, "gemm", "bf16", 512),
                                               (300, "g64x256", "bf16", 512), (300, "tiled", "bf16", 512),
                                               (77, None, "f32", 512), (300, "gemm", "bf16", 64),
                                               (300, "g128x256o2", "bf16", 64), (300, "mid10x6", "bf16", 512),
                                               (300, "mid4x12", "bf16", 64), (150, "mid6x6", "bf16", 512)])
def test_rope_at_large_positions(rows, kernel, dt, DM, gpu):
    import torch
    from io_aware_kv_amd import dllm
    log(f"[gpu] rotation at large positions: {rows} rows, d_model {DM}, {dt}, kernel {kernel or 'planner'}")
    rng = np.random.default_rng(9100 + rows)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((rows, DM)).astype(np.float32)).to(tdt).to(gpu)
    w = torch.from_numpy((rng.standard_normal((3 * N_OUT, DM)) / np.sqrt(DM)).astype(np.float32)).to(tdt).to(gpu)
    pos = rng.integers(0, (1 << 31) - 1, size=rows, dtype=np.int64)
    pos[:len(SPECIAL)] = SPECIAL
    pos = pos.astype(np.int32)
    cache_rows = rows + 37
    slot = rng.permutation(cache_rows)[:rows].astype(np.int32)
    q = torch.empty(rows, N_OUT, dtype=tdt, device=gpu)
    kc = torch.zeros(cache_rows, N_OUT, dtype=tdt, device=gpu)
    vc = torch.zeros(cache_rows, N_OUT, dtype=tdt, device=gpu)
    code = dllm.BF16 if dt == "bf16" else dllm.F32
    ws = torch.zeros(max(dllm.qkv_rope_cachewrite_workspace(code, rows, DM, H, D), 256), dtype=torch.uint8,
                     device=gpu)
    dllm.set_tuning("qkv_kernel", kernel)
    try:
        dllm.qkv_rope_cachewrite(x, w, torch.from_numpy(pos).to(gpu), torch.from_numpy(slot).to(gpu), q, kc, vc,
                                 H, D, BASE, ws)
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
    info = close(g(q), qo, *TOL[dt], f"q at large positions ({dt}, {kernel})")
    close(kcn[slot], ko, *TOL[dt], f"K rows at large positions ({dt}, {kernel})")
    close(vcn[slot], vo, *TOL[dt], f"V rows ({dt}, {kernel})")
    rest = np.setdiff1d(np.arange(cache_rows), slot)
    assert not kcn[rest].any() and not vcn[rest].any(), "a cache row no slot names was written"
    log(f"   q max_abs {info['max_abs']:.3e} (max/rms {info['max_over_rms']:.2e})")
