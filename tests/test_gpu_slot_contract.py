"""The projection's slot contract on every kernel: a row whose slot is -1,
another negative value or at least cache_rows writes no cache row, every other
row writes exactly its own slot, and q is written for every row.

The pages' cache write scatters each refreshed token's K/V rows to its flat
slot ([FD] 方法步骤详情 step 1 and 核心方法); rows without a slot (view rows of
the verify layout, rows whose page is missing) must not touch the cache.  The
caches start filled with a sentinel; rows with a valid slot are compared with
the oracle's projection and rotation, every other cache row must still hold
the sentinel, on the weight-streaming kernel (at most 128 rows), the mid-size
streaming kernel (three shapes), the GEMM (two
tile shapes), the LDS-tiled kernel, the fp32 kernel and, for the one-byte E4M3
caches, the streaming and GEMM kernels (a sentinel byte; written rows compared
as decoded codes).
"""
import numpy as np
import pytest

import oracle as O
from parity import TOL, close, log

pytestmark = pytest.mark.gpu

H, D, DM = 4, 128, 512
N_OUT = H * D
BASE = 5e5
SENTINEL = 7.0


def _slots(rows, cache_rows, rng):
    """Distinct valid slots for about 60% of the rows; the rest -1, another
    negative value, cache_rows, cache_rows + 5 or INT32_MAX."""
    slot = rng.permutation(cache_rows)[:rows].astype(np.int64)
    bad = rng.random(rows) < 0.4
    choices = np.array([-1, -7, -(1 << 31), cache_rows, cache_rows + 5, (1 << 31) - 1], dtype=np.int64)
    slot[bad] = rng.choice(choices, size=int(bad.sum()))
    slot[0], slot[1], slot[2] = -1, cache_rows, (1 << 31) - 1      # every kind appears
    return slot.astype(np.int32)


@pytest.mark.parametrize("rows,kernel,dt", [(100, None, "bf16"), (300, "gemm", "bf16"), (300, "g64x256", "bf16"),
                                            (300, "tiled", "bf16"), (77, None, "f32"), (100, None, "e4m3"),
                                            (300, "gemm", "e4m3"), (300, "mid10x6", "bf16"), (300, "mid8x12", "e4m3"),
                                            (200, "mid6x6", "bf16")])
def test_slots_outside_the_cache_write_nothing(rows, kernel, dt, gpu):
    import torch
    from io_aware_kv_amd import dllm
    log(f"[gpu] slot contract: {rows} rows, {dt}, kernel {kernel or 'planner'}")
    rng = np.random.default_rng(9300 + rows + (7 if dt == "e4m3" else 0))
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = torch.from_numpy(rng.standard_normal((rows, DM)).astype(np.float32)).to(tdt).to(gpu)
    w = torch.from_numpy((rng.standard_normal((3 * N_OUT, DM)) / np.sqrt(DM)).astype(np.float32)).to(tdt).to(gpu)
    pos = rng.integers(0, 4096, size=rows).astype(np.int32)
    cache_rows = rows + 41
    slot = _slots(rows, cache_rows, rng)
    q = torch.empty(rows, N_OUT, dtype=tdt, device=gpu)
    if dt == "e4m3":
        kc = torch.full((cache_rows, N_OUT), 0x5A, dtype=torch.uint8, device=gpu)
        code = dllm.BF16_E4M3KV
    else:
        kc = torch.full((cache_rows, N_OUT), SENTINEL, dtype=tdt, device=gpu)
        code = dllm.BF16 if dt == "bf16" else dllm.F32
    vc = kc.clone()
    ws = torch.zeros(max(dllm.qkv_rope_cachewrite_workspace(code, rows, DM, H, D), 256), dtype=torch.uint8,
                     device=gpu)
    dllm.set_tuning("qkv_kernel", kernel)
    try:
        dllm.qkv_rope_cachewrite(x, w, torch.from_numpy(pos).to(gpu), torch.from_numpy(slot).to(gpu), q, kc, vc,
                                 H, D, BASE, ws)
        torch.cuda.synchronize()
    finally:
        dllm.set_tuning("qkv_kernel", None)

    valid = (slot >= 0) & (slot < cache_rows)
    assert 0 < valid.sum() < rows
    untouched = np.setdiff1d(np.arange(cache_rows), slot[valid])
    kcn, vcn = kc.cpu().numpy() if dt == "e4m3" else kc.to(torch.float64).cpu().numpy(), \
        vc.cpu().numpy() if dt == "e4m3" else vc.to(torch.float64).cpu().numpy()
    fill = 0x5A if dt == "e4m3" else SENTINEL
    assert np.all(kcn[untouched] == fill) and np.all(vcn[untouched] == fill), \
        "a cache row no valid slot names was written"

    x64 = x.to(torch.float64).cpu().numpy()
    w64 = w.to(torch.float64).cpu().numpy()
    qo, ko, vo = O.project(x64, w64, N_OUT)
    qo = O.rope(qo.reshape(rows, H, D), pos, BASE).reshape(rows, N_OUT)
    ko = O.rope(ko.reshape(rows, H, D), pos, BASE).reshape(rows, N_OUT)
    tol = TOL["f32" if dt == "f32" else "bf16"]
    close(q.to(torch.float64).cpu().numpy(), qo, *tol, f"q ({dt}, {kernel})")
    if dt == "e4m3":
        # written rows hold the E4M3 codes of the rotated k and of v: 3 mantissa
        # bits round to within 2^-4 relative (plus the bf16 rounding before it);
        # the absolute term covers the subnormal spacing 2^-9
        kd, vd = O.e4m3_decode(kcn[slot[valid]]), O.e4m3_decode(vcn[slot[valid]])
        close(kd, ko[valid], 2e-2, 7e-2, f"K codes ({kernel})")
        close(vd, vo[valid], 2e-2, 7e-2, f"V codes ({kernel})")
    else:
        close(kcn[slot[valid]], ko[valid], *tol, f"K rows ({dt}, {kernel})")
        close(vcn[slot[valid]], vo[valid], *tol, f"V rows ({dt}, {kernel})")
    log(f"   {int(valid.sum())} rows written, {rows - int(valid.sum())} without a slot, "
        f"{len(untouched)} cache rows untouched")
