"""The one-call paged projection with many sequences, on every kernel family.

The paged entry point forms each row's cache slot from its sequence's
block-table row and its logical position ([FD] 方法步骤详情 step 1 and
核心方法: the flat cache is addressed through a per-sequence block table, and
K/V are written straight into it).  The cache-phase and mid-size kernels stage
cu_q (up to 1025 entries) and the rows' positions in LDS and resolve the page
entries themselves; the GEMM shapes take the slots from a launch of their own.
The parity workloads have at most 32 sequences, so these cases run 300 and
1024 sequences (the most the entry point takes), with empty sequences, rows
whose logical position is negative or past the sequence's pages, block-table
entries that are unassigned (-1) or outside the pool: the slots written back
must equal the block-table rule bit for bit, and q and every cache row must be
bit-identical to the slot-given call with those slots (the same kernels with
the same arithmetic).
"""
import numpy as np
import pytest

from parity import log

pytestmark = pytest.mark.gpu

H, D, DM = 4, 128, 512
N_OUT = H * D
BASE = 5e5
PAGE = 16


def _layout(n_seq, rows, max_pages, rng):
    """cu_q, logical positions, the block table and the expected slots."""
    cuts = np.sort(rng.integers(0, rows + 1, size=n_seq - 1))
    cu = np.concatenate([[0], cuts, [rows]]).astype(np.int32)
    pool = n_seq * max_pages
    perm = rng.permutation(pool).astype(np.int64)
    pt = perm.reshape(n_seq, max_pages).copy()
    odd = rng.random(pt.shape)
    pt[odd < 0.05] = -1                                   # unassigned pages
    pt[(odd >= 0.05) & (odd < 0.08)] = pool + 3           # outside the pool
    logical = np.empty(rows, dtype=np.int64)
    for b in range(n_seq):
        n = cu[b + 1] - cu[b]
        if n:
            logical[cu[b]:cu[b + 1]] = rng.permutation(max_pages * PAGE)[:n]
    bad = rng.random(rows) < 0.06
    logical[bad] = rng.choice([-1, -100, max_pages * PAGE, max_pages * PAGE + 17], size=int(bad.sum()))
    want = np.full(rows, -1, dtype=np.int64)
    for b in range(n_seq):
        for r in range(cu[b], cu[b + 1]):
            l = logical[r]
            if l < 0 or l // PAGE >= max_pages:
                continue
            p = pt[b, l // PAGE]
            if 0 <= p < pool:
                want[r] = p * PAGE + l % PAGE
    return cu, logical.astype(np.int32), pt.astype(np.int32), want.astype(np.int32), pool


@pytest.mark.parametrize("n_seq,rows,kernel", [(300, 100, None), (1024, 120, None), (300, 450, "mid10x6"),
                                               (1024, 700, "mid6x6"), (1024, 900, "mid8x12"),
                                               (300, 1500, "g256x256")])
def test_paged_slots_with_many_sequences(n_seq, rows, kernel, gpu):
    import torch
    from io_aware_kv_amd import dllm
    log(f"[gpu] paged projection: {n_seq} sequences, {rows} rows, kernel {kernel or 'planner'}")
    rng = np.random.default_rng(9500 + n_seq + rows)
    max_pages = 4
    cu, logical, pt, want, pool = _layout(n_seq, rows, max_pages, rng)
    assert (want >= 0).sum() > rows // 2 and (want < 0).any()
    assert len(np.unique(want[want >= 0])) == int((want >= 0).sum())
    x = torch.from_numpy(rng.standard_normal((rows, DM)).astype(np.float32)).to(torch.bfloat16).to(gpu)
    w = torch.from_numpy((rng.standard_normal((3 * N_OUT, DM)) / np.sqrt(DM)).astype(np.float32)).to(
        torch.bfloat16).to(gpu)
    pos = torch.from_numpy(rng.integers(0, 4096, size=rows).astype(np.int32)).to(gpu)
    cache_rows = pool * PAGE
    t = lambda a: torch.from_numpy(a).to(gpu)
    out = {}
    dllm.set_tuning("qkv_kernel", kernel)
    try:
        for mode in ("paged", "slots"):
            q = torch.zeros(rows, N_OUT, dtype=torch.bfloat16, device=gpu)
            kc = torch.full((cache_rows, N_OUT), 3.0, dtype=torch.bfloat16, device=gpu)
            vc = kc.clone()
            slot = torch.full((rows,), -99, dtype=torch.int32, device=gpu)
            if mode == "paged":
                dllm.qkv_rope_cachewrite_paged(x, w, pos, t(cu), t(logical), t(pt.reshape(-1)), max_pages, slot,
                                               q, kc, vc, H, D, BASE)
            else:
                slot.copy_(t(want))
                dllm.qkv_rope_cachewrite(x, w, pos, slot, q, kc, vc, H, D, BASE)
            torch.cuda.synchronize()
            out[mode] = (slot.cpu().numpy(), q.view(torch.int16).cpu().numpy(),
                         kc.view(torch.int16).cpu().numpy(), vc.view(torch.int16).cpu().numpy())
    finally:
        dllm.set_tuning("qkv_kernel", None)
    assert np.array_equal(out["paged"][0], want), "slots formed from the block table"
    for i, name in ((1, "q"), (2, "K cache"), (3, "V cache")):
        assert np.array_equal(out["paged"][i], out["slots"][i]), f"{name}: paged call differs from the slot-given call"
    untouched = np.setdiff1d(np.arange(cache_rows), want[want >= 0])
    assert np.all(out["paged"][2][untouched] == out["paged"][2][untouched[0]][0])
    log(f"  {int((want >= 0).sum())} rows with a slot, {int((want < 0).sum())} without; bit-identical")
