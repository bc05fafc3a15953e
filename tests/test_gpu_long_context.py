"""Attention over long contexts and degenerate batches: sequences whose keys span many more key
tiles than the workloads' (4100 keys with a partial last tile, 8704 keys — the
most a score is formed for — and 16384, the bf16 kernel's page-table limit),
on a shuffled page pool, through both attention paths (key splits merged by
the second launch, and the single launch, whose items of more than 64 tiles
take their copy bases from LDS rather than registers and whose score pass
runs over many rounds of key tiles).  q and the caches are seeded N(0, 1)
bf16 values ([FD] 核心方法: block-table scheduled attention over the paged
cache; 方法步骤详情 step 4, formula (2) for the window rows).

o and the per-head score terms of three heads are compared with the oracle on
the same stored values (bf16 tolerances); the other heads run the same code.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, TOL, close, log

pytestmark = pytest.mark.gpu

H, D = 32, 128
HEADS = (0, 13, 31)


def _cols(t, heads):
    import torch
    idx = torch.cat([torch.arange(h * D, (h + 1) * D) for h in heads]).to(t.device)
    return t.index_select(1, idx).to(torch.float64).cpu().numpy()


@pytest.mark.parametrize("kv,rows,mass,splits,cap", [
    ((4100, 8704), (72, 200), (32, 32), None, None),
    ((4100, 8704), (72, 200), (32, 32), "1", None),
    ((16384,), (64,), None, None, None),
    ((16384,), (64,), None, "1", None),
    # degenerate batches: an inactive sequence (no rows, no keys), one not
    # refreshed this step (keys, no rows), a single key and row, a partial
    # key tile, two query tiles over a partial key tile
    ((0, 100, 1, 40, 200), (0, 0, 1, 17, 130), (0, 0, 1, 5, 32), None, None),
    ((0, 100, 1, 40, 200), (0, 0, 1, 17, 130), (0, 0, 1, 5, 32), "1", None),
    # a score narrower than the longest sequence: keys at or past n_cap are not
    # recorded (n_cap not a multiple of the 64-key tile)
    ((4100, 8704), (72, 200), (32, 32), None, 5000),
    ((4100, 8704), (72, 200), (32, 32), "1", 5000),
])
def test_long_context_attention(kv, rows, mass, splits, cap, gpu):
    import torch
    from io_aware_kv_amd import dllm
    log(f"[gpu] long-context attention kv={kv} rows={rows} score={mass is not None} splits={splits or 'auto'} "
        f"n_cap={cap or 'max kv'}")
    lc = W.long_context(kv, rows, mass if mass is not None else [0] * len(kv), seed=len(kv) * 10 + (1 if splits else 0))
    n_seq, n_out = len(kv), H * D
    q, kc, vc = W.long_context_tensors(lc, n_out, gpu)
    R = int(lc.rows.sum())
    cu = np.concatenate([[0], np.cumsum(lc.rows)]).astype(np.int32)
    table_dev = torch.empty(n_seq * lc.max_pages, dtype=torch.int32, device=gpu)
    dllm.build_block_table(lc.seq_pages, lc.pool_perm, lc.pool_pages, lc.max_pages, table_dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(gpu)
    cu_d, kv_d = i32(cu), i32(lc.kv)
    max_kv = int(lc.kv.max())
    with_mass = mass is not None
    n_cap = cap or max_kv
    max_mass = int(lc.mass_count.max()) if with_mass else 0
    assert R > 0
    o = torch.empty(R, n_out, dtype=torch.bfloat16, device=gpu)
    score = torch.zeros(n_seq, H, n_cap, dtype=torch.float32, device=gpu)
    dllm.set_tuning("attn_splits", splits)
    try:
        ws_b = dllm.sched_attention_workspace(dllm.BF16, n_seq, R, H, D, max_kv, n_cap, max_mass)
        ws = torch.zeros(max(ws_b, 256), dtype=torch.uint8, device=gpu)
        dllm.sched_attention(q, cu_d, kc, vc, table_dev, lc.max_pages, kv_d, o, ws, H, D, max_kv,
                             mass_count=i32(lc.mass_count) if with_mass else None, max_mass_rows=max_mass,
                             mass_accum=score if with_mass else None, n_cap=n_cap, mass_overwrite=True)
        torch.cuda.synchronize()
    finally:
        dllm.set_tuning("attn_splits", None)

    table = O.build_block_table(lc.seq_pages, lc.pool_perm, lc.pool_pages, lc.max_pages)
    o_want, probs = O.attention(_cols(q, HEADS), _cols(kc, HEADS), _cols(vc, HEADS), table, cu, lc.kv,
                                len(HEADS), D, W.PAGE)
    info = close(_cols(o, HEADS), o_want, *TOL["bf16"], "long-context o")
    log(f"   o of heads {HEADS}: max_abs={info['max_abs']:.3e}")
    if with_mass:
        got = score.cpu().numpy()
        for j, h in enumerate(HEADS):
            want = O.column_mass([pb[j:j + 1] for pb in probs], lc.mass_count, n_cap) / H
            for b in range(n_seq):
                k = min(int(lc.kv[b]), n_cap)
                if lc.mass_count[b] == 0:
                    continue                              # no score rows: the term is not formed
                info = close(got[b, h, :k], want[b, :k], *MASS_TOL["bf16"], f"score term head {h} seq {b}")
        log(f"   score terms of heads {HEADS}: last max_abs={info['max_abs']:.3e}")
