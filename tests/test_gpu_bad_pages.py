"""Attention over a block table with out-of-range page entries.

The attention reads every key through the sequence's block table ([FD]
核心方法: block-table scheduled attention over the paged cache).  An entry
outside the pool (negative, or at least the pool's page count) is never
dereferenced: the keys of that page are hidden from every row, so each row's
softmax runs over the remaining keys and those keys receive no formula-(2)
score.  Here some pages of each sequence get such entries (-1, -2^31, the pool
size, the pool size + 100, 2^31 - 1; one sequence loses its first and its last,
partial page), and o and the score terms of three heads are compared with the
oracle run on the same table with those keys marked invisible (the oracle
reads any real row for them, which the zero probability then drops), on both
attention paths (keys split and merged by the second launch, and the single
launch that keeps the window rows' probabilities), with bf16 caches and with
one-byte E4M3 caches (seeded codes of moderate magnitude; the oracle reads
their decoded values).
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, TOL, close, log

pytestmark = pytest.mark.gpu

H, D = 32, 128
HEADS = (0, 17, 31)


def _cols(t, heads):
    import torch
    idx = torch.cat([torch.arange(h * D, (h + 1) * D) for h in heads]).to(t.device)
    return t.index_select(1, idx).to(torch.float64).cpu().numpy()


def _codes(shape, salt):
    """Seeded E4M3 codes with exponent fields 4..8 (magnitudes 1/8 .. 3.75) and random signs."""
    r = np.random.default_rng(9500 + salt)
    mag = r.integers(0x20, 0x48, size=shape)
    return (mag | (r.integers(0, 2, size=shape) << 7)).astype(np.uint8)


@pytest.mark.parametrize("splits,fmt", [(None, "bf16"), ("1", "bf16"), ("3", "bf16"), (None, "e4m3"), ("3", "e4m3")])
def test_out_of_range_pages_hide_their_keys(splits, fmt, gpu):
    import torch
    from io_aware_kv_amd import dllm
    log(f"[gpu] out-of-range page entries, splits {splits or 'auto'}, {fmt} cache")
    kv, rows, mass = (1000, 700, 2100), (72, 40, 130), (32, 16, 32)
    lc = W.long_context(kv, rows, mass, seed=61 + (0 if splits is None else int(splits)))
    n_seq, n_out = len(kv), H * D
    q, kc, vc = W.long_context_tensors(lc, n_out, gpu)
    if fmt == "e4m3":
        kc8, vc8 = _codes(tuple(kc.shape), 1), _codes(tuple(vc.shape), 2)
        kc, vc = torch.from_numpy(kc8).to(gpu), torch.from_numpy(vc8).to(gpu)
    table = O.build_block_table(lc.seq_pages, lc.pool_perm, lc.pool_pages, lc.max_pages).astype(np.int64)
    P = lc.pool_pages
    bad = {(0, 3): -1, (0, 10): P, (1, 0): -(1 << 31), (1, 20): P + 100, (2, 0): (1 << 31) - 1,
           (2, int(lc.seq_pages[2]) - 1): -1, (2, 40): P}
    for (b, j), v in bad.items():
        table[b, j] = v
    table32 = table.astype(np.int32)
    R = int(lc.rows.sum())
    cu = np.concatenate([[0], np.cumsum(lc.rows)]).astype(np.int32)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(gpu)
    table_dev = i32(table32.reshape(-1))
    cu_d, kv_d = i32(cu), i32(lc.kv)
    max_kv, n_cap = int(lc.kv.max()), int(lc.kv.max())
    max_mass = int(lc.mass_count.max())
    o = torch.empty(R, n_out, dtype=torch.bfloat16, device=gpu)
    score = torch.full((n_seq, H, n_cap), 7.0, dtype=torch.float32, device=gpu)
    dllm.set_tuning("attn_splits", splits)
    try:
        code = dllm.BF16 if fmt == "bf16" else dllm.BF16_E4M3KV
        ws_b = dllm.sched_attention_workspace(code, n_seq, R, H, D, max_kv, n_cap, max_mass)
        ws = torch.zeros(max(ws_b, 256), dtype=torch.uint8, device=gpu)
        dllm.sched_attention(q, cu_d, kc, vc, table_dev, lc.max_pages, kv_d, o, ws, H, D, max_kv,
                             mass_count=i32(lc.mass_count), max_mass_rows=max_mass, mass_accum=score,
                             n_cap=n_cap, mass_overwrite=True)
        torch.cuda.synchronize()
    finally:
        dllm.set_tuning("attn_splits", None)

    # the oracle: the same table with each bad entry pointing at page 0 and its keys invisible
    ok_table = np.where((table >= 0) & (table < P), table, 0).astype(np.int32)
    visible = []
    for b in range(n_seq):
        k = np.arange(int(lc.kv[b]))
        page_ok = (table[b, k // W.PAGE] >= 0) & (table[b, k // W.PAGE] < P)
        assert not page_ok.all()
        visible.append(np.broadcast_to(page_ok, (int(lc.rows[b]), len(k))))
    if fmt == "e4m3":
        idx = np.concatenate([np.arange(h * D, (h + 1) * D) for h in HEADS])
        k_or, v_or = O.e4m3_decode(kc8[:, idx]), O.e4m3_decode(vc8[:, idx])
    else:
        k_or, v_or = _cols(kc, HEADS), _cols(vc, HEADS)
    o_want, probs = O.attention(_cols(q, HEADS), k_or, v_or, ok_table, cu, lc.kv,
                                len(HEADS), D, W.PAGE, visible=visible)
    info = close(_cols(o, HEADS), o_want, *TOL["bf16"], "o with hidden pages")
    got = score.cpu().numpy()
    for j, h in enumerate(HEADS):
        want = O.column_mass([pb[j:j + 1] for pb in probs], lc.mass_count, n_cap) / H
        for b in range(n_seq):
            k = int(lc.kv[b])
            close(got[b, h, :k], want[b, :k], *MASS_TOL["bf16"], f"score head {h} seq {b}")
            hidden = ~visible[b][0]
            assert np.all(got[b, h, :k][hidden] == 0.0), "a hidden key received score"
    log(f"   o of heads {HEADS}: max_abs={info['max_abs']:.3e}; hidden keys score 0")
