"""The score rows of formula (2) at the C ABI: the first mass_count[b] query
rows of sequence b are the masked-window rows M_b ([FD] 方法步骤详情 step 4),
and the order of a sequence's rows is otherwise free.

dllm_sched_attention takes a count per sequence instead of a flag per row;
these tests pin down what that contract means on every attention path (the
single launch that keeps the window rows' probabilities, the key-split launch
whose merge forms the score, the fp32 kernel):

- permuting the rows after the window changes nothing but the order of o's
  rows: the score is bit-identical and every row's output is bit-identical;
- permuting the window rows among themselves permutes o the same way and
  changes the score only by the order of its row sum;
- the rows counted are the first mass_count[b], whatever they are: with the
  window moved to the end the score is the oracle's column mass of the rows
  now in front;
- a count outside 0..min(max_mass_rows, rows of b) is clamped to that range
  (a count of 0 or less leaves the sequence's score as it was).
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, close, log

pytestmark = pytest.mark.gpu


def _to64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def _attend(run, st, q, mass_count, max_mass, overwrite=True):
    """One attention call over layer 0's cache with the given query rows and
    score rows; returns (o, per-head score) as host arrays."""
    import torch
    from io_aware_kv_amd import dllm
    o = torch.empty_like(st.o)
    ws_b = dllm.sched_attention_workspace(run.dt_cache, run.wl.n_seq, st.n_rows, run.H, run.D, st.max_kv,
                                          run.n_cap, max_mass)
    ws = torch.zeros(max(ws_b, 256), dtype=torch.uint8, device=run.device)
    run.mass.fill_(7.0)                                    # sentinel: overwritten where a term is formed
    mc = torch.tensor(mass_count, dtype=torch.int32, device=run.device)
    dllm.sched_attention(q, st.cu_q, run.k_cache[0], run.v_cache[0], run.page_table, run.wl.max_pages,
                         st.kv_len, o, ws, run.H, run.D, st.max_kv, mass_count=mc, max_mass_rows=max_mass,
                         mass_accum=run.mass, n_cap=run.n_cap, mass_overwrite=overwrite)
    torch.cuda.synchronize()
    return o.cpu(), run.mass.cpu().numpy().copy()


@pytest.mark.parametrize("name,splits", [("tiny_f32", None), ("tiny_bf16", "1"), ("tiny_bf16", "2"),
                                         ("llada_b1", "1"), ("llada_b1", "4")])
def test_score_rows_are_the_first_mass_count_rows(name, splits, gpu):
    import torch
    from io_aware_kv_amd import dllm
    from io_aware_kv_amd.runner import FlashCacheRunner
    log(f"[gpu] score rows first: {name}, attention splits {splits or 'automatic'}")
    wl = W.make_workload(name)
    sh = wl.shape
    run = FlashCacheRunner(wl, device=gpu, layers=1)
    rows = W.full_refresh_rows(wl)                          # window rows first
    st = run.upload_step(rows)
    run.cache_update_paged(st, run.to_device_array(W.activations(wl, rows, 0, 0)),
                           run.to_device_array(W.weights(wl, 0)), 0)
    torch.cuda.synchronize()
    cu = rows.cu_q
    m = rows.mass_count
    mmax = int(m.max())
    assert np.all(m == mmax) and np.all(np.diff(cu) > mmax), "the clamp checks assume equal windows"
    rng = np.random.default_rng(77)
    # three orders of each sequence's rows: the rest shuffled, the window
    # shuffled, the window moved behind the rest
    rest_perm, win_perm, win_last = [], [], []
    for b in range(wl.n_seq):
        r0, r1, mb = int(cu[b]), int(cu[b + 1]), int(m[b])
        win, rest = np.arange(r0, r0 + mb), np.arange(r0 + mb, r1)
        rest_perm.append(np.concatenate([win, rng.permutation(rest)]))
        win_perm.append(np.concatenate([rng.permutation(win), rest]))
        win_last.append(np.concatenate([rest, win]))
    orders = {k: torch.from_numpy(np.concatenate(v)).to(gpu)
              for k, v in (("rest", rest_perm), ("win", win_perm), ("last", win_last))}
    dllm.set_tuning("attn_splits", splits)
    try:
        o0, s0 = _attend(run, st, st.q, m, mmax)
        got = {k: _attend(run, st, st.q[idx].contiguous(), m, mmax) for k, idx in orders.items()}
        # clamps: counts above the row cap and above the sequence's rows, and
        # counts of zero or less (the sequence keeps its old score)
        o_hi, s_hi = _attend(run, st, st.q, m + 1000, mmax)
        small = np.minimum(m, 3)
        o_cap, s_cap = _attend(run, st, st.q, m + 1000, 3)
        o_sm, s_sm = _attend(run, st, st.q, small, 3)
        neg = np.where(np.arange(wl.n_seq) % 2 == 0, -5, 0).astype(np.int32)
        _, s_neg = _attend(run, st, st.q, neg, mmax)
    finally:
        dllm.set_tuning("attn_splits", None)

    # rest permuted: score bit-identical, o rows permuted bit-identically
    idx = orders["rest"].cpu()
    assert torch.equal(got["rest"][0], o0[idx]), "o changed when the non-window rows were reordered"
    assert np.array_equal(got["rest"][1], s0), "score changed when the non-window rows were reordered"
    # window permuted: o permuted bit-identically; score equal up to the row-sum order
    idx = orders["win"].cpu()
    assert torch.equal(got["win"][0], o0[idx])
    info = close(got["win"][1], s0, *MASS_TOL[sh.dtype], f"{name} score, window rows reordered")
    log(f"   window rows reordered: score max_abs {info['max_abs']:.2e}")
    # clamps
    assert np.array_equal(s_hi, s0) and torch.equal(o_hi, o0), "count above max_mass_rows not clamped"
    assert np.array_equal(s_cap, s_sm) and torch.equal(o_cap, o_sm), "count above the row cap not clamped"
    assert not np.array_equal(s_sm, s0)
    assert np.all(s_neg == 7.0), "a sequence with no score rows had its score changed"

    # the window moved last: the score is the column mass of the rows now first,
    # by the oracle on the GPU's own q and cache rows
    table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
    q_last = _to64(st.q[orders["last"]])
    kc, vc = _to64(run.k_cache[0]), _to64(run.v_cache[0])
    _, probs = O.attention(q_last, kc, vc, table, cu, rows.kv_len, sh.n_heads, sh.head_dim, W.PAGE)
    want = O.column_mass(probs, m, wl.n_cap)
    _, probs0 = O.attention(_to64(st.q), kc, vc, table, cu, rows.kv_len, sh.n_heads, sh.head_dim, W.PAGE)
    want0 = O.column_mass(probs0, m, wl.n_cap)
    # keys at or past kv_len keep the sentinel (the term is stored for the keys only)
    keys = np.arange(wl.n_cap)[None, :] < rows.kv_len[:, None]
    gs_last = np.where(keys, got["last"][1].sum(axis=1, dtype=np.float64), 0.0)
    gs0 = np.where(keys, s0.sum(axis=1, dtype=np.float64), 0.0)
    assert np.all(got["last"][1][~np.broadcast_to(keys[:, None, :], s0.shape)] == 7.0)
    info = close(gs_last, want, *MASS_TOL[sh.dtype], f"{name} score of the rows in front")
    close(gs0, want0, *MASS_TOL[sh.dtype], f"{name} score of the window rows")
    assert np.abs(want - want0).max() > 10 * MASS_TOL[sh.dtype][0], "the two row sets give the same score"
    log(f"   window moved last: score of the rows in front max_abs {info['max_abs']:.2e}")
