"""Block-granular caching steps (DualCache and the active window of
PrefixCache / FreeCache) in the oracle: the row sets, and the property that
makes such caching exact when the cache holds current values.

[FST] Fast-dLLM article (senqingzn.com), block-wise KV cache section: the
prefix, and with DualCache also the masked suffix, is read from the cache
while the current block is decoded.  [FDLM] FlashDLM notes (papernotes.org),
FreeCache: the active window is the current block and every later block; the
prompt and the finished blocks are frozen.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W


def _tiny_with_suffix():
    """tiny_f32's layer with two sequences of prompt 64 + gen 128, one block
    decoded: the window 96..127 has a masked suffix 128..191 behind it."""
    base = W.make_workload("tiny_f32")
    rng = np.random.default_rng(3)
    seqs = [W._cache_seq(rng, 192, 64, 1, 4, 44) for _ in range(2)]
    seq_pages = np.array([s.pages for s in seqs], dtype=np.int32)
    pool = int(seq_pages.sum())
    return W.Workload(name="tiny_f32", wid=base.wid, shape=base.shape, seqs=seqs, seq_pages=seq_pages,
                      pool_pages=pool, pool_perm=rng.permutation(pool).astype(np.int32),
                      max_pages=int(seq_pages.max()))


def _full_then(name, mode):
    wl = _tiny_with_suffix() if name == "tiny_suffix" else W.make_workload(name)
    sh = wl.shape
    table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
    w = W.as_f64(wl, W.weights(wl, 0))
    rows0 = W.full_refresh_rows(wl)
    x0 = W.as_f64(wl, W.activations(wl, rows0, 0))
    n = sh.n_heads * sh.head_dim
    kc = np.zeros((wl.pool_pages * W.PAGE, n))
    vc = np.zeros_like(kc)
    out0 = O.layer_step(x0, w, rows0.pos, rows0.logical, rows0.cu_q, rows0.kv_len, rows0.mass_count, kc, vc,
                        table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
    rows = W.block_cache_rows(wl, mode)
    # the same activations the full refresh used at these positions
    pick = []
    for b in range(wl.n_seq):
        lg0 = rows0.logical[rows0.cu_q[b]:rows0.cu_q[b + 1]]
        where = {int(p): rows0.cu_q[b] + i for i, p in enumerate(lg0)}
        pick += [where[int(p)] for p in rows.logical[rows.cu_q[b]:rows.cu_q[b + 1]]]
    pick = np.array(pick)
    out = O.layer_step(x0[pick], w, rows.pos, rows.logical, rows.cu_q, rows.kv_len, rows.mass_count,
                       out0["k_cache"], out0["v_cache"], table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
    return wl, rows, out0, out, pick


@pytest.mark.parametrize("mode", W.BLOCK_CACHE_MODES)
def test_row_sets(mode):
    for name in ("tiny_f32", "mixed_b8", "llada_b32"):
        wl = W.make_workload(name)
        rows = W.block_cache_rows(wl, mode)
        assert not rows.mass_count.any() and rows.visible is None
        for b, s in enumerate(wl.seqs):
            lg = rows.logical[rows.cu_q[b]:rows.cu_q[b + 1]]
            w0 = int(s.window[0])
            want = s.window if mode == "dual" else np.arange(w0, s.ctx)
            assert np.array_equal(lg, want)
            assert np.array_equal(rows.pos[rows.cu_q[b]:rows.cu_q[b + 1]], lg)
            assert rows.kv_len[b] == s.ctx
            # the frozen part: the prompt and every finished block
            assert w0 == s.prompt + W.BLOCK * s.decoded_blocks


@pytest.mark.parametrize("mode", W.BLOCK_CACHE_MODES)
def test_exact_cache_reproduces_the_full_refresh(mode):
    """With every cached K/V equal to what a full forward computes, a block
    step that rewrites its rows from the same inputs leaves the cache as it
    was and gives its rows the full refresh's outputs."""
    wl, rows, out0, out, pick = _full_then("tiny_suffix", mode)
    np.testing.assert_allclose(out["o"], out0["o"][pick], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["q"], out0["q"][pick], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["k_cache"], out0["k_cache"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["v_cache"], out0["v_cache"], rtol=1e-12, atol=1e-13)


def test_stale_suffix_changes_only_what_reads_it():
    """DualCache reads the masked suffix from the cache: perturbing a cached
    suffix key changes the window rows' outputs, while perturbing it in an
    active-window step changes nothing (the step rewrites the suffix first)."""
    name = "tiny_suffix"
    wl, rows_d, out0, out_d, pick_d = _full_then(name, "dual")
    _, rows_a, _, out_a, pick_a = _full_then(name, "active")
    sh = wl.shape
    table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
    s = wl.seqs[0]
    suffix_pos = int(s.window[-1]) + 1
    assert suffix_pos < s.ctx
    slot = int(O.row_slots(table, [0, 1], [suffix_pos], W.PAGE)[0])
    k_bad = out0["k_cache"].copy()
    v_bad = out0["v_cache"].copy()
    v_bad[slot] += 3.0
    w = W.as_f64(wl, W.weights(wl, 0))
    x0 = W.as_f64(wl, W.activations(wl, W.full_refresh_rows(wl), 0))
    d = O.layer_step(x0[pick_d], w, rows_d.pos, rows_d.logical, rows_d.cu_q, rows_d.kv_len, rows_d.mass_count,
                     k_bad, v_bad, table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
    a = O.layer_step(x0[pick_a], w, rows_a.pos, rows_a.logical, rows_a.cu_q, rows_a.kv_len, rows_a.mass_count,
                     k_bad, v_bad, table, sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
    r0, r1 = rows_d.cu_q[0], rows_d.cu_q[1]
    assert np.abs(d["o"][r0:r1] - out_d["o"][r0:r1]).min() > 0      # every window row sees the stale value
    np.testing.assert_allclose(a["o"], out_a["o"], rtol=1e-12, atol=1e-13)
