"""The bench line's roofline accounting, on the CPU.

Every fraction the bench reports divides a kernel's time into its bound: the
algorithmic bytes over 8 TB/s or the algorithmic flops over 2.5 PFLOP/s,
whichever is larger.  The algorithmic work per unit is fixed by the method
([FD] 研究动机's per-layer traffic model and 核心方法's fused write): per
projection launch W_qkv once (3 n d bf16 values); per refreshed row x in, q
out and its K and V rows written; per cached key of a sequence its K and V
row read; per row q in and o out; 2 d 3n flops per projected row and 4 n flops
per visible (row, key) pair.  These cases write those closed forms out for
the workloads' steps (the batch-1 cache-phase and full-refresh steps, the
verify step under its mask, both steps of the batch-32 sweep and the tiny fp32
case) and compare the bench's figures with them, and check that a
counter-traffic record is used only while its kernel source is unchanged.
"""
import hashlib
import json
import os

import numpy as np
import pytest

import bench
from io_aware_kv_amd import workloads as W

D_MODEL = 4096          # d = n = H D for the LLaDA-8B-shaped layer
BF16 = 2


def _closed_form(R, kv, visible_pairs, d, n, el, kel):
    qkv_bytes = 3 * n * d * el + R * (d * el + n * el + 2 * n * kel)
    qkv_flops = 2 * R * d * 3 * n
    attn_bytes = sum(kv) * 2 * n * kel + 2 * R * n * el
    attn_flops = 4 * visible_pairs * n
    return qkv_bytes, qkv_flops, attn_bytes, attn_flops


def _bounds_us(b, f):
    return max(b / 8.0e12, f / 2.5e15) * 1e6


@pytest.mark.parametrize("name,kind,R,kv_each,n_seq,sum_bounds_us", [
    ("llada_b1", "step", 72, 512, 1, 14.07),          # HBM 12.88 + HBM 1.20
    ("llada_b1", "full", 512, 512, 1, 22.71),         # MFMA 20.62 + HBM 2.10
    ("llada_b32", "step", 2304, 2048, 32, 231.71),    # MFMA 92.77 + HBM 138.94
    ("llada_b32", "full", 65536, 2048, 32, 3518.44),  # MFMA 2638.83 + MFMA 879.61
])
def test_layer_work_matches_the_closed_forms(name, kind, R, kv_each, n_seq, sum_bounds_us):
    wl = W.make_workload(name)
    rows = W.full_refresh_rows(wl) if kind == "full" else W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    assert rows.n_rows == R and list(rows.kv_len) == [kv_each] * n_seq
    w = bench.layer_work(wl.shape, rows)
    qb, qf, ab, af = _closed_form(R, [kv_each] * n_seq, R * kv_each, D_MODEL, D_MODEL, BF16, BF16)
    assert (w["qkv_bytes"], w["qkv_flops"], w["attn_bytes"], w["attn_flops"]) == (qb, qf, ab, af)
    assert w["qkv_bound_us"] == pytest.approx(_bounds_us(qb, qf), rel=1e-12)
    assert w["attn_bound_us"] == pytest.approx(_bounds_us(ab, af), rel=1e-12)
    assert w["sum_of_bounds_us"] == pytest.approx(sum_bounds_us, abs=0.01)
    assert w["overlap_bound_us"] == pytest.approx(_bounds_us(qb + ab, qf + af), rel=1e-12)
    assert w["overlap_bound_us"] <= w["sum_of_bounds_us"] + 1e-9


def test_verify_step_counts_only_visible_pairs():
    """The verify step's flops count the (row, key) pairs its mask lets a row
    see: 4 sequences of 72 rows over 1056 keys (1024 context + 32 view slots),
    the 16 stale search entries hidden from every row, the view slots hidden
    from the ordinary rows and partly from the views."""
    wl = W.make_workload("verify_b4")
    rows = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    assert rows.n_rows == 288 and list(rows.kv_len) == [1056] * 4 and rows.visible is not None
    pairs = int(sum(v.sum() for v in rows.visible))
    assert pairs < 288 * 1056
    w = bench.layer_work(wl.shape, rows)
    qb, qf, ab, af = _closed_form(288, [1056] * 4, pairs, D_MODEL, D_MODEL, BF16, BF16)
    assert (w["qkv_bytes"], w["qkv_flops"], w["attn_bytes"], w["attn_flops"]) == (qb, qf, ab, af)
    assert w["qkv_bound"] == "hbm" and w["attn_bound"] == "hbm"
    assert w["sum_of_bounds_us"] == pytest.approx(23.00, abs=0.01)   # HBM 13.76 + HBM 9.24


def test_fp32_and_one_byte_caches():
    wl = W.make_workload("tiny_f32")
    rows = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    sh = wl.shape
    n = sh.n_heads * sh.head_dim
    vis = int(sum(v.sum() for v in rows.visible)) if rows.visible is not None else \
        int(sum((rows.cu_q[b + 1] - rows.cu_q[b]) * rows.kv_len[b] for b in range(len(rows.kv_len))))
    w = bench.layer_work(sh, rows)
    assert (w["qkv_bytes"], w["attn_bytes"]) == _closed_form(rows.n_rows, list(rows.kv_len), vis, sh.d_model, n,
                                                             4, 4)[0::2]
    wl = W.make_workload("llada_b32")
    rows = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    w8 = bench.layer_work(wl.shape, rows, cache_el=1)      # E4M3 K/V: one byte per element
    qb, _, ab, _ = _closed_form(2304, [2048] * 32, 0, D_MODEL, D_MODEL, BF16, 1)
    assert (w8["qkv_bytes"], w8["attn_bytes"]) == (qb, ab)


def test_counter_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    (tmp_path / "profiles").mkdir()
    rec = {"source": "kernel.hip", "source_sha256": hashlib.sha256(src.read_bytes()).hexdigest(),
           "bytes_per_launch": 123456789.0}
    (tmp_path / "profiles" / "k_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("k_traffic.json") == 123456789.0
    assert bench.counter_traffic("missing_traffic.json") is None
    src.write_text("// kernel v2\n")
    assert bench.counter_traffic("k_traffic.json") is None


def test_committed_traffic_records_match_their_sources():
    """Every committed counter record names an existing source, and its
    figure is the calibrated sum of its raw counter readings."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prof = os.path.join(root, "profiles")
    recs = [f for f in os.listdir(prof) if f.endswith("_traffic.json")]
    assert recs
    for f in recs:
        r = json.load(open(os.path.join(prof, f)))
        assert os.path.exists(os.path.join(root, r["source"])), f
        fetch = r.get("fetch_kib_raw", r.get("fetch_kib_per_launch"))
        write = r.get("write_kib_raw", r.get("write_kib_per_launch"))
        want = fetch * 1024 * r["fetch_factor"] + write * 1024 * r["write_factor"]
        assert r["bytes_per_launch"] == pytest.approx(want, rel=1e-9), f
        assert np.isfinite(r["bytes_per_launch"]) and r["bytes_per_launch"] > 0
