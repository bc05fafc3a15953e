"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/dllm.h declares, rejects bad arguments before touching the device,
and its workspace queries are pure functions of the shapes.  No compute call
is made (there is no GPU here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from io_aware_kv_amd import dllm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dllm.LIB_PATH):
        from io_aware_kv_amd import build
        build.build()
    return dllm.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dllm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(dllm.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert dllm.version() == 100
    assert dllm.status_string(0) == "ok"
    assert "duplicate" in dllm.status_string(-3)


NULL = None


def bbt(lib, n_seq, page_size, pool_pages, max_pages, seq_pages, perm, table, n_rows=0, cu=None,
        lg=None, slot=None):
    arr = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.int32)
    sp, pp, cu_, lg_ = arr(seq_pages), arr(perm), arr(cu), arr(lg)
    ptr = lambda a: None if a is None else a.ctypes.data
    return lib.dllm_build_block_table(n_seq, page_size, pool_pages, max_pages, ptr(sp), ptr(pp),
                                      table, n_rows, ptr(cu_), ptr(lg_), slot, None)


def test_block_table_errors_before_any_device_work(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every case fails validation first
    E_ARG, E_RANGE = -1, -3
    assert bbt(lib, 2, 16, 4, 2, [3, 1], [0, 1, 2, 3], fake) == E_RANGE      # > max_pages
    assert bbt(lib, 2, 16, 4, 4, [3, 2], [0, 1, 2, 3], fake) == E_RANGE      # > pool
    assert bbt(lib, 1, 16, 4, 4, [2], [0, 1, 1, 3], fake) == E_RANGE         # not a bijection
    assert bbt(lib, 1, 16, 4, 4, [2], [0, 1, 2, 4], fake) == E_RANGE
    assert bbt(lib, 1, 16, 4, 4, [-1], [0, 1, 2, 3], fake) == E_ARG
    assert bbt(lib, 1, 0, 4, 4, [1], [0, 1, 2, 3], fake) == E_ARG
    assert bbt(lib, 1, 16, 4, 4, [1], [0, 1, 2, 3], None) == E_ARG          # null table
    # rows: logical beyond the sequence, duplicate slot, bad cu_q
    assert bbt(lib, 1, 16, 4, 4, [1], [0, 1, 2, 3], fake, 1, [0, 1], [16], fake) == E_RANGE
    assert bbt(lib, 1, 16, 4, 4, [1], [0, 1, 2, 3], fake, 2, [0, 2], [3, 3], fake) == E_RANGE
    assert bbt(lib, 1, 16, 4, 4, [1], [0, 1, 2, 3], fake, 2, [0, 1], [3, 4], fake) == E_ARG
    assert bbt(lib, 2, 16, 4, 4, [1, 1], [0, 1, 2, 3], fake, 2, [0, 2, 1], [3, 4], fake) == E_ARG


def test_kernel_entry_points_reject_bad_shapes(lib):
    fake = ctypes.c_void_p(0x1000)
    f = lib.dllm_qkv_rope_cachewrite
    args = lambda dt, R, d, H, D, base: (dt, R, d, H, D, base, fake, fake, fake, fake, fake, fake, fake,
                                          1024, fake, 1 << 30, None)
    assert f(*args(1, 8, 4096, 32, 96, 5e5)) == -2          # head_dim 96
    assert f(*args(1, 8, 4000, 32, 128, 5e5)) == -2         # d_model not a multiple of 64
    assert f(*args(1, 8, 4096, 3, 64, 5e5)) == -2           # H*D not a multiple of 128
    assert f(*args(7, 8, 4096, 32, 128, 5e5)) == -2         # dtype
    assert f(*args(1, -1, 4096, 32, 128, 5e5)) == -1
    assert f(*args(1, 8, 4096, 32, 128, 0.0)) == -1         # rope base
    assert f(1, 8, 4096, 32, 128, 5e5, None, fake, fake, fake, fake, fake, fake, 1024, fake, 1 << 30,
             None) == -1                                     # null x
    assert f(*args(1, 0, 4096, 32, 128, 5e5)) == 0           # empty: nothing to do

    fp = lib.dllm_qkv_rope_cachewrite_paged
    def paged(dt=1, n_seq=1, R=8, d=4096, H=32, D=128, base=5e5, max_pages=32, page=16, table=fake):
        return fp(dt, n_seq, R, d, H, D, base, fake, fake, fake, fake, fake, table, max_pages, page, fake,
                  fake, fake, fake, 1024, fake, 1 << 30, None)
    assert paged(D=96) == -2                                 # same shape rules as the slot-taking call
    assert paged(n_seq=0) == -1
    assert paged(n_seq=1025) == -2                           # more sequences than the kernel stages
    assert paged(max_pages=0) == -1
    assert paged(page=0) == -1
    assert paged(table=None) == -1                           # null block table
    assert paged(R=0) == 0                                   # empty: nothing to do

    # the unfused comparison arm: bf16 only
    assert lib.dllm_qkv_project(0, 8, 4096, 32, 128, fake, fake, fake, None, 0, None) == -2
    assert lib.dllm_qkv_project(1, 8, 4096, 32, 96, fake, fake, fake, None, 0, None) == -2
    assert lib.dllm_qkv_project(1, 8, 4096, 32, 128, None, fake, fake, None, 0, None) == -1
    assert lib.dllm_qkv_project(1, 0, 4096, 32, 128, fake, fake, fake, None, 0, None) == 0
    assert lib.dllm_rope_apply(1, 8, 32, 128, 0.0, fake, fake, fake, None) == -1
    assert lib.dllm_rope_apply(1, 8, 32, 96, 5e5, fake, fake, fake, None) == -2
    assert lib.dllm_rope_apply(1, 8, 32, 128, 5e5, fake, None, fake, None) == -1
    assert lib.dllm_cache_write(0, 8, 32, 128, fake, fake, fake, fake, 1024, None) == -2
    assert lib.dllm_cache_write(1, 8, 32, 128, fake, None, fake, fake, 1024, None) == -1
    assert lib.dllm_cache_write(1, 0, 32, 128, fake, fake, fake, fake, 1024, None) == 0

    a = lib.dllm_sched_attention
    def att(dt=1, n_seq=1, R=8, H=32, D=128, page=16, max_kv=512, mask=None, off=None, words=0,
            mass=None, max_mass=0, macc=None, n_cap=512, ws=1 << 30, max_pages=32):
        return a(dt, n_seq, R, H, D, page, max_kv, fake, fake, fake, fake, 1 << 16, fake, max_pages,
                 fake, mask, off, words, mass, max_mass, macc, 0, n_cap, fake, fake, ws, None)
    assert att(D=64) == -2                                   # bf16 kernel is D = 128
    assert att(page=32) == -2
    assert att(max_kv=0) == -1
    assert att(n_seq=2000) == -2
    assert att(mask=fake, off=None, words=0) == -1           # mask without offsets
    assert att(mass=fake, macc=None) == -1                   # half of the mass arguments
    assert att(mass=fake, macc=fake, max_mass=200) == -2     # more than 128 window rows
    assert att(max_pages=5000) == -2
    assert att(dt=0, D=64, max_kv=10000) == -2               # fp32 path key limit
    # a score on the fused path needs the probability scratch; a short one is refused
    need = lib.dllm_sched_attention_workspace(1, 32, 2304, 32, 128, 2048, 2048, 32)
    assert att(n_seq=32, R=2304, max_kv=2048, n_cap=2048, mass=fake, macc=fake, max_mass=32,
               ws=need - 1, max_pages=128) == -1

    t = lib.dllm_topk_tracked
    assert t(1, 32, 512, 0, fake, fake, fake, fake, fake, 0, None) == -1
    assert t(1, 32, 512, 300, fake, fake, fake, fake, fake, 0, None) == -2
    assert t(1, 32, 5000, 32, fake, fake, fake, fake, fake, 0, None) == -2
    assert t(1, 0, 512, 32, fake, fake, fake, fake, fake, 0, None) == -1
    assert t(1, 32, 512, 32, None, fake, fake, fake, fake, 0, None) == -1
    assert lib.dllm_map_slots(0, 8, 16, 4, 4, fake, fake, fake, fake, None) == -1

    # the E4M3-cache dtype (2): accepted by the cache-writing projection and the
    # attention with head_dim 128; refused by the calls that have no cache
    assert lib.dllm_qkv_project(2, 8, 4096, 32, 128, fake, fake, fake, None, 0, None) == -2
    assert lib.dllm_rope_apply(2, 8, 32, 128, 5e5, fake, fake, fake, None) == -2
    assert lib.dllm_cache_write(2, 8, 32, 128, fake, fake, fake, fake, 1024, None) == -2
    assert f(*args(2, 8, 4096, 32, 64, 5e5)) == -2              # E4M3 caches need head_dim 128
    assert f(*args(2, 0, 4096, 32, 128, 5e5)) == 0               # accepted (empty: nothing to do)
    assert f(*args(3, 8, 4096, 32, 128, 5e5)) == -2              # no such dtype
    assert att(dt=2, D=64) == -2
    assert att(dt=3) == -2
    assert lib.dllm_qkv_rope_cachewrite_workspace(2, 72, 4096, 32, 128) == 0

    # decode side: sizes, dtype, stride, pointers and the workspace size are
    # checked before any launch
    c = lib.dllm_confidence_argmax
    assert c(1, -1, 1000, fake, 1000, fake, fake, fake, 1 << 20, None) == -1
    assert c(1, 4, 0, fake, 1000, fake, fake, fake, 1 << 20, None) == -1           # empty vocabulary
    assert c(1, 4, 1000, fake, 999, fake, fake, fake, 1 << 20, None) == -1         # stride < vocab
    assert c(5, 4, 1000, fake, 1000, fake, fake, fake, 1 << 20, None) == -1         # dtype
    assert c(1, 4, 1000, None, 1000, fake, fake, fake, 1 << 20, None) == -1         # null logits
    assert c(1, 4, 1000, fake, 1000, None, fake, fake, 1 << 20, None) == -1         # null token
    assert c(1, 4, 1000, fake, 1000, fake, fake, fake, 16, None) == -1              # short workspace
    assert c(1, 4, 1000, fake, 1000, fake, fake, None, 1 << 20, None) == -1         # no workspace
    assert c(1, 0, 1000, None, 1000, None, None, None, 0, None) == 0                # empty: nothing to do
    dc = lib.dllm_decode_commit
    assert dc(1, 1, 4, None, 1000, fake, 1000, 0.9, fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert dc(1, -1, 4, fake, 1000, fake, 1000, 0.9, fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert dc(1, 0, 4, fake, 1000, fake, 1000, 0.9, fake, fake, fake, fake, fake, 1 << 20, None) == 0
    dv = lib.dllm_decode_verify
    assert dv(1, 1, 4, fake, 1000, fake, 1000, None, 0.8, fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert dv(0, 1, 4, fake, 1000, fake, 999, fake, 0.8, fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert lib.dllm_confidence_commit(1, 4, None, fake, 0.9, fake, fake, None) == -1
    assert lib.dllm_confidence_commit(0, 4, None, None, 0.9, None, None, None) == 0
    assert lib.dllm_verify_accept(1, 4, fake, fake, None, fake, 0.8, fake, fake, None) == -1


def test_workspace_queries(lib):
    # the projection never needs scratch; attention needs it only when keys are
    # split (too few sequence x head pairs to fill the GPU), and then exactly
    # the per-split partial outputs and row statistics
    q = lib.dllm_qkv_rope_cachewrite_workspace
    for shape in ((1, 72, 4096, 32, 128), (0, 88, 256, 4, 64), (1, 65536, 4096, 32, 128)):
        assert q(*shape) == 0
    w = lib.dllm_sched_attention_workspace
    assert w(1, 32, 2304, 32, 128, 2048, 2048, 0) == 0       # 1024 pairs: fused path, no score
    # fused path with a score: bf16 probabilities (128 B per 64-key tile) and an
    # fp32 reference per window row, key tile, sequence and head
    assert w(1, 32, 2304, 32, 128, 2048, 2048, 32) == 32 * 32 * 32 * 32 * (128 + 4)
    assert w(2, 32, 2304, 32, 128, 2000, 2048, 7) == 32 * 32 * 32 * 7 * (128 + 4)
    assert w(0, 2, 88, 4, 64, 128, 128, 32) == 0             # fp32 path
    assert w(1, 32, 2304, 32, 128, 2048, 2048, 129) == 0     # more window rows than a query tile: refused
    small = w(1, 1, 72, 32, 128, 512, 512, 0)                # batch 1: keys split
    assert small > 0 and small % (128 * (128 * 2 + 2 * 4)) == 0   # bf16 partial rows and (max, sum)
    assert small == w(1, 1, 72, 32, 128, 512, 512, 32)       # the split path forms the score from its partials


def test_confidence_workspace_is_one_partial_per_row_and_split(lib):
    w = lib.dllm_confidence_workspace
    assert w(0, 1000) == 0 and w(4, 0) == 0
    assert w(1024, 131072) == 1024 * 16                       # many rows: one workgroup per row
    assert w(32, 131072) == 32 * 16 * 16                       # few rows: rows split 16 ways
    assert w(1, 1000) == 16                                    # narrow rows are never split
    for R, V in ((3, 4099), (40, 262147), (7, 65539)):
        assert w(R, V) % (16 * R) == 0 and w(R, V) // (16 * R) <= 64


def test_pack_mask_layout():
    rng = np.random.default_rng(0)
    vis = [rng.random((3, 70)) < 0.5, rng.random((2, 33)) < 0.5]
    bits, off = dllm.pack_mask(vis)
    assert off.tolist() == [0, 3 * 3]
    for b, v in enumerate(vis):
        words = (v.shape[1] + 31) // 32
        for i in range(v.shape[0]):
            for j in range(v.shape[1]):
                w = int(bits[off[b] + i * words + j // 32])
                assert ((w >> (j % 32)) & 1) == int(v[i, j])


def test_tuning_override(lib):
    # unknown knobs and values are refused and change nothing; NULL / "" restore
    # the automatic choice
    assert lib.dllm_set_tuning(b"nonsense", b"1") == -1
    assert lib.dllm_set_tuning(None, b"1") == -1
    assert lib.dllm_set_tuning(b"attn_splits", b"x3") == -1
    assert lib.dllm_set_tuning(b"attn_splits", b"-1") == -1
    assert lib.dllm_set_tuning(b"qkv_kernel", b"g999x1") == -1
    w = lib.dllm_sched_attention_workspace
    auto = w(1, 1, 72, 32, 128, 512, 512, 32)
    assert lib.dllm_set_tuning(b"attn_splits", b"2") == 0
    forced = w(1, 1, 72, 32, 128, 512, 512, 32)
    assert lib.dllm_set_tuning(b"attn_splits", None) == 0
    assert w(1, 1, 72, 32, 128, 512, 512, 32) == auto
    assert forced != auto and forced % (128 * (128 * 2 + 2 * 4)) == 0
    for name in (b"tiled", b"gemm", b"g256x256", b"g128x256o2", b"g128x128", b"mid6x6", b"mid8x12"):
        assert lib.dllm_set_tuning(b"qkv_kernel", name) == 0
    assert lib.dllm_set_tuning(b"qkv_kernel", b"") == 0


def test_noalloc_refuses_before_touching_the_device(lib):
    # the batch-32, 2048-key score needs more scratch than the static array:
    # refused with UNSUPPORTED before any HIP call (none is possible here)
    need = lib.dllm_sched_attention_workspace(1, 32, 2304, 32, 128, 2048, 2048, 32)
    assert need > dllm.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    rc = lib.dllm_sched_attention_noalloc(1, 32, 2304, 32, 128, 16, 2048, fake, fake, fake, fake, 65536, fake,
                                          128, fake, None, None, 0, fake, 32, fake, 1, 2048, fake, None)
    assert rc == -2
    # argument errors as the workspace-taking call
    assert lib.dllm_sched_attention_noalloc(1, 1, 72, 32, 128, 16, 512, None, fake, fake, fake, 512, fake,
                                            32, fake, None, None, 0, None, 0, None, 0, 0, fake, None) == -1
