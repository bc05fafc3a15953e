"""The allocation-free attention entry point (dllm_sched_attention_noalloc,
for callers that cannot allocate: graph capture, serving loops) against the
workspace-taking dllm_sched_attention, through the C ABI.  Both run the same
kernels, so o and the score must agree bit for bit.  Two calls in a row share
the static scratch array, the second with a smaller input: the mixed batch
(no key split; the score keeps its probabilities in the scratch array), then
the batch-1 step (keys split; partial outputs in the scratch array), then the
verify step under its mask.  A call that would need more than the array is
refused before any work is enqueued."""
import numpy as np
import pytest

from io_aware_kv_amd import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(name, gpu):
    import torch
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = W.make_workload(name)
    run = FlashCacheRunner(wl, device=gpu, layers=1)
    g = torch.Generator(device=gpu)
    g.manual_seed(1234 + wl.wid)
    for c in (run.k_cache[0], run.v_cache[0]):
        c.copy_(torch.randn(c.shape, generator=g, device=gpu).to(c.dtype))
    rows = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    st = run.upload_step(rows)
    st.q.copy_(torch.randn(st.q.shape, generator=g, device=gpu).to(st.q.dtype))
    return wl, run, st


def _attend(wl, run, st, noalloc):
    import torch
    from io_aware_kv_amd import dllm
    sh = wl.shape
    o = torch.full_like(st.o, float("nan"))
    mass = torch.full_like(run.mass, 7.0)
    kw = dict(mask_bits=st.mask_bits, mask_off=st.mask_off, mass_count=st.mass_count,
              max_mass_rows=st.max_mass, mass_accum=mass, n_cap=run.n_cap, mass_overwrite=True)
    if noalloc:
        dllm.sched_attention_noalloc(st.q, st.cu_q, run.k_cache[0], run.v_cache[0], run.page_table,
                                     wl.max_pages, st.kv_len, o, sh.n_heads, sh.head_dim, st.max_kv, **kw)
    else:
        dllm.sched_attention(st.q, st.cu_q, run.k_cache[0], run.v_cache[0], run.page_table, wl.max_pages,
                             st.kv_len, o, st.ws_attn, sh.n_heads, sh.head_dim, st.max_kv, **kw)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy(), mass.cpu().numpy()


def test_noalloc_matches_workspace_entry_point(gpu):
    from io_aware_kv_amd import dllm
    seen = []
    for name in ("mixed_b8", "llada_b1", "verify_b4"):
        wl, run, st = _inputs(name, gpu)
        sh = wl.shape
        need = dllm.sched_attention_workspace(dllm.BF16, wl.n_seq, st.n_rows, sh.n_heads, sh.head_dim,
                                              st.max_kv, run.n_cap, st.max_mass)
        assert 0 < need <= dllm.NOALLOC_SCRATCH_BYTES, (name, need)
        seen.append(need)
        o_ref, m_ref = _attend(wl, run, st, noalloc=False)
        o_na, m_na = _attend(wl, run, st, noalloc=True)
        assert np.array_equal(o_ref, o_na), name
        assert np.array_equal(m_ref, m_na), name
        print(f"[gpu] no-alloc attention {name}: {st.n_rows} rows, scratch {need / 2**20:.1f} MiB, "
              f"o and score bit-identical", flush=True)
    assert seen[1] < seen[0]        # the second call is the smaller one


def test_noalloc_refuses_more_than_its_array(gpu):
    import torch
    from io_aware_kv_amd import dllm
    wl = W.make_workload("llada_b32")
    sh = wl.shape
    rows = W.config_step_rows(wl, W.seeded_tracked(wl, 1))
    need = dllm.sched_attention_workspace(dllm.BF16, wl.n_seq, rows.n_rows, sh.n_heads, sh.head_dim, 2048,
                                          wl.n_cap, 32)
    assert need > dllm.NOALLOC_SCRATCH_BYTES
    lib = dllm.load()
    fake = torch.empty(16, dtype=torch.int32, device=gpu).data_ptr()
    rc = lib.dllm_sched_attention_noalloc(dllm.BF16, wl.n_seq, rows.n_rows, sh.n_heads, sh.head_dim, 16, 2048,
                                          fake, fake, fake, fake, 65536, fake, wl.max_pages, fake, None, None,
                                          0, fake, 32, fake, 1, wl.n_cap, fake, None)
    assert rc == -2
