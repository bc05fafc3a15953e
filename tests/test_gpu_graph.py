"""The step is deterministic and survives hipGraph capture: repeated eager runs
and repeated graph replays (with eager work and synchronisation between them)
give bit-identical outputs.  The kernels reduce in fixed orders and clear
their own counters, so nothing depends on replay count."""
import numpy as np
import pytest

from parity import Case, log

pytestmark = pytest.mark.gpu


def _snapshot(run, st):
    import torch
    torch.cuda.synchronize()
    return {"q": st.q.view(torch.int16).cpu().numpy().copy() if st.q.dtype == torch.bfloat16 else st.q.cpu().numpy().copy(),
            "o": st.o.view(torch.int16).cpu().numpy().copy() if st.o.dtype == torch.bfloat16 else st.o.cpu().numpy().copy(),
            "k": run.k_cache[0].view(torch.int16).cpu().numpy().copy(),
            "idx": run.top_idx.cpu().numpy().copy(), "val": run.top_val.cpu().numpy().copy(),
            "cnt": run.top_cnt.cpu().numpy().copy()}


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["tiny_bf16", "llada_b1", "verify_b4"])
def test_graph_replay_bit_identical(name, gpu):
    import torch
    from io_aware_kv_amd.runner import FlashCacheRunner
    log(f"[gpu] graph replay {name}")
    c = Case(name)
    run = FlashCacheRunner(c.wl, device=gpu, layers=1)
    run.k_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.k1_in)))
    run.v_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.v1_in)))
    st = run.upload_step(c.rows1)
    x = run.to_device_array(c.x1_raw)
    w = run.to_device_array(c.w_raw)

    def step():
        run.layer_step(st, x, w, 0)
        run.topk(clear_mass=True)

    step()
    ref = _snapshot(run, st)
    step()
    _same(ref, _snapshot(run, st))                      # eager determinism

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        st.o.zero_()
        st.q.zero_()
        run.top_idx.fill_(-7)
        junk = torch.randn(1024, device=gpu).sum()      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        _same(ref, _snapshot(run, st))
        assert float(junk) == float(junk)
