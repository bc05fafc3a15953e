"""Tracked-set statistics from the middle layers only: a 24-layer model whose
formula-(2) term is formed in layers 5 to 20 (1-based) and skipped in the
others ([FD] 研究动机: the attention concentrates on few decoded tokens in the
middle layers).  Every layer runs the same kernels; the layers outside the
range call the attention without score rows.

The GPU's summed score is compared with the oracle's layer_range_score over
the same layers (mass tolerance), and the top-k with the usual rule: identical
on the GPU's own scores, and against the oracle's scores outside the near-tie
window.  Each layer has its own seeded weights and inputs.
"""
import types

import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, check_topk, close, log

pytestmark = pytest.mark.gpu

LAYERS, FIRST, LAST = 24, 5, 20


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16"])
def test_middle_layer_score(name, gpu):
    import torch
    import test_gpu_parity as T
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = W.make_workload(name)
    sh = wl.shape
    print(f"[gpu] middle-layer score {name}: {LAYERS} layers, score from {FIRST}..{LAST}", flush=True)
    table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
    n = sh.n_heads * sh.head_dim
    run = FlashCacheRunner(wl, device=gpu, layers=LAYERS)
    rows = W.full_refresh_rows(wl)
    st = run.upload_step(rows)
    terms = []
    for l in range(LAYERS):
        w_raw, x_raw = W.weights(wl, l), W.activations(wl, rows, 0, l)
        run.layer_step(st, run.to_device_array(x_raw), run.to_device_array(w_raw), l,
                       with_mass=FIRST <= l + 1 <= LAST)
        zeros = np.zeros((wl.pool_pages * W.PAGE, n))
        out = O.layer_step(W.as_f64(wl, x_raw), W.as_f64(wl, w_raw), rows.pos, rows.logical, rows.cu_q,
                           rows.kv_len, rows.mass_count, zeros, zeros.copy(), table, sh.n_heads, sh.head_dim,
                           sh.rope_base, W.PAGE)
        terms.append(out["mass"])
    torch.cuda.synchronize()
    score = T.head_sum(run.mass.cpu().numpy())
    run.topk(clear_mass=True)
    torch.cuda.synchronize()
    want = O.layer_range_score(terms, FIRST, LAST)
    info = close(score, want, *MASS_TOL[sh.dtype], f"{name} middle-layer score")
    log(f"   {name} score over layers {FIRST}..{LAST}: max_abs={info['max_abs']:.3e}")
    # the score is not the all-layer one
    assert np.abs(O.layer_range_score(terms, 1, LAYERS) - want).max() > 10 * MASS_TOL[sh.dtype][0]
    case = types.SimpleNamespace(wl=wl, kind=sh.dtype)
    check_topk(case, score, run.top_idx.cpu().numpy(), run.top_val.cpu().numpy(), run.top_cnt.cpu().numpy(),
               want)
