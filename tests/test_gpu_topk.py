"""GPU top-k (dllm_topk_tracked) against the oracle's top-k, outside the layer
step: every shape class of the kernel (one, two, four or eight positions per
thread; score rows that are or are not 16-byte aligned), tie-heavy scores
(small multiples of 1/8, so fp32 head sums are exact and many positions tie
at the k-th score), empty and full candidate sets, k = 1 and the maximum 256.

The kernel's scores are the fp32 sums over heads in ascending head order; the
oracle's top-k, run on those same fp32 scores, must give the same positions
in the same order, bit for bit, the same count, and values equal to the
scores.  With clear_mass the per-head input must read zero afterwards.
"""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    # (n_seq, n_heads, n_cap, k, eligible fraction, tie-heavy)
    (1, 32, 512, 32, 0.6, False),
    (2, 32, 512, 32, 0.6, True),
    (2, 32, 512, 256, 0.9, True),      # one per thread, ranks across all eight waves
    (1, 1, 1, 1, 1.0, False),
    (2, 3, 7, 4, 1.0, True),
    (3, 32, 1001, 32, 0.5, True),      # two per thread, ragged tail
    (2, 32, 1024, 256, 0.9, True),
    (4, 32, 1056, 32, 0.6, True),      # four per thread, aligned runs
    (2, 8, 1057, 17, 0.7, True),       # four per thread, unaligned rows: scalar loads
    (2, 32, 2048, 32, 0.6, False),
    (1, 32, 3001, 256, 0.4, True),     # eight per thread, unaligned
    (2, 32, 4096, 100, 0.5, True),     # eight per thread, aligned, maximum n_cap
    (2, 4, 300, 32, 0.0, False),       # no candidates
    (2, 4, 300, 256, 0.3, False),      # fewer candidates than k
    (1, 2, 64, 8, 1.0, True),          # everything tied at one value
]


def fp32_head_sum(m: np.ndarray) -> np.ndarray:
    out = np.zeros((m.shape[0], m.shape[2]), dtype=np.float32)
    for h in range(m.shape[1]):
        out = (out + m[:, h, :]).astype(np.float32)
    return out


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}h{c[1]}n{c[2]}k{c[3]}" for c in CASES])
@pytest.mark.parametrize("clear", [False, True])
def test_topk_matches_oracle(case, clear, gpu):
    import torch
    from io_aware_kv_amd import dllm
    B, H, n_cap, k, frac, ties = case
    rng = np.random.default_rng(1000 + n_cap + 7 * k + B)
    if ties:
        if n_cap == 64:
            m = np.full((B, H, n_cap), 0.25, dtype=np.float32)
        else:
            m = (rng.integers(0, 6, size=(B, H, n_cap)) / 8.0).astype(np.float32)
    else:
        m = (rng.random((B, H, n_cap)) * 1e-3).astype(np.float32)
    elig = (rng.random((B, n_cap)) < frac).astype(np.uint8)
    print(f"[gpu] topk B={B} H={H} n_cap={n_cap} k={k} clear={clear}", flush=True)
    mass = torch.from_numpy(m).to(gpu)
    el = torch.from_numpy(elig).to(gpu)
    idx = torch.full((B, k), -7, dtype=torch.int32, device=gpu)
    val = torch.full((B, k), 7.0, dtype=torch.float32, device=gpu)
    cnt = torch.full((B,), -7, dtype=torch.int32, device=gpu)
    dllm.topk_tracked(mass, el, k, idx, val, cnt, clear_mass=clear)
    torch.cuda.synchronize()
    score = fp32_head_sum(m)
    o_idx, o_val, o_cnt = O.topk(score.astype(np.float64), elig.astype(bool), k)
    g_idx, g_val, g_cnt = idx.cpu().numpy(), val.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(g_cnt, o_cnt)
    assert np.array_equal(g_idx, o_idx)
    for b in range(B):
        n = int(g_cnt[b])
        assert np.array_equal(g_val[b, :n], score[b, g_idx[b, :n]])
        assert not g_val[b, n:].any()
    after = mass.cpu().numpy()
    if clear:
        assert not after.any()
    else:
        assert np.array_equal(after, m)
