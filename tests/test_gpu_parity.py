"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Step 0 of every workload is a full refresh (every position queried and
written); step 1 is the workload's own step (cache phase, mixed batch or
verify views).  Integer outputs (page table, slots, cache placement, top-k)
are compared bit for bit; floating outputs within the tolerances in
tests/parity.py; cache rows a step must not write are compared bit for bit
against the sentinel they held.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import (MASS_TOL, TOL, Case, check_topk, close, device_bits, device_values, log, measure)

pytestmark = pytest.mark.gpu

_CASES = {}


def case(name, heavy=False):
    key = (name, heavy)
    if key not in _CASES:
        _CASES[key] = Case(name, heavy)
    return _CASES[key]


def head_sum(m):
    """[B, H, n_cap] per-head scores -> [B, n_cap], summed in ascending head
    order in fp32, the way dllm_topk_tracked forms its scores."""
    out = np.zeros((m.shape[0], m.shape[2]), dtype=np.float32)
    for h in range(m.shape[1]):
        out = (out + m[:, h, :]).astype(np.float32)
    return out


def run_gpu_step(c: Case, step: int, gpu, fused_slots: bool = True, unfused: bool = False):
    import torch
    from io_aware_kv_amd.runner import FlashCacheRunner
    wl = c.wl
    rows = c.rows0 if step == 0 else c.rows1
    x_raw = c.x0_raw if step == 0 else c.x1_raw
    run = FlashCacheRunner(wl, device=gpu, layers=1)
    if step == 0:
        run.k_cache[0].copy_(run.to_device_array(c.k_init_raw))
        run.v_cache[0].copy_(run.to_device_array(c.v_init_raw))
    else:
        run.k_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.k1_in)))
        run.v_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.v1_in)))
    k_before = device_bits(run.k_cache[0])
    v_before = device_bits(run.v_cache[0])
    st = run.upload_step(rows)
    x = run.to_device_array(x_raw)
    w = run.to_device_array(c.w_raw)
    run.layer_step(st, x, w, 0, fused_slots=fused_slots, unfused=unfused)
    mass = head_sum(run.mass.cpu().numpy())
    run.topk(clear_mass=True)
    torch.cuda.synchronize()
    return {"run": run, "st": st, "k_before": k_before, "v_before": v_before, "mass": mass,
            "page_table": run.page_table.cpu().numpy().reshape(wl.n_seq, wl.max_pages),
            "slot": st.slot.cpu().numpy(), "q": device_values(st.q), "o": device_values(st.o),
            "k_cache": device_values(run.k_cache[0]), "v_cache": device_values(run.v_cache[0]),
            "k_bits": device_bits(run.k_cache[0]), "v_bits": device_bits(run.v_cache[0]),
            "idx": run.top_idx.cpu().numpy(), "val": run.top_val.cpu().numpy(),
            "cnt": run.top_cnt.cpu().numpy(), "mass_after": run.mass.cpu().numpy()}


def compare_step(c: Case, g: dict, step: int, exact_topk: bool = False, o_ref=None):
    """o_ref: the oracle o to gate o against (default: the step's own)."""
    out = c.out0 if step == 0 else c.out1
    atol, rtol = TOL[c.kind]
    # integer outputs, bit-exact
    assert np.array_equal(g["page_table"], c.table.astype(np.int32))
    assert np.array_equal(g["slot"], out["slots"].astype(np.int32))
    written = np.zeros(g["k_bits"].shape[0], dtype=bool)
    written[out["slots"]] = True
    assert np.array_equal(g["k_bits"][~written], g["k_before"][~written]), "unwritten K rows changed"
    assert np.array_equal(g["v_bits"][~written], g["v_before"][~written]), "unwritten V rows changed"
    infos = [close(g["q"], out["q"], atol, rtol, "q_out"),
             close(g["k_cache"][out["slots"]], out["k"], atol, rtol, "K rows"),
             close(g["v_cache"][out["slots"]], out["v"], atol, rtol, "V rows"),
             close(g["o"], out["o"] if o_ref is None else o_ref, atol, rtol, "o")]
    ma, mr = MASS_TOL[c.kind]
    infos.append(close(g["mass"], out["mass"], ma, mr, "mass"))
    assert not g["mass_after"].any(), "top-k did not clear the score"
    check_topk(c, g["mass"], g["idx"], g["val"], g["cnt"], out["mass"], exact_set=exact_topk)
    for i in infos:
        log(f"   {c.wl.name} step{step} {i['what']}: max_abs={i['max_abs']:.3e} "
            f"max/rms={i['max_over_rms']:.3e} beyond 30 bf16 ulps: {i['n_over_30ulp_bf16']}")


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16", "llada_b1", "mixed_b8", "verify_b4"])
@pytest.mark.parametrize("step", [0, 1])
def test_workload_step_parity(name, step, gpu):
    log(f"[gpu] parity {name} step {step}")
    c = case(name)
    g = run_gpu_step(c, step, gpu)
    compare_step(c, g, step)


@pytest.mark.parametrize("name", ["llada_b1", "verify_b4"])
def test_heavy_hitter_topk_exact(name, gpu):
    """Planted heavy hitters (step-0 x rows scaled by 2) separate the top-k,
    so the GPU's set must equal the oracle's exactly.  Every output keeps the
    workload gate.  Scaling x by 2 scales q and k of those rows by 2 and their
    scores by 4, and the bf16 stores of q and of the cached K move a score in
    proportion to its size: o is gated against the oracle with those stores
    modelled (q, K, V rounded once to bf16 before the attention); its distance
    from the float64-stored oracle is logged."""
    log(f"[gpu] heavy-hitter top-k {name}")
    c = case(name, heavy=True)
    g = run_gpu_step(c, 0, gpu)
    atol, rtol = TOL[c.kind]
    m = measure(g["o"], c.out0["o"], atol, rtol, "o against the float64-stored oracle")
    log(f"   heavy {name} o against the float64-stored oracle: max_abs={m['max_abs']:.3e} n_bad={m['n_bad']} "
        f"worst err/limit={m['worst_ratio']:.3f}")
    m = measure(c.out0_store["o"], c.out0["o"], atol, rtol, "bf16-stored oracle vs float64-stored oracle")
    log(f"   heavy {name} oracle with bf16 stores vs without: max_abs={m['max_abs']:.3e} n_bad={m['n_bad']}")
    compare_step(c, g, 0, exact_topk=True, o_ref=c.out0_store["o"])


@pytest.mark.parametrize("name,splits", [("tiny_bf16", "2"), ("llada_b1", "1"), ("llada_b1", "3"),
                                         ("verify_b4", "1"), ("verify_b4", "5"), ("mixed_b8", "3")])
def test_attention_split_paths(name, splits, gpu):
    """Both attention paths (fused single launch, and key splits merged by a
    second launch), including uneven splits, give the same parity.  Small
    unmasked split launches run 64-row query tiles (tiny_bf16, llada_b1: 72
    rows make a full tile and an 8-row one); mixed_b8 puts sequences of 40-72
    rows and full refreshes of 512 and 1024 rows (4 and 8 query tiles of 128)
    through the merge."""
    log(f"[gpu] attention with {splits} key splits on {name}")
    from io_aware_kv_amd import dllm
    c = case(name)
    dllm.set_tuning("attn_splits", splits)
    try:
        g = run_gpu_step(c, 1, gpu)
    finally:
        dllm.set_tuning("attn_splits", None)
    compare_step(c, g, 1)


@pytest.mark.parametrize("name,kernel", [("llada_b1", "gemm"), ("mixed_b8", "tiled"), ("tiny_bf16", "gemm"),
                                         ("llada_b1", "g128x256"), ("llada_b1", "g128x256o2"),
                                         ("mixed_b8", "g64x256"), ("llada_b1", "g64x256o2"),
                                         ("mixed_b8", "g256x128"), ("mixed_b8", "g256x128o2"),
                                         ("tiny_bf16", "g128x128"), ("mixed_b8", "g128x128o2"),
                                         ("llada_b1", "mid10x6"), ("mixed_b8", "mid6x6"), ("tiny_bf16", "mid4x12"),
                                         ("llada_b1", "mid12x6"), ("mixed_b8", "mid16x6"), ("tiny_bf16", "mid8x12"),
                                         ("tiny_bf16", "mid10x6")])
def test_projection_kernel_paths(name, kernel, gpu):
    """The projection for more than 128 rows has the 128 x 128 LDS-tiled
    kernel, the whole-head GEMM in five tile shapes (256 x 256, 128 x 256,
    64 x 256, 256 x 128, 128 x 128), the smaller four alone on a compute unit
    with a deep ring or two per compute unit ("o2"), and the mid-size
    weight-streaming kernel in six shapes (16 MT rows of x by 8 NT pairs,
    "midMTxNT"); forcing one the shape would not pick gives the same parity,
    ragged row tails included (6297 rows leaves tails of 153, 25 and 25 rows
    at 256-, 64- and 128-row tiles and 57 and 153 rows at 96- and 256-row
    groups; 512 rows leaves 32 rows in the last 160-row group; tiny_bf16 is
    one row tile by three or six column tiles over a contraction of 256, and
    four or eight pair groups of the mid-size kernel, fewer stages than its
    ring holds)."""
    log(f"[gpu] projection kernel {kernel} on {name}")
    from io_aware_kv_amd import dllm
    c = case(name)
    dllm.set_tuning("qkv_kernel", kernel)
    try:
        g = run_gpu_step(c, 0, gpu)
    finally:
        dllm.set_tuning("qkv_kernel", None)
    compare_step(c, g, 0)


@pytest.mark.parametrize("name,step", [("tiny_bf16", 1), ("llada_b1", 1), ("verify_b4", 1), ("mixed_b8", 0)])
def test_separate_slot_mapping_path(name, step, gpu):
    """dllm_map_slots followed by dllm_qkv_rope_cachewrite (slots as an
    input) gives the same parity as the one-call paged entry point the other
    tests use (which maps the slots inside the cache-phase projection kernel,
    and as a launch of its own for larger row counts)."""
    log(f"[gpu] separate slot mapping {name} step {step}")
    c = case(name)
    g = run_gpu_step(c, step, gpu, fused_slots=False)
    compare_step(c, g, step)


@pytest.mark.parametrize("name,step", [("tiny_bf16", 0), ("tiny_bf16", 1), ("llada_b1", 0), ("llada_b1", 1),
                                       ("verify_b4", 1), ("mixed_b8", 0)])
def test_unfused_arm_parity(name, step, gpu):
    """The unfused comparison arm (projection to memory, rotary, cache write as
    launches of their own) meets the same gates as the fused call: q and K/V
    are rounded to bf16 twice instead of once, well inside the bf16 tolerance.
    The row counts cover the weight-streaming (72, 88), mid-size (256, 288,
    512) and 256 x 256 GEMM (6297) projection kernels."""
    log(f"[gpu] unfused arm {name} step {step}")
    c = case(name)
    g = run_gpu_step(c, step, gpu, unfused=True)
    compare_step(c, g, step)


@pytest.mark.parametrize("name", ["llada_b1", "mixed_b8", "tiny_f32"])
def test_score_overwrite(name, gpu):
    """mass_overwrite stores the layer's term instead of adding it: from a
    score buffer full of a sentinel, the step's score equals the oracle's term
    for keys below each sequence's kv_len (the split merge launch, the fused
    score pass and the fp32 kernel), and the sentinel stays past kv_len."""
    import torch
    from io_aware_kv_amd.runner import FlashCacheRunner
    c = case(name)
    wl = c.wl
    log(f"[gpu] score overwrite {name}")
    run = FlashCacheRunner(wl, device=gpu, layers=1)
    run.k_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.k1_in)))
    run.v_cache[0].copy_(run.to_device_array(c.to_cache_raw(c.v1_in)))
    run.mass.fill_(5.0)
    st = run.upload_step(c.rows1)
    run.layer_step(st, run.to_device_array(c.x1_raw), run.to_device_array(c.w_raw), 0, mass_overwrite=True)
    torch.cuda.synchronize()
    m = run.mass.cpu().numpy()
    kv = c.rows1.kv_len
    ma, mr = MASS_TOL[c.kind]
    for b in range(wl.n_seq):
        k = min(int(kv[b]), run.n_cap)
        close(head_sum(m[b:b + 1, :, :k])[0], c.out1["mass"][b, :k], ma, mr, f"{name} seq {b} score")
        assert np.all(m[b, :, k:] == 5.0)
