"""Full-size parity of the 32-layer LLaDA-8B-shaped workload (batch 32,
context 2048): a full-refresh step (65536 rows per layer) and a cache-phase
step (2304 rows per layer), every layer adding its formula (2) term to the
score and one top-k after the last layer.

The GPU runs every layer, sequence and head at full size.  The oracle checks
a seeded sample:
  * cache phase: all 32 layers for the sequences in SEQS, every head: q, the
    written K/V rows, o and each layer's per-head score term, then those
    sequences' top-k against the oracle's score summed over the 32 layers;
  * full refresh: the layers in FULL_LAYERS for the sequences in SEQS, every
    head (q, K/V rows, o, score terms).
The top-k selection of every sequence is also checked exactly on the GPU's
own scores.  Sequences are independent in these kernels, so the oracle runs
one sequence's rows over its own keys (an identity page table in logical
order), with the full W of the layer.

Per-step isolation without a 32-layer full-refresh oracle: before the
cache-phase step, each layer's caches are filled with seeded bf16 values
(io_aware_kv_amd.workloads.device_cache_fill); the oracle starts from the
same values.  The cache-phase row set is a seeded draw (it must not depend on
either side's top-k).  Oracle time: about 64 x 0.6 s for the cache phase and
4 x 11 s for the full refresh on 8 cores.
"""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W
from parity import MASS_TOL, TOL, close, log
from test_gpu_parity import head_sum

pytestmark = pytest.mark.gpu

SEQS = (3, 20)            # sampled sequences
FULL_LAYERS = (0, 31)     # full-refresh layers compared with the oracle
CHUNKS = 4                # the 32 cache-phase layers are compared in 4 tests of 8
P = W.PAGE


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(t):
    return W.bf16_bits_to_f64(_bits(t))


class B32:
    """The workload, its runner, and the oracle's page table (slots are
    addressed with the oracle's table; the GPU's table is compared with it)."""

    def __init__(self, gpu):
        from io_aware_kv_amd.runner import FlashCacheRunner
        self.wl = wl = W.make_workload("llada_b32")
        self.run = FlashCacheRunner(wl, device=gpu)
        self.gpu = gpu
        self.table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
        sh = wl.shape
        self.H, self.D, self.n = sh.n_heads, sh.head_dim, sh.n_heads * sh.head_dim
        log(f"[gpu] llada_b32: {self.run.layers} layers, caches "
            f"{2 * self.run.layers * self.run.k_cache[0].numel() * 2 / 2**30:.1f} GiB")

    def slots(self, b, positions):
        positions = np.asarray(positions, dtype=np.int64)
        return self.table[b, positions // P] * P + positions % P

    def weights64(self, layer):
        return _f64(W.device_weights(self.wl, layer, self.gpu))


@pytest.fixture(scope="module")
def b32(gpu):
    t = B32(gpu)
    assert np.array_equal(t.run.page_table.cpu().numpy().reshape(t.wl.n_seq, t.wl.max_pages),
                          t.table.astype(np.int32))
    return t


def _run_step(t, rows, step, seeded_cache):
    """All 32 layers of one step on the GPU; returns, per layer, the sampled
    sequences' outputs and per-head score terms, plus the final score and
    top-k of every sequence."""
    import torch
    run, wl = t.run, t.wl
    st = run.upload_step(rows)
    run.map_slots(st)
    run.mass.zero_()
    out = {"layers": {}}
    for l in range(run.layers):
        if seeded_cache:
            run.k_cache[l].copy_(W.device_cache_fill(wl, l, 0, t.gpu))
            run.v_cache[l].copy_(W.device_cache_fill(wl, l, 1, t.gpu))
        before = run.mass.clone()
        x = W.device_activations(wl, rows, step, l, t.gpu)
        run.cache_update(st, x, W.device_weights(wl, l, t.gpu), l)
        # the first layer stores its term (the product's mode), later layers add
        run.attention(st, l, mass_overwrite=l == 0)
        keep = seeded_cache or l in FULL_LAYERS
        if not keep:
            continue
        torch.cuda.synchronize()
        term = (run.mass - before).cpu().numpy()
        rec = {}
        for b in SEQS:
            r0, r1 = int(rows.cu_q[b]), int(rows.cu_q[b + 1])
            kv = int(rows.kv_len[b])
            sl = torch.from_numpy(t.slots(b, rows.logical[r0:r1])).to(t.gpu)
            rec[b] = {"x": _bits(x[r0:r1]), "q": _bits(st.q[r0:r1]), "o": _bits(st.o[r0:r1]),
                      "k": _bits(run.k_cache[l][sl]), "v": _bits(run.v_cache[l][sl]),
                      "term": term[b, :, :kv].copy()}
        out["layers"][l] = rec
        del x
    torch.cuda.synchronize()
    out["slot"] = st.slot.cpu().numpy()
    out["score"] = head_sum(run.mass.cpu().numpy())
    run.topk(clear_mass=True)
    out["idx"] = run.top_idx.cpu().numpy()
    out["cnt"] = run.top_cnt.cpu().numpy()
    out["rows"] = rows
    log(f"[gpu] llada_b32 step {step}: {rows.n_rows} rows per layer, 32 layers done")
    return out


@pytest.fixture(scope="module")
def full_step(b32):
    return _run_step(b32, W.full_refresh_rows(b32.wl), 0, seeded_cache=False)


@pytest.fixture(scope="module")
def cache_step(b32, full_step):
    # runs after the full refresh (whose outputs are already on the host)
    rows = W.config_step_rows(b32.wl, W.seeded_tracked(b32.wl, 1))
    return _run_step(b32, rows, 1, seeded_cache=True)


_ORACLE_TERMS = {}


def _check_layer(t, res, l, b, k_prev, v_prev, w64, tag):
    """One (layer, sequence) against the oracle, every head; returns the
    oracle's formula (2) term of the sequence for this layer."""
    H, D, n = t.H, t.D, t.n
    rows = res["rows"]
    r0, r1 = int(rows.cu_q[b]), int(rows.cu_q[b + 1])
    kv = int(rows.kv_len[b])
    g = res["layers"][l][b]
    pages = (kv + P - 1) // P
    table = O.build_block_table([pages], list(range(pages)), pages, pages)
    out = O.layer_step(W.bf16_bits_to_f64(g["x"]), w64, rows.pos[r0:r1], rows.logical[r0:r1],
                       [0, r1 - r0], [kv], [int(rows.mass_count[b])], k_prev, v_prev, table, H, D,
                       t.wl.shape.rope_base, P)
    atol, rtol = TOL["bf16"]
    ma, mr = MASS_TOL["bf16"]
    infos = [close(W.bf16_bits_to_f64(g["q"]), out["q"], atol, rtol, tag + " q"),
             close(W.bf16_bits_to_f64(g["k"]), out["k"], atol, rtol, tag + " K rows"),
             close(W.bf16_bits_to_f64(g["v"]), out["v"], atol, rtol, tag + " V rows"),
             close(W.bf16_bits_to_f64(g["o"]), out["o"], atol, rtol, tag + " o")]
    # per-head terms: the GPU's carry 1/(H |M|) each; the oracle's column mass
    # sums the heads, so take each head's window-row probabilities directly
    m = int(rows.mass_count[b])
    probs = out["probs"][0]
    want = probs[:, :m, :].sum(axis=1) / (H * m)
    infos.append(close(g["term"], want, ma, mr, tag + " per-head score term"))
    log(f"   {tag}: " + ", ".join(f"{i['what'].split()[-1] if 'term' not in i['what'] else 'term'} "
                                  f"{i['max_abs']:.1e}" for i in infos))
    return out["mass"][0, :kv]


@pytest.mark.parametrize("layer", FULL_LAYERS)
def test_llada_b32_full_refresh(b32, full_step, layer):
    """Full refresh: every position of every sequence queried and written;
    the sampled layers and sequences against the oracle, every head."""
    res = full_step
    w64 = b32.weights64(layer)
    for b in SEQS:
        kv = int(res["rows"].kv_len[b])
        zeros = np.zeros((kv, b32.n))       # every key is rewritten by this step
        _check_layer(b32, res, layer, b, zeros, zeros, w64, f"llada_b32 full layer{layer} seq{b}")
    if layer == FULL_LAYERS[0]:
        # slots of the whole step, bit-exact
        want = O.row_slots(b32.table, res["rows"].cu_q, res["rows"].logical, P)
        assert np.array_equal(res["slot"], want.astype(np.int32))
        # the selection on the GPU's own scores, every sequence
        o_idx, _, o_cnt = O.topk(res["score"].astype(np.float64), b32.wl.eligible().astype(bool),
                                 b32.wl.shape.top_k)
        assert np.array_equal(res["idx"], o_idx) and np.array_equal(res["cnt"], o_cnt)


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_llada_b32_cache_phase_layers(b32, cache_step, chunk):
    """Cache phase from seeded caches: layers 8c .. 8c+7, the sampled
    sequences, every head."""
    import torch
    res = cache_step
    rows = res["rows"]
    L = b32.run.layers
    per = L // CHUNKS
    for l in range(chunk * per, (chunk + 1) * per):
        w64 = b32.weights64(l)
        kc = W.device_cache_fill(b32.wl, l, 0, b32.gpu)
        vc = W.device_cache_fill(b32.wl, l, 1, b32.gpu)
        for b in SEQS:
            kv = int(rows.kv_len[b])
            sl = torch.from_numpy(b32.slots(b, np.arange(kv))).to(b32.gpu)
            k_prev = _f64(kc[sl])
            v_prev = _f64(vc[sl])
            _ORACLE_TERMS[(l, b)] = _check_layer(b32, res, l, b, k_prev, v_prev, w64,
                                                 f"llada_b32 cache layer{l} seq{b}")
        del kc, vc


def test_llada_b32_cache_phase_topk(b32, cache_step):
    """After the 32 layers: the selection on the GPU's own scores equals the
    oracle's rule exactly for every sequence; for the sampled sequences the
    GPU's summed score matches the oracle's sum over the 32 layers, and the
    selected set agrees outside the tie window around the k-th score."""
    import torch
    res = cache_step
    rows = res["rows"]
    wl = b32.wl
    k = wl.shape.top_k
    elig = wl.eligible().astype(bool)
    o_idx, _, o_cnt = O.topk(res["score"].astype(np.float64), elig, k)
    assert np.array_equal(res["idx"], o_idx) and np.array_equal(res["cnt"], o_cnt)
    ma, mr = MASS_TOL["bf16"]
    for b in SEQS:
        kv = int(rows.kv_len[b])
        total = np.zeros(wl.n_cap)
        for l in range(b32.run.layers):
            if (l, b) not in _ORACLE_TERMS:       # the layer test did not run: compute it here
                kc = W.device_cache_fill(wl, l, 0, b32.gpu)
                vc = W.device_cache_fill(wl, l, 1, b32.gpu)
                sl = torch.from_numpy(b32.slots(b, np.arange(kv))).to(b32.gpu)
                _ORACLE_TERMS[(l, b)] = _check_layer(b32, res, l, b, _f64(kc[sl]), _f64(vc[sl]),
                                                     b32.weights64(l), f"llada_b32 cache layer{l} seq{b}")
            total[:kv] += _ORACLE_TERMS[(l, b)]
        close(res["score"][b, :kv], total[:kv], ma, mr, f"llada_b32 seq{b} 32-layer score")
        r_idx, _, r_cnt = O.topk(total[None, :], elig[b:b + 1], k)
        n = int(r_cnt[0])
        assert int(res["cnt"][b]) == n
        sel = set(res["idx"][b, :n].tolist())
        ak = total[r_idx[0, n - 1]]
        win = max(1e-3 * ak, ma + mr * ak)
        for i in np.flatnonzero(elig[b]):
            if total[i] > ak + win:
                assert i in sel, (b, i, total[i], ak)
            elif total[i] < ak - win:
                assert i not in sel, (b, i, total[i], ak)
        log(f"   llada_b32 seq{b}: top-{k} agrees with the oracle's 32-layer score "
            f"(k-th {ak:.4e}, {len(sel ^ set(r_idx[0, :n].tolist())) // 2} swaps inside the tie window)")
