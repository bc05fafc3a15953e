"""Pins of the CPU oracle against closed forms, invariants and brute force.

Each test ties one oracle function to something other than itself, chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a wrong normaliser) fails at least one of them.  Pages cited:
  [FD]  "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
        Memory-Efficient Diffusion LLMs" (paper summary page)
  [AIP] "Flash-dLLM 是什麼？擴散語言模型推論快 11 倍" (aiposthub explainer)
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W

P = 16


# ---------------------------------------------------------------------------
# a0: block table, slots
# ---------------------------------------------------------------------------

def _inverse(table):
    inv = {}
    for b in range(table.shape[0]):
        for j in range(table.shape[1]):
            if table[b, j] >= 0:
                assert table[b, j] not in inv
                inv[int(table[b, j])] = (b, j)
    return inv


def test_block_table_identity_perm_is_consecutive():
    # closed form: with the identity permutation, sequence b owns pages
    # off_b .. off_b + n_b - 1 in order
    t = O.build_block_table([3, 0, 2], list(range(6)), 6, 4)
    assert t.tolist() == [[0, 1, 2, -1], [-1, -1, -1, -1], [3, 4, -1, -1]]


def test_block_table_bijection_and_round_trip_exhaustive():
    # brute force over every permutation of a 5-page pool and several splits
    for perm in itertools.permutations(range(5)):
        for split in ([5], [2, 3], [1, 1, 2], [0, 4], [2, 2]):
            t = O.build_block_table(split, perm, 5, 5)
            inv = _inverse(t)
            assert len(inv) == sum(split)                    # pages used once each
            assert all(0 <= p < 5 for p in inv)
            for b, n in enumerate(split):
                assert (t[b, :n] >= 0).all() and (t[b, n:] == -1).all()
            # slot -> (page, offset) -> (sequence, logical page) -> logical position
            cu = np.cumsum([0] + [n * P for n in split])
            logical = np.concatenate([np.arange(n * P) for n in split]).astype(int)
            slots = O.row_slots(t, cu, logical, P)
            for b in range(len(split)):
                for r in range(cu[b], cu[b + 1]):
                    page, off = divmod(int(slots[r]), P)
                    bb, j = inv[page]
                    assert bb == b and j * P + off == logical[r]


@pytest.mark.parametrize("args", [
    ([3, 3], list(range(5)), 5, 3),          # more pages than the pool
    ([2], [0, 0, 1], 3, 2),                  # not a permutation
    ([2], [0, 1], 3, 2),                     # permutation of the wrong size
    ([4], list(range(4)), 4, 3),             # exceeds max_pages
    ([-1], list(range(4)), 4, 3),            # negative count
])
def test_block_table_rejects(args):
    with pytest.raises(O.OracleError):
        O.build_block_table(*args)


def test_slots_reject_range_and_duplicates():
    t = O.build_block_table([1, 1], [1, 0], 2, 2)
    with pytest.raises(O.OracleError):
        O.row_slots(t, [0, 1, 2], [16, 0], P)          # beyond sequence 0's page
    with pytest.raises(O.OracleError):
        O.row_slots(t, [0, 2, 2], [3, 3], P)           # one slot twice
    with pytest.raises(O.OracleError):
        O.row_slots(t, [0, 1, 1], [-1], P)
    assert O.row_slots(t, [0, 1, 2], [5, 5], P).tolist() == [1 * P + 5, 0 * P + 5]


# ---------------------------------------------------------------------------
# a1: projection
# ---------------------------------------------------------------------------

def test_projection_small_integers_hand_computed():
    x = np.array([[1.0, 2.0]])
    w = np.array([[1, 0], [0, 1],       # Q = x
                  [1, 1], [2, 0],       # K = (x0 + x1, 2 x0)
                  [0, 3], [1, -1]],     # V = (3 x1, x0 - x1)
                 dtype=float)
    q, k, v = O.project(x, w, 2)
    assert q.tolist() == [[1.0, 2.0]]
    assert k.tolist() == [[3.0, 2.0]]
    assert v.tolist() == [[6.0, -1.0]]


def test_projection_stacked_identity_and_block_order():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 8))
    eye = np.eye(8)
    q, k, v = O.project(x, np.vstack([eye, eye, eye]), 8)
    assert np.array_equal(q, x) and np.array_equal(k, x) and np.array_equal(v, x)
    z = np.zeros((8, 8))
    q, k, v = O.project(x, np.vstack([z, eye, z]), 8)
    assert not q.any() and np.array_equal(k, x) and not v.any()


def test_projection_brute_force_and_linearity():
    rng = np.random.default_rng(1)
    x1, x2 = rng.standard_normal((2, 3, 4))
    w = rng.standard_normal((3 * 2, 4))
    q, k, v = O.project(x1, w, 2)
    qkv = np.hstack([q, k, v])
    for r in range(3):
        for n in range(6):
            assert math.isclose(qkv[r, n], math.fsum(x1[r, c] * w[n, c] for c in range(4)),
                                rel_tol=1e-13, abs_tol=1e-13)
    a = np.hstack(O.project(2.0 * x1 - 3.0 * x2, w, 2))
    b = 2.0 * np.hstack(O.project(x1, w, 2)) - 3.0 * np.hstack(O.project(x2, w, 2))
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# a2: rotary embedding (rotate-half)
# ---------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    t = np.random.default_rng(2).standard_normal((3, 2, 8))
    assert np.array_equal(O.rope(t, [0, 0, 0], 1e4), t)


def test_rope_probe_distinguishes_rotate_half():
    # e_0 at position m: theta_0 = 1, so out[0] = cos m and out[D/2] = sin m;
    # an interleaved form would put sin m at index 1 instead.
    D = 8
    for m in (1, 5, 37):
        e0 = np.zeros((1, 1, D)); e0[0, 0, 0] = 1.0
        out = O.rope(e0, [m], 5e5)[0, 0]
        want = np.zeros(D); want[0] = math.cos(m); want[D // 2] = math.sin(m)
        assert np.allclose(out, want, atol=1e-15)
        # the partner: e_{D/2} goes to (-sin m) at 0 and cos m at D/2
        eh = np.zeros((1, 1, D)); eh[0, 0, D // 2] = 1.0
        out = O.rope(eh, [m], 5e5)[0, 0]
        want = np.zeros(D); want[0] = -math.sin(m); want[D // 2] = math.cos(m)
        assert np.allclose(out, want, atol=1e-15)


def test_rope_frequency_value():
    # theta_1 for base 1e4 and D = 64 is 10^(-1/8) = 0.74989420933245582...
    D = 64
    e1 = np.zeros((1, 1, D)); e1[0, 0, 1] = 1.0
    out = O.rope(e1, [1], 1e4)[0, 0]
    assert math.isclose(out[1], math.cos(0.7498942093324558), abs_tol=1e-14)
    assert math.isclose(out[1 + D // 2], math.sin(0.7498942093324558), abs_tol=1e-14)


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(3)
    t = rng.standard_normal((4, 3, 16))
    pos = [0, 7, 300, 2047]
    out = O.rope(t, pos, 5e5)
    n_in = t[..., :8] ** 2 + t[..., 8:] ** 2
    n_out = out[..., :8] ** 2 + out[..., 8:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)
    # rotating by a then by b equals rotating by a + b
    two = O.rope(O.rope(t, [3, 4, 5, 6], 1e4), [10, 20, 30, 40], 1e4)
    one = O.rope(t, [13, 24, 35, 46], 1e4)
    assert np.allclose(two, one, rtol=1e-12, atol=1e-12)


def test_rope_dot_depends_only_on_offset():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    def dot(m, n):
        return float(np.sum(O.rope(q, [m], 5e5) * O.rope(k, [n], 5e5)))
    for m, n, shift in ((5, 2, 100), (0, 511, 1000), (2047, 1500, -1400)):
        a, b = dot(m, n), dot(m + shift, n + shift)
        assert math.isclose(a, b, rel_tol=1e-10, abs_tol=1e-10)
    assert not math.isclose(dot(5, 2), dot(5, 3), rel_tol=1e-6)


# ---------------------------------------------------------------------------
# a3: cache write
# ---------------------------------------------------------------------------

def test_scatter_touches_only_its_slots():
    cache = np.random.default_rng(5).standard_normal((32, 4))
    rows = np.arange(8.0).reshape(2, 4)
    out = O.scatter(cache, [17, 3], rows)
    assert np.array_equal(out[17], rows[0]) and np.array_equal(out[3], rows[1])
    keep = [i for i in range(32) if i not in (3, 17)]
    assert np.array_equal(out[keep], cache[keep])


# ---------------------------------------------------------------------------
# a4: attention
# ---------------------------------------------------------------------------

def _one_seq_cache(kv, H, D, rng, pages=None):
    npg = -(-kv // P) if pages is None else pages
    table = O.build_block_table([npg], list(range(npg)), npg, npg)
    K = rng.standard_normal((npg * P, H * D))
    V = rng.standard_normal((npg * P, H * D))
    return table, K, V


def test_attention_hand_computed_probabilities():
    # D = 4, so scores are q.k / 2.  Head 0 row 0 scores (0, ln 2, ln 3) give
    # probabilities (1, 2, 3)/6; head 0 row 1 has q = 0 (uniform); head 1 row 0
    # scores (0, ln 4, 0) give (1, 4, 1)/6.
    H, D, kv = 2, 4, 3
    table = O.build_block_table([1], [0], 1, 1)
    K = np.zeros((P, H * D)); V = np.zeros((P, H * D))
    K[1, 0] = 1.0; K[2, 1] = 1.0               # head 0 keys: 0, e0, e1
    K[1, D + 0] = 1.0                           # head 1 keys: 0, e0, 0
    V[0, 0], V[1, 1], V[2, 2] = 6.0, 6.0, 6.0   # head 0 values 6 e_j
    V[0:3, D + 3] = [1.0, 2.0, 3.0]             # head 1 values j + 1 in the last dim
    q = np.zeros((2, H * D))
    q[0, 0], q[0, 1] = 2 * math.log(2), 2 * math.log(3)
    q[0, D + 0] = 2 * math.log(4)
    o, probs = O.attention(q, K, V, table, [0, 2], [kv], H, D, P)
    p = probs[0]
    assert np.allclose(p[0, 0], np.array([1, 2, 3]) / 6, rtol=1e-14)
    assert np.allclose(p[0, 1], np.ones(3) / 3, rtol=1e-14)
    assert np.allclose(p[1, 0], np.array([1, 4, 1]) / 6, rtol=1e-14)
    assert np.allclose(o[0, :D], [1, 2, 3, 0], rtol=1e-14, atol=1e-14)
    assert math.isclose(o[0, D + 3], (1 + 8 + 3) / 6, rel_tol=1e-14)


def test_attention_constant_values_and_single_key():
    rng = np.random.default_rng(6)
    H, D, kv = 3, 8, 40
    table, K, V = _one_seq_cache(kv, H, D, rng)
    q = rng.standard_normal((5, H * D)) * 3
    Vc = np.tile(np.arange(H * D, dtype=float), (V.shape[0], 1))
    vis = [rng.random((5, kv)) < 0.5]
    vis[0][:, 0] = True
    for v_ in (None, vis):
        o, _ = O.attention(q, K, Vc, table, [0, 5], [kv], H, D, P, v_)
        assert np.allclose(o, np.tile(np.arange(H * D, dtype=float), (5, 1)), rtol=1e-13)
    one = [np.zeros((5, kv), dtype=bool)]
    one[0][np.arange(5), [3, 9, 0, 39, 17]] = True
    o, _ = O.attention(q, K, V, table, [0, 5], [kv], H, D, P, one)
    assert np.allclose(o, V[[3, 9, 0, 39, 17]], rtol=1e-14)


def test_attention_zero_query_is_mean_and_dark_row_is_zero():
    rng = np.random.default_rng(7)
    H, D, kv = 2, 8, 33
    table, K, V = _one_seq_cache(kv, H, D, rng)
    q = np.zeros((2, H * D))
    vis = [np.ones((2, kv), dtype=bool)]
    vis[0][1, :] = False
    o, probs = O.attention(q, K, V, table, [0, 2], [kv], H, D, P, vis)
    assert np.allclose(o[0], V[:kv].mean(axis=0), rtol=1e-13)
    assert not o[1].any() and not probs[0][:, 1].any()


def test_attention_empty_key_and_row_sets():
    # a sequence with no keys: each of its rows sees no key (o = 0, no
    # probabilities); a sequence with no rows contributes nothing; the other
    # sequences of the batch are unaffected
    rng = np.random.default_rng(8)
    H, D = 2, 8
    table = np.array([[0, -1], [1, 2], [-1, -1]], dtype=np.int32)
    K = rng.standard_normal((3 * P, H * D))
    V = rng.standard_normal((3 * P, H * D))
    q = rng.standard_normal((5, H * D))
    cu, kv = [0, 0, 3, 5], [16, 20, 0]                     # no rows / three rows / two rows, no keys
    o, probs = O.attention(q, K, V, table, cu, kv, H, D, P)
    assert [p.shape for p in probs] == [(H, 0, 16), (H, 3, 20), (H, 2, 0)]
    assert not o[3:].any()
    o1, _ = O.attention(q[:3], K, V, table[1:2], [0, 3], [20], H, D, P)
    assert np.array_equal(o[:3], o1)
    m = O.column_mass(probs, [0, 3, 0], 20)
    assert not m[0].any() and not m[2].any() and abs(m[1].sum() - 1.0) < 1e-12


def _tiled_online_softmax(q, K, V, tile):
    """Test-local flash-style recurrence: running max, running sum, rescaled
    accumulator, over key tiles.  Must equal the dense oracle."""
    m = np.full(q.shape[0], -np.inf)
    l = np.zeros(q.shape[0])
    acc = np.zeros((q.shape[0], V.shape[1]))
    for t0 in range(0, K.shape[0], tile):
        s = q @ K[t0:t0 + tile].T
        m_new = np.maximum(m, s.max(axis=1))
        scale = np.exp(m - m_new)
        p = np.exp(s - m_new[:, None])
        l = l * scale + p.sum(axis=1)
        acc = acc * scale[:, None] + p @ V[t0:t0 + tile]
        m = m_new
    return acc / l[:, None]


def test_attention_equals_tiled_online_softmax():
    rng = np.random.default_rng(8)
    H, D, kv = 2, 16, 70
    table, K, V = _one_seq_cache(kv, H, D, rng)
    q = rng.standard_normal((6, H * D)) * 2
    o, _ = O.attention(q, K, V, table, [0, 6], [kv], H, D, P)
    for h in range(H):
        sl = slice(h * D, (h + 1) * D)
        ref = _tiled_online_softmax(q[:, sl] / math.sqrt(D), K[:kv, sl], V[:kv, sl], 16)
        assert np.allclose(o[:, sl], ref, rtol=1e-12, atol=1e-13)


def test_attention_page_permutation_and_poison_invariance():
    rng = np.random.default_rng(9)
    H, D, kv, npg = 2, 8, 50, 4
    Kl = rng.standard_normal((kv, H * D))
    Vl = rng.standard_normal((kv, H * D))
    q = rng.standard_normal((3, H * D))
    vis = [rng.random((3, kv)) < 0.7]
    outs = []
    for perm in ([0, 1, 2, 3], [3, 1, 0, 2], [2, 3, 1, 0]):
        table = O.build_block_table([npg], perm, npg, npg)
        K = np.full((npg * P, H * D), 1e4)       # poison everywhere first
        V = np.full((npg * P, H * D), -1e4)
        for j in range(kv):
            s = table[0, j // P] * P + j % P
            K[s], V[s] = Kl[j], Vl[j]
        outs.append(O.attention(q, K, V, table, [0, 3], [kv], H, D, P, vis)[0])
        # hidden keys poisoned with +-1e4 must not matter
        K2, V2 = K.copy(), V.copy()
        for j in range(kv):
            if not vis[0][:, j].any():
                s = table[0, j // P] * P + j % P
                K2[s], V2[s] = 1e4, -1e4
        assert np.allclose(O.attention(q, K2, V2, table, [0, 3], [kv], H, D, P, vis)[0],
                           outs[-1], rtol=1e-13)
    assert np.allclose(outs[0], outs[1], rtol=1e-13) and np.allclose(outs[0], outs[2], rtol=1e-13)


# ---------------------------------------------------------------------------
# a5: formula (2) column mass
# ---------------------------------------------------------------------------

def test_column_mass_hand_computed():
    # same probabilities as test_attention_hand_computed_probabilities
    p = np.zeros((2, 2, 3))
    p[0, 0] = np.array([1, 2, 3]) / 6
    p[0, 1] = np.ones(3) / 3
    p[1, 0] = np.array([1, 4, 1]) / 6
    p[1, 1] = np.array([2, 1, 3]) / 6
    m1 = O.column_mass([p], [1], 4)[0]          # only row 0 is a mask row
    assert np.allclose(m1, [1 / 6, 1 / 2, 1 / 3, 0], rtol=1e-14)
    m2 = O.column_mass([p], [2], 4)[0]
    want = (p[0, 0] + p[0, 1] + p[1, 0] + p[1, 1]) / 4
    assert np.allclose(m2[:3], want, rtol=1e-14) and m2[3] == 0
    assert not O.column_mass([p], [0], 4).any()
    # a score narrower than the keys keeps the first n_cap entries (hand values)
    assert np.allclose(O.column_mass([p], [1], 2)[0], [1 / 6, 1 / 2], rtol=1e-14)


def test_column_mass_sums_to_one_and_uniform_for_zero_queries():
    rng = np.random.default_rng(10)
    H, D, kv = 4, 8, 45
    table, K, V = _one_seq_cache(kv, H, D, rng)
    q = rng.standard_normal((7, H * D))
    _, probs = O.attention(q, K, V, table, [0, 7], [kv], H, D, P)
    m = O.column_mass(probs, [5], table.shape[1] * P)[0]
    assert math.isclose(m.sum(), 1.0, rel_tol=1e-13)
    q[:3] = 0.0
    _, probs = O.attention(q, K, V, table, [0, 7], [kv], H, D, P)
    m = O.column_mass(probs, [3], table.shape[1] * P)[0]
    assert np.allclose(m[:kv], 1.0 / kv, rtol=1e-13) and not m[kv:].any()
    # one mass row and one head: the row's own softmax
    _, probs = O.attention(q[3:4, :D], K[:, :D], V[:, :D], table, [0, 1], [kv], 1, D, P)
    m = O.column_mass(probs, [1], table.shape[1] * P)[0]
    s = q[3, :D] @ K[:kv, :D].T / math.sqrt(D)
    e = np.exp(s - s.max())
    assert np.allclose(m[:kv], e / e.sum(), rtol=1e-13)


# ---------------------------------------------------------------------------
# a6: top-k
# ---------------------------------------------------------------------------

def _check_topk(mass, elig, k, idx, val, cnt):
    for b in range(mass.shape[0]):
        cand = np.flatnonzero(elig[b])
        n = min(k, len(cand))
        assert cnt[b] == n
        sel = idx[b, :n]
        assert (idx[b, n:] == -1).all() and len(set(sel.tolist())) == n
        assert all(elig[b, i] for i in sel)
        assert np.array_equal(val[b, :n], mass[b, sel])
        assert all(val[b, j] >= val[b, j + 1] for j in range(n - 1))
        rest = [i for i in cand if i not in set(sel.tolist())]
        if rest and n:
            worst = mass[b, sel].min()
            assert max(mass[b, rest]) <= worst
            # ties at the boundary go to the lower position
            tied_out = [i for i in rest if mass[b, i] == worst]
            tied_in = [i for i in sel if mass[b, i] == worst]
            assert not tied_out or max(tied_in) < min(tied_out)


def test_topk_brute_force_small():
    rng = np.random.default_rng(11)
    for trial in range(200):
        B, N = 2, int(rng.integers(1, 12))
        mass = rng.integers(0, 4, size=(B, N)).astype(float)   # many ties
        elig = rng.random((B, N)) < 0.7
        k = int(rng.integers(1, 8))
        idx, val, cnt = O.topk(mass, elig, k)
        _check_topk(mass, elig, k, idx, val, cnt)
        # brute force: the chosen set has the largest score sum of all
        # size-n subsets, and is the lexicographically smallest such set
        for b in range(B):
            cand = list(np.flatnonzero(elig[b]))
            n = int(cnt[b])
            best = max(sum(mass[b, list(c)]) for c in itertools.combinations(cand, n)) if n else 0
            assert sum(mass[b, idx[b, :n]]) == best
            tops = sorted(c for c in itertools.combinations(cand, n)
                          if sum(mass[b, list(c)]) == best)
            assert sorted(idx[b, :n].tolist()) == list(tops[0])


def test_topk_planted_and_short():
    mass = np.zeros((1, 64)); elig = np.ones((1, 64), dtype=bool)
    planted = [50, 3, 17, 41]
    for r, i in enumerate(planted):
        mass[0, i] = 10.0 - r
    idx, val, cnt = O.topk(mass, elig, 4)
    assert idx[0].tolist() == planted and cnt[0] == 4
    elig[0, 5:] = False
    idx, val, cnt = O.topk(mass, elig, 8)
    assert idx[0].tolist() == [3, 0, 1, 2, 4, -1, -1, -1] and cnt[0] == 5


# ---------------------------------------------------------------------------
# verify-step visibility ([FD] 方法步骤详情 step 3, [AIP] Flash-Verify section)
# ---------------------------------------------------------------------------

def test_verify_visibility_brute_force_rules():
    wl = W.make_workload("verify_b4")
    s = wl.seqs[0]
    vis = W.verify_visibility(s, 40)
    m, ctx = 16, s.ctx
    for r in range(vis.shape[0]):
        for j in range(vis.shape[1]):
            if j < ctx:
                want = j not in set(s.search.tolist())
            elif r < m:                                   # mask view r
                k = j - ctx
                want = (k < m and k < r) or (k >= m and k - m == r)
            elif r < 2 * m:                               # draft view r - m
                k = j - ctx
                want = k < m and k <= r - m
            else:
                want = False
            assert vis[r, j] == want, (r, j)


def test_verify_mask_view_ignores_own_and_later_drafts():
    # perturbing the draft rows of search tokens i..m-1 leaves mask view i's
    # output unchanged (exactly), and perturbing an earlier draft changes it
    wl = W.make_workload("verify_b4")
    s = wl.seqs[0]
    rng = np.random.default_rng(12)
    H, D = 2, 8
    n_tv = 4
    tv = np.array([int(s.window[0]) if int(s.window[0]) not in s.search else 0, 5, 100, 800])
    m = 16
    rows = 2 * m + n_tv
    kv = s.ctx + 2 * m
    vis = [W.verify_visibility(s, n_tv)]
    npg = -(-kv // P)
    table = O.build_block_table([npg], list(range(npg)), npg, npg)
    w = rng.standard_normal((3 * H * D, 32)) / 6
    base_x = rng.standard_normal((rows, 32))
    logical = np.concatenate([np.arange(s.ctx + m, s.ctx + 2 * m), np.arange(s.ctx, s.ctx + m), tv])
    pos = np.concatenate([s.search, s.search, tv])
    K0 = rng.standard_normal((npg * P, H * D))
    V0 = rng.standard_normal((npg * P, H * D))

    def run(x):
        return O.layer_step(x, w, pos, logical, [0, rows], [kv], [m], K0, V0, table,
                            H, D, 5e5, P, vis)["o"]
    ref = run(base_x)
    for i in (0, 7, 15):
        x = base_x.copy()
        x[m + i:2 * m] += rng.standard_normal((m - i, 32))   # drafts i..m-1
        got = run(x)
        assert np.array_equal(got[i], ref[i])
        if i > 0:
            x = base_x.copy()
            x[m + i - 1] += 1.0                                 # draft i-1
            assert not np.allclose(run(x)[i], ref[i])


def test_layer_range_score_sums_only_its_layers():
    """Formula (2) over layers first..last: the full range is the plain sum of
    every term; a term outside the range changes nothing; the score is linear
    in the terms; a one-layer range is that layer's term."""
    rng = np.random.default_rng(41)
    L = 32
    terms = [rng.random((3, 40)) for _ in range(L)]
    full = O.layer_range_score(terms, 1, L)
    np.testing.assert_allclose(full, np.sum(terms, axis=0), rtol=1e-13)
    mid = O.layer_range_score(terms, 5, 20)
    bumped = list(terms)
    bumped[3] = terms[3] + 7.0          # layer 4
    bumped[20] = terms[20] + 7.0        # layer 21
    assert np.array_equal(O.layer_range_score(bumped, 5, 20), mid)
    bumped[4] = terms[4] + 1.0          # layer 5 is inside
    np.testing.assert_allclose(O.layer_range_score(bumped, 5, 20), mid + 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.layer_range_score(terms, 9, 9), terms[8], rtol=0)
    doubled = [2 * t for t in terms]
    np.testing.assert_allclose(O.layer_range_score(doubled, 5, 20), 2 * mid, rtol=1e-13)
    for bad in ((0, 3), (5, 33), (7, 6)):
        with pytest.raises(O.OracleError):
            O.layer_range_score(terms, *bad)


# ---------------------------------------------------------------------------
# bf16 store rounding (round_bf16)
# ---------------------------------------------------------------------------

def _bf16_values(bits):
    """bf16 bit patterns -> their values (the upper half of a float32)."""
    with np.errstate(invalid="ignore"):            # NaN patterns
        return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_round_bf16_fixes_every_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = _bf16_values(bits)
    fin = np.isfinite(v)
    got = O.round_bf16(v[fin])
    assert np.array_equal(got, v[fin])
    assert np.array_equal(np.signbit(got), np.signbit(v[fin]))


def test_round_bf16_ties_to_even_and_nearest():
    # consecutive positive finite bf16 values (normals and subnormals) and the
    # exact midpoints between them: ties go to the even bit pattern, and a
    # hair either side of a tie goes to the nearer neighbour
    bits = np.arange(0, 0x7f7f, dtype=np.uint32)
    lo, hi = _bf16_values(bits), _bf16_values(bits + 1)
    mid = (lo + hi) / 2                      # exact in float64
    even = np.where(bits % 2 == 0, lo, hi)
    assert np.array_equal(O.round_bf16(mid), even)
    assert np.array_equal(O.round_bf16(-mid), -even)
    gap = hi - lo
    assert np.array_equal(O.round_bf16(mid - gap / 64), lo)
    assert np.array_equal(O.round_bf16(mid + gap / 64), hi)
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                  # tie at 1: to the even 1.0
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie above 1 + 2^-7: to the even one


def test_round_bf16_matches_float32_bit_rounding():
    # an independent route for float32 inputs: add 0x7fff plus the lowest kept
    # bit to the float32 pattern and drop the low half
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7fff + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    assert np.array_equal(O.round_bf16(f.astype(np.float64)), _bf16_values(r))


def test_layer_step_bf16_store_reads_the_rounded_rows():
    # with store="bf16" the step's q, K and V are the rounded ones, the cache
    # holds them, and the attention equals the exact oracle run on those values
    rng = np.random.default_rng(3)
    H, D, d = 2, 8, 16
    kv = 24
    table = O.build_block_table([2], [1, 0], 2, 2)
    x = rng.standard_normal((5, d))
    w = rng.standard_normal((3 * H * D, d)) / 4
    logical = np.array([3, 7, 11, 20, 23])
    kc = rng.standard_normal((32, H * D))
    vc = rng.standard_normal((32, H * D))
    a = O.layer_step(x, w, logical, logical, [0, 5], [kv], [2], kc, vc, table, H, D, 1e4, 16, store="bf16")
    b = O.layer_step(x, w, logical, logical, [0, 5], [kv], [2], kc, vc, table, H, D, 1e4, 16)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], O.round_bf16(b[key]))
        assert not np.array_equal(a[key], b[key])
    slots = a["slots"]
    assert np.array_equal(a["k_cache"][slots], a["k"]) and np.array_equal(a["v_cache"][slots], a["v"])
    o, _ = O.attention(a["q"], a["k_cache"], a["v_cache"], table, [0, 5], [kv], H, D, 16)
    assert np.array_equal(o, a["o"])
    with pytest.raises(O.OracleError):
        O.layer_step(x, w, logical, logical, [0, 5], [kv], [2], kc, vc, table, H, D, 1e4, 16, store="fp16")
