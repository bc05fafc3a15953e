"""Plain float64 definitions of the Flash-Cache per-layer step.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests, the smoke
check and the CPU baseline of bench.py, never by the product path.

Citation keys:
  [FD]  "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
        Memory-Efficient Diffusion LLMs", paper summary page (paper.rainbus.top).
        Sections used: 核心方法 (core method), 方法步骤详情 (Algorithm 2 and
        formula (2)), 研究动机 (motivation), 技术新颖性 (novelty).
  [AIP] "Flash-dLLM 是什麼？擴散語言模型推論快 11 倍" (aiposthub explainer),
        sections on Flash-Cache, selective refresh and Flash-Verify.
  [FST] Fast-dLLM article (senqingzn.com), sections on the block-wise
        PrefixCache / DualCache.

Readings of points the pages leave open (each is also listed with its reason
in the project's design notes):
  * no input norm and no projection bias; W_qkv is [3n, d_in] (out x in) with
    the Q, K, V blocks in that order and head h at rows h*D .. h*D+D-1 of each;
  * rotary embedding is the rotate-half form: pairs (i, i + D/2), frequencies
    theta_i = base^(-2i/D), angle = position * theta_i, q and k rotated, v not;
  * the cache holds K after rotation; this step's rows are written before the
    attention reads the cache, so each row sees its own fresh K/V;
  * keys are every logical position 0..kv_len-1 of the sequence, no causal
    mask (bidirectional), scale 1/sqrt(D), unless a visibility matrix is given;
  * formula (2)'s S is the post-softmax probability; the masked-window rows are
    the first mass_count[b] rows of each sequence; the per-layer term is
    added into a running score;
  * top-k ties go to the lower position; fewer than k candidates pad with -1.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from .lowbit import e4m3_round


class OracleError(ValueError):
    """An input the method cannot accept (bad table, range or duplicate)."""


# ---------------------------------------------------------------------------
# a0: block table and slot mapping
# ---------------------------------------------------------------------------

def build_block_table(seq_pages: Sequence[int], pool_perm: Sequence[int], pool_pages: int,
                      max_pages: int) -> np.ndarray:
    """Per-sequence page table over one shared page pool.

    [FD] 核心方法 and 技术新颖性 describe a block table that maps each
    sequence's query blocks to its KV blocks; [FD] 方法步骤详情 step 1
    preallocates one flat cache of B*N_max rows that is never reallocated.
    Reading: sequence b takes the next seq_pages[b] entries of a caller-given
    permutation of the pool; table[b][j] is the physical page of its j-th
    logical page, -1 past the end."""
    seq_pages = [int(p) for p in seq_pages]
    perm = [int(p) for p in pool_perm]
    if pool_pages < 0 or max_pages < 0:
        raise OracleError("negative size")
    if any(p < 0 for p in seq_pages):
        raise OracleError("negative page count")
    if any(p > max_pages for p in seq_pages):
        raise OracleError("sequence needs more pages than max_pages")
    if sum(seq_pages) > pool_pages:
        raise OracleError("pages requested exceed the pool")
    if len(perm) != pool_pages or sorted(perm) != list(range(pool_pages)):
        raise OracleError("pool_perm is not a permutation of the pool")
    table = np.full((len(seq_pages), max_pages), -1, dtype=np.int64)
    taken = 0
    for b, n in enumerate(seq_pages):
        for j in range(n):
            table[b, j] = perm[taken + j]
        taken += n
    return table


def row_slots(page_table: np.ndarray, cu_q: Sequence[int], logical: Sequence[int],
              page_size: int) -> np.ndarray:
    """Flat cache row written by each query row: the row's logical position
    split into (logical page, offset), the page looked up in its sequence's
    table.  Two rows may not share a slot (that would be a write race)."""
    B = len(cu_q) - 1
    slots = np.empty(len(logical), dtype=np.int64)
    for b in range(B):
        for r in range(int(cu_q[b]), int(cu_q[b + 1])):
            lg = int(logical[r])
            if lg < 0:
                raise OracleError("negative logical position")
            page_idx, off = divmod(lg, page_size)
            if page_idx >= page_table.shape[1] or page_table[b, page_idx] < 0:
                raise OracleError("logical position beyond the sequence's pages")
            slots[r] = int(page_table[b, page_idx]) * page_size + off
    if len(set(slots.tolist())) != len(slots):
        raise OracleError("two rows map to one cache slot")
    return slots


# ---------------------------------------------------------------------------
# a1..a3: projection, rotary embedding, cache write
# ---------------------------------------------------------------------------

def project(x: np.ndarray, w: np.ndarray, n_out: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """QKV projection qkv = x W^T, split into q, k, v of width n_out each
    ([FD] 核心方法: the projection is the first stage of the fused kernel)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if w.shape != (3 * n_out, x.shape[1]):
        raise OracleError("W_qkv shape")
    qkv = np.matmul(x, w.T)
    return qkv[:, :n_out], qkv[:, n_out:2 * n_out], qkv[:, 2 * n_out:]


def rope(t: np.ndarray, pos: Sequence[int], base: float) -> np.ndarray:
    """Rotate-half rotary embedding of t [R, H, D] at integer positions.

    For i < D/2: theta_i = base^(-2i/D), phi = pos * theta_i,
      out[i]       = t[i] cos phi - t[i + D/2] sin phi
      out[i + D/2] = t[i + D/2] cos phi + t[i] sin phi.
    ([FD] 研究动机 and 核心方法 name RoPE as the second fused stage.)"""
    t = np.asarray(t, dtype=np.float64)
    R, H, D = t.shape
    half = D // 2
    p = np.asarray(pos, dtype=np.float64).reshape(R, 1)
    out = np.empty_like(t)
    for i in range(half):
        theta = float(base) ** (-2.0 * i / D)
        c, s = np.cos(p * theta), np.sin(p * theta)       # [R, 1], broadcast over heads
        a = t[:, :, i]
        b = t[:, :, i + half]
        out[:, :, i] = a * c - b * s
        out[:, :, i + half] = b * c + a * s
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value, ties to even: 8 significant bits
    (the bfloat16 format keeps float32's 8-bit exponent and 7 stored fraction
    bits), spacing 2^(e-8) for |a| in [2^(e-1), 2^e), and 2^-133 below the
    smallest normal 2^-126.  Models a buffer of the path that stores bf16 (q,
    and the K/V cache rows, written once per step)."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                      # a = m 2^e with 1/2 <= |m| < 1 (e = 0 at 0)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(a, 8 - e)), e - 8)


def scatter(cache: np.ndarray, slots: Sequence[int], rows: np.ndarray) -> np.ndarray:
    """Write rows into the flat cache at the given slots; nothing else changes
    ([FD] 核心方法: K/V go straight into the preallocated flat layout)."""
    out = np.array(cache, dtype=np.float64, copy=True)
    for r, s in enumerate(slots):
        out[int(s)] = rows[r]
    return out


# ---------------------------------------------------------------------------
# a4: attention over the paged cache
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, page_table: np.ndarray,
              cu_q: Sequence[int], kv_len: Sequence[int], n_heads: int, head_dim: int,
              page_size: int, visible: Optional[List[np.ndarray]] = None
              ) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Dense softmax attention of each query row over its sequence's cached keys.

    Keys are logical positions 0..kv_len[b]-1 read through the block table
    ([FD] 核心方法: block-table scheduled attention; 方法步骤详情 step 2:
    bidirectional attention over the full cache).  Scores q.k/sqrt(D); keys
    hidden by `visible` get probability 0; a row that sees no key outputs 0.
    Returns o [R, H*D] and, per sequence, probabilities [H, rows_b, kv_b]."""
    H, D = n_heads, head_dim
    R = q.shape[0]
    o = np.zeros((R, H * D), dtype=np.float64)
    probs = []
    for b in range(len(cu_q) - 1):
        r0, r1 = int(cu_q[b]), int(cu_q[b + 1])
        kv = int(kv_len[b])
        slot = np.array([int(page_table[b, j // page_size]) * page_size + j % page_size
                         for j in range(kv)], dtype=np.int64)
        if kv and slot.min() < 0:
            raise OracleError("key beyond the sequence's pages")
        K = k_cache[slot].reshape(kv, H, D)
        V = v_cache[slot].reshape(kv, H, D)
        Q = q[r0:r1].reshape(r1 - r0, H, D)
        pb = np.zeros((H, r1 - r0, kv), dtype=np.float64)
        vis = None if visible is None else np.asarray(visible[b], dtype=bool)
        for h in range(H):
            s = np.matmul(Q[:, h, :], K[:, h, :].T) / np.sqrt(D)
            if vis is not None:
                s = np.where(vis, s, -np.inf)
            seen = np.isfinite(s).any(axis=1)              # rows with a visible key
            top = np.where(seen, np.max(np.where(np.isfinite(s), s, -np.inf), axis=1, initial=-np.inf), 0.0)
            e = np.where(np.isfinite(s), np.exp(s - top[:, None]), 0.0)
            tot = e.sum(axis=1)
            pb[h] = np.where(seen[:, None], e / np.where(seen, tot, 1.0)[:, None], 0.0)
            o[r0:r1, h * D:(h + 1) * D] = np.matmul(pb[h], V[:, h, :])
        probs.append(pb)
    return o, probs


# ---------------------------------------------------------------------------
# a5: one layer's term of formula (2); a6: top-k
# ---------------------------------------------------------------------------

def column_mass(probs: List[np.ndarray], mass_count: Sequence[int], n_cap: int) -> np.ndarray:
    """One layer's term of the tracked-set score ([FD] 方法步骤详情 step 4,
    formula (2)): for key i, the attention it receives from the masked-window
    query rows, averaged over those rows and over the heads.  Summing these
    terms over the layers gives a_i.  The score has n_cap entries per
    sequence: keys at or past n_cap are not recorded."""
    out = np.zeros((len(probs), n_cap), dtype=np.float64)
    for b, pb in enumerate(probs):
        H, _, kv = pb.shape
        m = int(mass_count[b])
        if m == 0:
            continue
        k = min(kv, n_cap)
        out[b, :k] = (pb[:, :m, :].sum(axis=(0, 1)) / (H * m))[:k]
    return out


def layer_range_score(terms: Sequence[np.ndarray], first: int, last: int) -> np.ndarray:
    """The tracked-set score summed over layers first..last only (1-based,
    inclusive) instead of every layer: the statistics taken from the middle
    layers where [FD] 研究动机 reports the attention to be concentrated (5 to
    20).  terms[l-1] is layer l's formula-(2) term."""
    if not 1 <= first <= last <= len(terms):
        raise OracleError("layer range outside the model")
    out = np.zeros_like(np.asarray(terms[0], dtype=np.float64))
    for layer in range(first, last + 1):
        out = out + np.asarray(terms[layer - 1], dtype=np.float64)
    return out


def topk(mass: np.ndarray, eligible: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per sequence, the k eligible positions with the largest score, highest
    first, ties to the lower position; -1 / 0 padding when fewer are eligible
    ([FD] 方法步骤详情 step 4: top-k decoded tokens by attention score)."""
    B, _ = mass.shape
    idx = np.full((B, k), -1, dtype=np.int64)
    val = np.zeros((B, k), dtype=np.float64)
    cnt = np.zeros(B, dtype=np.int64)
    for b in range(B):
        cand = [i for i in range(mass.shape[1]) if eligible[b, i]]
        cand.sort(key=lambda i: (-mass[b, i], i))
        take = cand[:k]
        cnt[b] = len(take)
        for j, i in enumerate(take):
            idx[b, j] = i
            val[b, j] = mass[b, i]
    return idx, val, cnt


# ---------------------------------------------------------------------------
# one layer of one step, end to end
# ---------------------------------------------------------------------------

def layer_step(x, w, pos, logical, cu_q, kv_len, mass_count, k_cache, v_cache, page_table,
               n_heads: int, head_dim: int, rope_base: float, page_size: int,
               visible=None, kv_format: str = "plain", store: str = "exact"):
    """Steps a1..a5 of one layer in the method's order: project, rotate q and
    k, write K/V rows into the cache, attend over the updated cache, and form
    this layer's formula-(2) term.  Returns a dict of float64 arrays.

    kv_format "e4m3": the rows are stored in the low-bit cache format of
    oracle/lowbit.py, so the cache (and "k", "v" of the result) hold the
    stored values, which the attention reads.
    store "bf16": q, K and V are rounded once to bf16 where the step stores
    them (q between the cache update and the attention, K/V in a bf16 cache),
    so the attention reads the stored values; "exact" keeps them in float64."""
    n = n_heads * head_dim
    q, k, v = project(x, w, n)
    R = q.shape[0]
    q = rope(q.reshape(R, n_heads, head_dim), pos, rope_base).reshape(R, n)
    k = rope(k.reshape(R, n_heads, head_dim), pos, rope_base).reshape(R, n)
    if store == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif store != "exact":
        raise OracleError(f"unknown store precision {store}")
    if kv_format == "e4m3":
        k, v = e4m3_round(k), e4m3_round(v)
    elif kv_format != "plain":
        raise OracleError(f"unknown cache format {kv_format}")
    slots = row_slots(page_table, cu_q, logical, page_size)
    kc = scatter(k_cache, slots, k)
    vc = scatter(v_cache, slots, v)
    o, probs = attention(q, kc, vc, page_table, cu_q, kv_len, n_heads, head_dim, page_size,
                         visible)
    mass = column_mass(probs, mass_count, page_table.shape[1] * page_size)
    return {"q": q, "k": k, "v": v, "slots": slots, "k_cache": kc, "v_cache": vc,
            "o": o, "probs": probs, "mass": mass}
