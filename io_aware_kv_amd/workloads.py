"""Seeded synthetic inputs for the Flash-Cache per-layer denoising step.

This module is the only code shared by the HIP path's callers (tests, bench) and
the CPU oracle.  It holds none of the method's arithmetic: no projection, no
rotary embedding, no attention, no column mass and no selection.  It draws
random numbers, rounds the draws once to bf16, and lays out the structure of
each workload (sequence lengths, decode progress, which logical positions are
queried, the page pool permutation, and the Flash-Verify visibility pattern as
a boolean input matrix).

Citation keys used below:
  [FD]  "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
        Memory-Efficient Diffusion LLMs" (paper summary page, paper.rainbus.top)
  [AIP] "Flash-dLLM 是什麼？擴散語言模型推論快 11 倍" (aiposthub explainer)
  [FST] Fast-dLLM article (senqingzn.com): block-wise PrefixCache / DualCache
  [FDLM] FlashDLM notes (papernotes.org): FreeCache

Workloads (all synthetic, random-init; LLaDA-8B-shaped where stated):
  tiny_f32   1 layer, d_model 256, 4 heads x 64, RoPE base 1e4, fp32;
             2 sequences of 128 (prompt 64 + gen 64), window 32 + 4 new + top-8.
  llada_b1   1 layer, d_model 4096, 32 heads x 128, RoPE base 5e5, bf16;
             1 sequence of 512 (prompt 256 + gen 256), window 32 + 8 new + top-32.
  mixed_b8   same layer; 8 sequences: 6 in the cache phase (context 512..1024,
             40..72 query rows) and 2 in full refresh (512 and 1024 rows).
  verify_b4  same layer; 4 sequences of 1024 (prompt 768 + gen 256) plus 32
             scratch positions for the draft and mask views of 16 search tokens.
  llada_b32  32 layers with distinct weights; 32 sequences of 2048 (prompt 1536
             + gen 512); cache-phase steps of 72 rows per sequence and full
             refresh steps of 2048 rows per sequence.
  tiny_bf16  1 layer, d_model 256, 2 heads x 128, RoPE base 1e4, bf16; shaped
             like tiny_f32 (a quick check of the bf16 kernels).

Seeds: numpy PCG64 seeded with [1000 * workload_id + stream, ...]; streams are
1 = weights (per layer), 2 = x (per step and layer), 3 = pool permutation,
4 = decode positions (new / search rows), 5 = sequence lengths and progress,
6 = planted heavy-hitter positions.
Decode-side workloads (logits rows of masked window positions, width VOCAB)
seed PCG64 with [7000 + seed, vocab] for the row structure and [7100 + seed,
vocab] for host logits; device logits use torch's generator seeded from the
same seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PAGE = 16          # tokens per KV page
BLOCK = 32         # generation block (decode granularity) of these workloads

WORKLOAD_IDS = {"tiny_f32": 1, "llada_b1": 2, "mixed_b8": 3, "verify_b4": 4, "llada_b32": 5,
                "tiny_bf16": 6}


@dataclass(frozen=True)
class LayerShape:
    d_model: int
    n_heads: int
    head_dim: int
    rope_base: float
    dtype: str          # "f32" or "bf16"
    layers: int
    top_k: int


@dataclass
class Sequence:
    ctx: int                    # context length (prompt + generation), logical 0..ctx-1
    prompt: int                 # prompt length
    decoded_blocks: int         # generation blocks already decoded
    window: np.ndarray          # logical positions of the masked window (query rows, mass rows)
    new: np.ndarray             # positions decoded by the previous step (refreshed this step)
    n_rows: int                 # query rows of the workload's own step
    full_refresh: bool          # the workload's own step refreshes every position
    scratch: int = 0            # extra logical slots after ctx (verify views)
    search: Optional[np.ndarray] = None   # verify step: search positions, ascending

    @property
    def cap(self) -> int:
        return self.ctx + self.scratch

    @property
    def pages(self) -> int:
        return -(-self.cap // PAGE)

    def eligible(self, n_cap: int) -> np.ndarray:
        """Decoded generation positions not decoded by the previous step."""
        e = np.zeros(n_cap, dtype=bool)
        e[self.prompt:self.prompt + BLOCK * self.decoded_blocks] = True
        e[self.new] = False
        return e


@dataclass
class Workload:
    name: str
    wid: int
    shape: LayerShape
    seqs: List[Sequence]
    seq_pages: np.ndarray       # int32 [B]
    pool_pages: int
    pool_perm: np.ndarray       # int32 [pool_pages], a permutation of the pool
    max_pages: int
    heavy: bool = False         # planted heavy hitters in step 0

    @property
    def n_seq(self) -> int:
        return len(self.seqs)

    @property
    def n_cap(self) -> int:
        return self.max_pages * PAGE

    def eligible(self) -> np.ndarray:
        return np.stack([s.eligible(self.n_cap) for s in self.seqs]).astype(np.uint8)


@dataclass
class StepRows:
    """Query rows of one step.  Rows of sequence b are cu_q[b]..cu_q[b+1]-1; the
    first mass_count[b] of them are the masked-window rows whose attention feeds
    the tracked-set score."""
    cu_q: np.ndarray            # int32 [B+1]
    logical: np.ndarray         # int32 [R] cache position written by the row
    pos: np.ndarray             # int32 [R] rotary position of the row
    mass_count: np.ndarray      # int32 [B]
    kv_len: np.ndarray          # int32 [B] keys attended (logical 0..kv_len-1)
    visible: Optional[List[np.ndarray]] = None   # per sequence bool [rows_b, kv_b]

    @property
    def n_rows(self) -> int:
        return int(self.cu_q[-1])


def _rng(wid: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([1000 * wid + stream, *extra]))


def round_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sorted_choice(rng: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    return np.sort(rng.choice(np.arange(lo, hi), size=n, replace=False)).astype(np.int32)


def _cache_seq(rng: np.random.Generator, ctx: int, prompt: int, decoded: int, n_new: int,
               n_rows: int, full: bool = False) -> Sequence:
    w0 = prompt + BLOCK * decoded
    window = np.arange(w0, w0 + BLOCK, dtype=np.int32)
    new = _sorted_choice(rng, w0 - BLOCK, w0, n_new)
    return Sequence(ctx=ctx, prompt=prompt, decoded_blocks=decoded, window=window, new=new,
                    n_rows=n_rows, full_refresh=full)


def make_workload(name: str, heavy: bool = False) -> Workload:
    wid = WORKLOAD_IDS[name]
    pos_rng = _rng(wid, 4)
    len_rng = _rng(wid, 5)
    if name == "tiny_f32":
        shape = LayerShape(256, 4, 64, 1e4, "f32", 1, 8)
        seqs = [_cache_seq(pos_rng, 128, 64, 1, 4, 32 + 4 + 8) for _ in range(2)]
    elif name == "tiny_bf16":
        shape = LayerShape(256, 2, 128, 1e4, "bf16", 1, 8)
        seqs = [_cache_seq(pos_rng, 128, 64, 1, 4, 32 + 4 + 8) for _ in range(2)]
    elif name == "llada_b1":
        shape = LayerShape(4096, 32, 128, 5e5, "bf16", 1, 32)
        seqs = [_cache_seq(pos_rng, 512, 256, 4, 8, 72)]
    elif name == "mixed_b8":
        shape = LayerShape(4096, 32, 128, 5e5, "bf16", 1, 32)
        seqs = []
        for _ in range(6):
            ctx = int(len_rng.integers(512, 1025))
            rows = int(len_rng.integers(40, 73))
            dec = int(len_rng.integers(2, 8))
            seqs.append(_cache_seq(pos_rng, ctx, ctx - 256, dec, min(8, rows - 32), rows))
        for ctx in (512, 1024):
            dec = int(len_rng.integers(2, 8))
            seqs.append(_cache_seq(pos_rng, ctx, ctx - 256, dec, 8, ctx, full=True))
        order = len_rng.permutation(len(seqs))
        seqs = [seqs[i] for i in order]
    elif name == "verify_b4":
        shape = LayerShape(4096, 32, 128, 5e5, "bf16", 1, 32)
        seqs = []
        for _ in range(4):
            s = _cache_seq(pos_rng, 1024, 768, 4, 8, 16 + 8 + 16 + 16 + 16)
            s.scratch = 2 * 16
            s.search = _sorted_choice(pos_rng, int(s.window[0]), int(s.window[-1]) + 1, 16)
            seqs.append(s)
    elif name == "llada_b32":
        shape = LayerShape(4096, 32, 128, 5e5, "bf16", 32, 32)
        seqs = []
        for _ in range(32):
            dec = int(len_rng.integers(2, 15))
            seqs.append(_cache_seq(pos_rng, 2048, 1536, dec, 8, 72))
    else:
        raise KeyError(name)
    seq_pages = np.array([s.pages for s in seqs], dtype=np.int32)
    pool_pages = int(seq_pages.sum())
    pool_perm = _rng(wid, 3).permutation(pool_pages).astype(np.int32)
    return Workload(name=name, wid=wid, shape=shape, seqs=seqs, seq_pages=seq_pages,
                    pool_pages=pool_pages, pool_perm=pool_perm,
                    max_pages=int(seq_pages.max()), heavy=heavy)


def full_refresh_rows(wl: Workload) -> StepRows:
    """Step 0 of every workload: every context position is a query row and is
    written to the cache ([FD] 方法步骤详情 / Algorithm 2 step 1: one forward over
    the whole sequence fills the cache).  The masked-window rows come first."""
    cu = [0]
    logical, mass = [], []
    for s in wl.seqs:
        rest = np.setdiff1d(np.arange(s.ctx, dtype=np.int32), s.window)
        logical.append(np.concatenate([s.window, rest]).astype(np.int32))
        mass.append(len(s.window))
        cu.append(cu[-1] + s.ctx)
    lg = np.concatenate(logical)
    return StepRows(cu_q=np.array(cu, dtype=np.int32), logical=lg, pos=lg.copy(),
                    mass_count=np.array(mass, dtype=np.int32),
                    kv_len=np.array([s.ctx for s in wl.seqs], dtype=np.int32))


def verify_visibility(s: Sequence, n_tv: int) -> np.ndarray:
    """Visibility of one verify-step sequence, rows ordered [mask views (m),
    draft views (m), T_v (n_tv)] and keys 0..ctx+2m-1, where the draft view of
    search token i sits at logical ctx+i and its mask view at ctx+m+i.

    Reading of [FD] 核心方法 / 方法步骤详情 step 3 and [AIP] Flash-Verify section:
    the two views of a token cannot see each other; a mask view cannot see its
    own draft but sees the drafts of earlier search tokens (position order);
    drafts are causal among themselves; no draft sees a mask view; ordinary
    rows see no view; nobody sees the stale cache entries of the search
    positions, which the views stand in for.  Every other context key is
    visible to every row."""
    m = len(s.search)
    kv = s.ctx + 2 * m
    rows = 2 * m + n_tv
    vis = np.zeros((rows, kv), dtype=bool)
    vis[:, :s.ctx] = True
    vis[:, s.search] = False
    d0, m0 = s.ctx, s.ctx + m
    for i in range(m):
        # mask view i (row i): drafts of earlier search tokens, and itself
        vis[i, d0:d0 + i] = True
        vis[i, m0 + i] = True
        # draft view i (row m+i): drafts 0..i
        vis[m + i, d0:d0 + i + 1] = True
    return vis


def config_step_rows(wl: Workload, tracked: List[np.ndarray]) -> StepRows:
    """The workload's own step (step 1).  tracked[b] lists the top-k positions
    of step 0 in descending score order; the first n of them are queried.

    Cache phase ([FD] 方法步骤详情 step 2): window + new + tracked, window first.
    Verify step ([FD] 方法步骤详情 step 3): mask views, draft views, then T_v =
    the other window positions, the new positions and 16 tracked positions."""
    cu = [0]
    logical, pos, mass, kv, vis = [], [], [], [], []
    for b, s in enumerate(wl.seqs):
        if s.full_refresh:
            rest = np.setdiff1d(np.arange(s.ctx, dtype=np.int32), s.window)
            lg = np.concatenate([s.window, rest]).astype(np.int32)
            ps = lg.copy()
            mass.append(len(s.window))
            kv.append(s.ctx)
            vis.append(None)
        elif s.search is not None:
            m = len(s.search)
            others = np.setdiff1d(s.window, s.search)
            n_tr = s.n_rows - 2 * m - len(others) - len(s.new)
            tr = np.asarray(tracked[b][:n_tr], dtype=np.int32)
            tv = np.concatenate([others, s.new, tr]).astype(np.int32)
            lg = np.concatenate([np.arange(s.ctx + m, s.ctx + 2 * m),   # mask views
                                 np.arange(s.ctx, s.ctx + m),           # draft views
                                 tv]).astype(np.int32)
            ps = np.concatenate([s.search, s.search, tv]).astype(np.int32)
            mass.append(m)
            kv.append(s.ctx + 2 * m)
            vis.append(verify_visibility(s, len(tv)))
        else:
            n_tr = s.n_rows - len(s.window) - len(s.new)
            tr = np.asarray(tracked[b][:n_tr], dtype=np.int32)
            lg = np.concatenate([s.window, s.new, tr]).astype(np.int32)
            ps = lg.copy()
            mass.append(len(s.window))
            kv.append(s.ctx)
            vis.append(None)
        assert len(lg) == s.n_rows
        logical.append(lg)
        pos.append(ps)
        cu.append(cu[-1] + len(lg))
    has_mask = any(v is not None for v in vis)
    if has_mask:
        vis = [v if v is not None else np.ones((cu[b + 1] - cu[b], kv[b]), dtype=bool)
               for b, v in enumerate(vis)]
    return StepRows(cu_q=np.array(cu, dtype=np.int32), logical=np.concatenate(logical),
                    pos=np.concatenate(pos), mass_count=np.array(mass, dtype=np.int32),
                    kv_len=np.array(kv, dtype=np.int32), visible=vis if has_mask else None)


BLOCK_CACHE_MODES = ("dual", "active")


def block_cache_rows(wl: Workload, mode: str) -> StepRows:
    """Query rows of a block-granular caching step, over the same cache and
    kernels as the Flash-Cache step (no formula-(2) rows, no verify mask).

    "dual":   only the current block (the masked window) is queried and
              written; every other position, the masked suffix included, is
              read from the cache ([FST] block-wise DualCache).
    "active": the current block and every later generation block (the active
              window B_i..B_N) are queried and written; the prompt and the
              finished blocks before the window are frozen in the cache
              ([FST] PrefixCache, which recomputes the suffix; [FDLM] FreeCache,
              which freezes blocks once they are fully decoded).
    Keys are the whole context in both modes."""
    if mode not in BLOCK_CACHE_MODES:
        raise ValueError(mode)
    cu = [0]
    logical = []
    for s in wl.seqs:
        w0 = int(s.window[0])
        lg = s.window if mode == "dual" else np.arange(w0, s.ctx)
        logical.append(np.asarray(lg, dtype=np.int32))
        cu.append(cu[-1] + len(lg))
    lg = np.concatenate(logical)
    return StepRows(cu_q=np.array(cu, dtype=np.int32), logical=lg, pos=lg.copy(),
                    mass_count=np.zeros(wl.n_seq, dtype=np.int32),
                    kv_len=np.array([s.ctx for s in wl.seqs], dtype=np.int32))


def weights(wl: Workload, layer: int = 0) -> np.ndarray:
    """W_qkv of one layer, [3 d_model, d_model] (out x in; Q, K, V blocks), drawn
    N(0, 1/d_model) in fp32.  bf16 workloads get uint16 bf16 bits."""
    sh = wl.shape
    n = sh.n_heads * sh.head_dim
    w = _rng(wl.wid, 1, layer).standard_normal((3 * n, sh.d_model), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(sh.d_model))
    return w if sh.dtype == "f32" else round_bf16_bits(w)


def activations(wl: Workload, rows: StepRows, step: int, layer: int = 0) -> np.ndarray:
    """Layer input x, [R, d_model], N(0,1) in fp32 (bf16 bits for bf16 workloads).
    With planted heavy hitters, step 0 rows of 32 seeded eligible positions per
    sequence are scaled by 2, which makes their keys attract more attention."""
    sh = wl.shape
    x = _rng(wl.wid, 2, step, layer).standard_normal((rows.n_rows, sh.d_model), dtype=np.float32)
    if wl.heavy and step == 0:
        hr = _rng(wl.wid, 6)
        for b, s in enumerate(wl.seqs):
            cand = np.flatnonzero(s.eligible(wl.n_cap))
            hh = hr.choice(cand, size=min(32, len(cand)), replace=False)
            lg = rows.logical[rows.cu_q[b]:rows.cu_q[b + 1]]
            sel = np.flatnonzero(np.isin(lg, hh)) + rows.cu_q[b]
            x[sel] *= np.float32(2.0)
    return x if sh.dtype == "f32" else round_bf16_bits(x)


def as_f64(wl: Workload, a: np.ndarray) -> np.ndarray:
    """The exact values of a drawn array as float64."""
    return a.astype(np.float64) if wl.shape.dtype == "f32" else bf16_bits_to_f64(a)


def sentinel_cache(wl: Workload, rows: int, width: int, salt: int) -> np.ndarray:
    """A recognisable fill for cache rows that a step must not touch."""
    r = _rng(wl.wid, 7, salt)
    v = r.uniform(-4.0, 4.0, size=(rows, width)).astype(np.float32)
    return v if wl.shape.dtype == "f32" else round_bf16_bits(v)


# ---------------------------------------------------------------------------
# Large workloads: draws on the device (torch's seeded generator), because
# drawing ~10^8 normals per layer on the host would dominate every run.  The
# oracle receives copies of the same device values.
# ---------------------------------------------------------------------------

def device_normal_bf16(shape, std: float, seed: int, device):
    """N(0, std^2) drawn in fp32 with a seeded torch generator on `device`,
    rounded once (RNE) to bf16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def device_weights(wl: Workload, layer: int, device):
    sh = wl.shape
    n = sh.n_heads * sh.head_dim
    return device_normal_bf16((3 * n, sh.d_model), 1.0 / np.sqrt(sh.d_model),
                              (1000 * wl.wid + 1) * 4096 + layer, device)


def device_activations(wl: Workload, rows: StepRows, step: int, layer: int, device):
    return device_normal_bf16((rows.n_rows, wl.shape.d_model), 1.0,
                              ((1000 * wl.wid + 2) * 64 + step) * 4096 + layer, device)


def device_cache_fill(wl: Workload, layer: int, which: int, device):
    """Contents of a layer's K (which = 0) or V (which = 1) cache before a
    step that is checked on its own, without the full refresh that would
    otherwise fill it: every row N(0, 1) in bf16, the spread of a projected
    K or V element of these inputs (x ~ N(0, 1), W ~ N(0, 1/d_model))."""
    sh = wl.shape
    n = sh.n_heads * sh.head_dim
    return device_normal_bf16((wl.pool_pages * PAGE, n), 1.0,
                              ((1000 * wl.wid + 9) * 4 + which) * 4096 + layer, device)


def seeded_tracked(wl: Workload, step: int) -> List[np.ndarray]:
    """Tracked positions chosen by a seeded draw among the eligible ones (used
    where a step's row set must not depend on either side's top-k)."""
    r = _rng(wl.wid, 8, step)
    out = []
    for s in wl.seqs:
        cand = np.flatnonzero(s.eligible(wl.n_cap))
        out.append(np.sort(r.choice(cand, size=min(wl.shape.top_k, len(cand)), replace=False)).astype(np.int32))
    return out


# ---------------------------------------------------------------------------
# Decode-side inputs: one logits row per masked window position of a step.
# ---------------------------------------------------------------------------

# Assumed LM-head width.  The pages give no vocabulary size, so the decode-side
# workloads take a round 128 Ki tokens; every kernel takes the width as an
# argument.
VOCAB = 131072


@dataclass
class DecodeRows:
    cu: np.ndarray        # int32 [n_seq + 1]: rows of sequence b are cu[b] .. cu[b+1]-1
    peak_tok: np.ndarray  # int32 [R]: token given the planted peak
    peak_val: np.ndarray  # float32 [R]: height of the planted peak (before bf16 rounding)
    twin_tok: np.ndarray  # int32 [R]: a second token given the same height, or -1
    draft: np.ndarray     # int32 [R]: draft-view token of the row (Flash-Verify input)


def decode_rows(seed: int, lens, vocab: int, twin_frac: float = 0.0, agree: float = 0.85) -> DecodeRows:
    """Row structure of a decode-side workload: per row a planted peak whose
    height spreads the softmax maximum over roughly 0.1 .. 0.99 for N(0,1)
    background logits (ln(vocab) + 1/2 is where the peak equals the background
    mass), optionally a twin peak of the same height at a random other token,
    and a draft token that equals the peak token with probability `agree`."""
    r = np.random.Generator(np.random.PCG64([7000 + int(seed), int(vocab)]))
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    R = int(cu[-1])
    peak_tok = r.integers(0, vocab, size=R).astype(np.int32)
    base = np.log(vocab) + 0.5
    peak_val = (base + r.uniform(-2.5, 5.5, size=R)).astype(np.float32)
    twin_tok = np.full(R, -1, dtype=np.int32)
    if vocab > 1:
        pick = r.random(R) < twin_frac
        other = (peak_tok + r.integers(1, vocab, size=R)) % vocab
        twin_tok[pick] = other[pick]
    draft = np.where(r.random(R) < agree, peak_tok, r.integers(0, vocab, size=R)).astype(np.int32)
    return DecodeRows(cu=cu, peak_tok=peak_tok, peak_val=peak_val, twin_tok=twin_tok, draft=draft)


def _plant(z: np.ndarray, rows: DecodeRows) -> None:
    ar = np.arange(len(rows.peak_tok))
    z[ar, rows.peak_tok] = rows.peak_val
    t = rows.twin_tok >= 0
    z[ar[t], rows.twin_tok[t]] = rows.peak_val[t]


def decode_logits_host(seed: int, rows: DecodeRows, vocab: int, dtype: str = "bf16") -> np.ndarray:
    """[R, vocab] logits: N(0,1) background drawn in fp32 with the planted peaks,
    then rounded once to bf16 (returned as uint16 bit patterns) or kept fp32."""
    r = np.random.Generator(np.random.PCG64([7100 + int(seed), int(vocab)]))
    z = r.standard_normal((len(rows.peak_tok), vocab), dtype=np.float32)
    _plant(z, rows)
    return round_bf16_bits(z) if dtype == "bf16" else z


def decode_logits_device(seed: int, rows: DecodeRows, vocab: int, device):
    """The same structure drawn on the device (torch's seeded generator) for
    full-size workloads: bf16 [R, vocab]."""
    import torch
    R = len(rows.peak_tok)
    t = device_normal_bf16((R, vocab), 1.0, 7200 * 4096 + int(seed), device)
    ar = torch.arange(R, device=device)
    t[ar, torch.from_numpy(rows.peak_tok.astype(np.int64)).to(device)] = \
        torch.from_numpy(rows.peak_val).to(device).to(torch.bfloat16)
    tw = np.flatnonzero(rows.twin_tok >= 0)
    if len(tw):
        twi = torch.from_numpy(tw.astype(np.int64)).to(device)
        t[twi, torch.from_numpy(rows.twin_tok[tw].astype(np.int64)).to(device)] = \
            torch.from_numpy(rows.peak_val[tw]).to(device).to(torch.bfloat16)
    return t


# ---------------------------------------------------------------------------
# Long contexts for the attention alone: sequences whose keys span more key
# tiles than the workloads above (up to the bf16 kernel's 16384-key page
# table), on a shuffled page pool, with seeded q and cache contents.
# ---------------------------------------------------------------------------

@dataclass
class LongContext:
    kv: np.ndarray            # keys per sequence
    rows: np.ndarray          # query rows per sequence
    mass_count: np.ndarray    # score rows per sequence (the first rows)
    seq_pages: np.ndarray     # pages per sequence (ceil(kv / 16))
    pool_pages: int
    pool_perm: np.ndarray     # the pool's page order (sequence b takes the next seq_pages[b])
    max_pages: int
    seed: int


def long_context(kv, rows, mass_count, seed: int) -> LongContext:
    kv = np.asarray(kv, dtype=np.int32)
    seq_pages = (kv + PAGE - 1) // PAGE
    pool = int(seq_pages.sum()) + 8                  # a few spare pages
    perm = np.random.default_rng([7300, seed]).permutation(pool).astype(np.int32)
    return LongContext(kv=kv, rows=np.asarray(rows, dtype=np.int32),
                       mass_count=np.asarray(mass_count, dtype=np.int32), seq_pages=seq_pages,
                       pool_pages=pool, pool_perm=perm, max_pages=int(seq_pages.max()), seed=seed)


def long_context_tensors(lc: LongContext, n_out: int, device):
    """q [sum(rows), n_out] and the K, V caches [pool_pages * 16, n_out],
    N(0, 1) in bf16."""
    R = int(lc.rows.sum())
    base = (7400 + lc.seed) * 16
    return (device_normal_bf16((R, n_out), 1.0, base, device),
            device_normal_bf16((lc.pool_pages * PAGE, n_out), 1.0, base + 1, device),
            device_normal_bf16((lc.pool_pages * PAGE, n_out), 1.0, base + 2, device))
