"""Device state and step driver of the Flash-Cache path.

[FD] "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
Memory-Efficient Diffusion LLMs" (paper summary page), 方法步骤详情:
step 1 preallocates one flat cache per layer and never reallocates it; each
later step queries a fixed-size row set (tracked ∪ masked window), runs the
fused cache update and the attention layer by layer, and after the last layer
picks the next tracked set by formula (2).

torch provides the device memory and the stream; every operation is a call
into libdllm.so through io_aware_kv_amd.dllm.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import dllm
from .workloads import PAGE, StepRows, Workload


@dataclass
class StepDevice:
    """Per-step device arrays (sized once per row set)."""
    n_rows: int
    cu_q: torch.Tensor
    logical: torch.Tensor
    pos: torch.Tensor
    slot: torch.Tensor
    mass_count: torch.Tensor
    kv_len: torch.Tensor
    max_kv: int
    max_mass: int
    mask_bits: Optional[torch.Tensor]
    mask_off: Optional[torch.Tensor]
    q: torch.Tensor
    o: torch.Tensor
    ws_qkv: torch.Tensor
    ws_attn: torch.Tensor
    qkv_raw: Optional[torch.Tensor] = None      # unfused arm: unrotated q|k|v rows


class FlashCacheRunner:
    def __init__(self, wl: Workload, device="cuda", layers: Optional[int] = None,
                 cache_copies: int = 1, kv_format: str = "plain"):
        """kv_format "e4m3": the caches hold one-byte E4M3 codes (bf16 layers)."""
        sh = wl.shape
        self.wl = wl
        self.device = torch.device(device)
        self.dtype = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
        self.dt = dllm.BF16 if sh.dtype == "bf16" else dllm.F32
        if kv_format not in ("plain", "e4m3") or (kv_format == "e4m3" and sh.dtype != "bf16"):
            raise ValueError(f"cache format {kv_format} for a {sh.dtype} layer")
        self.kv_format = kv_format
        cache_dtype = torch.uint8 if kv_format == "e4m3" else self.dtype
        self.dt_cache = dllm.BF16_E4M3KV if kv_format == "e4m3" else self.dt
        self.H, self.D = sh.n_heads, sh.head_dim
        self.n_out = sh.n_heads * sh.head_dim
        self.layers = sh.layers if layers is None else layers
        self.cache_rows = wl.pool_pages * PAGE
        self.n_cap = wl.n_cap
        # the flat caches: allocated once, never reallocated
        self.k_cache: List[torch.Tensor] = []
        self.v_cache: List[torch.Tensor] = []
        for _ in range(self.layers * cache_copies):
            self.k_cache.append(torch.zeros(self.cache_rows, self.n_out, dtype=cache_dtype, device=self.device))
            self.v_cache.append(torch.zeros(self.cache_rows, self.n_out, dtype=cache_dtype, device=self.device))
        self.page_table = torch.empty(wl.n_seq * wl.max_pages, dtype=torch.int32, device=self.device)
        dllm.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages, self.page_table)
        # formula (2) per-head running scores [B, H, n_cap]; top-k sums the heads
        self.mass = torch.zeros(wl.n_seq, self.H, self.n_cap, dtype=torch.float32, device=self.device)
        self.eligible = torch.from_numpy(wl.eligible()).to(self.device)
        k = sh.top_k
        self.top_idx = torch.empty(wl.n_seq, k, dtype=torch.int32, device=self.device)
        self.top_val = torch.empty(wl.n_seq, k, dtype=torch.float32, device=self.device)
        self.top_cnt = torch.empty(wl.n_seq, dtype=torch.int32, device=self.device)

    # ------------------------------------------------------------------
    def to_device_array(self, a: np.ndarray) -> torch.Tensor:
        """bf16 bits (uint16) or fp32 host array -> device tensor of the path dtype."""
        if self.dtype == torch.bfloat16:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)
            return t.view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)

    def upload_step(self, rows: StepRows) -> StepDevice:
        dev = self.device
        R = rows.n_rows
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        mask_bits = mask_off = None
        if rows.visible is not None:
            bits, off = dllm.pack_mask(rows.visible)
            mask_bits = torch.from_numpy(bits.view(np.int32)).to(dev)
            mask_off = torch.from_numpy(off).to(dev)
        max_kv = int(rows.kv_len.max())
        max_mass = int(rows.mass_count.max())
        ws_qkv_b = dllm.qkv_rope_cachewrite_workspace(self.dt, R, self.wl.shape.d_model, self.H, self.D)
        ws_attn_b = dllm.sched_attention_workspace(self.dt_cache, self.wl.n_seq, R, self.H, self.D, max_kv,
                                                   self.n_cap, max_mass)
        return StepDevice(
            n_rows=R, cu_q=i32(rows.cu_q), logical=i32(rows.logical), pos=i32(rows.pos),
            slot=torch.empty(R, dtype=torch.int32, device=dev), mass_count=i32(rows.mass_count),
            kv_len=i32(rows.kv_len), max_kv=max_kv, max_mass=max_mass,
            mask_bits=mask_bits, mask_off=mask_off,
            q=torch.empty(R, self.n_out, dtype=self.dtype, device=dev),
            o=torch.empty(R, self.n_out, dtype=self.dtype, device=dev),
            ws_qkv=torch.zeros(max(ws_qkv_b, 256), dtype=torch.uint8, device=dev),
            ws_attn=torch.zeros(max(ws_attn_b, 256), dtype=torch.uint8, device=dev))

    # ------------------------------------------------------------------
    def map_slots(self, st: StepDevice) -> None:
        dllm.map_slots(st.cu_q, st.logical, self.page_table, st.slot, self.wl.max_pages,
                       self.wl.pool_pages)

    def cache_update(self, st: StepDevice, x: torch.Tensor, w: torch.Tensor, layer: int = 0) -> None:
        dllm.qkv_rope_cachewrite(x, w, st.pos, st.slot, st.q, self.k_cache[layer], self.v_cache[layer],
                                 self.H, self.D, self.wl.shape.rope_base, st.ws_qkv)

    def cache_update_paged(self, st: StepDevice, x: torch.Tensor, w: torch.Tensor, layer: int = 0) -> None:
        """a0-a3 in one call: slots from the block table inside the projection."""
        dllm.qkv_rope_cachewrite_paged(x, w, st.pos, st.cu_q, st.logical, self.page_table, self.wl.max_pages,
                                       st.slot, st.q, self.k_cache[layer], self.v_cache[layer], self.H, self.D,
                                       self.wl.shape.rope_base, st.ws_qkv)

    def cache_update_unfused(self, st: StepDevice, x: torch.Tensor, w: torch.Tensor, layer: int = 0) -> None:
        """The unfused comparison arm of a1-a3: projection, rotary and cache write
        as three launches with q|k|v in memory between them (slots from map_slots)."""
        if st.qkv_raw is None:
            st.qkv_raw = torch.empty(st.n_rows, 3 * self.n_out, dtype=self.dtype, device=self.device)
        dllm.qkv_project(x, w, st.qkv_raw, self.H, self.D, st.ws_qkv)
        dllm.rope_apply(st.qkv_raw, st.pos, st.q, self.H, self.D, self.wl.shape.rope_base)
        dllm.cache_write(st.qkv_raw, st.slot, self.k_cache[layer], self.v_cache[layer], self.H, self.D)

    def attention(self, st: StepDevice, layer: int = 0, with_mass: bool = True,
                  mass_overwrite: bool = False) -> None:
        """mass_overwrite: this layer's term replaces the score (the first
        scoring layer of a step; then the top-k need not clear it)."""
        dllm.sched_attention(st.q, st.cu_q, self.k_cache[layer], self.v_cache[layer], self.page_table,
                             self.wl.max_pages, st.kv_len, st.o, st.ws_attn, self.H, self.D, st.max_kv,
                             mask_bits=st.mask_bits, mask_off=st.mask_off,
                             mass_count=st.mass_count if with_mass else None,
                             max_mass_rows=st.max_mass if with_mass else 0,
                             mass_accum=self.mass if with_mass else None, n_cap=self.n_cap,
                             mass_overwrite=mass_overwrite)

    def topk(self, clear_mass: bool = True) -> None:
        dllm.topk_tracked(self.mass, self.eligible, self.wl.shape.top_k, self.top_idx, self.top_val,
                          self.top_cnt, clear_mass=clear_mass)

    def layer_step(self, st: StepDevice, x: torch.Tensor, w: torch.Tensor, layer: int = 0,
                   fused_slots: bool = True, unfused: bool = False, with_mass: bool = True,
                   mass_overwrite: bool = False) -> None:
        """a0..a5 of one layer: slots and the fused cache update (one call, or
        the slot mapping as a call of its own; or the unfused three-launch arm),
        then attention + mass."""
        if unfused:
            self.map_slots(st)
            self.cache_update_unfused(st, x, w, layer)
        elif fused_slots:
            self.cache_update_paged(st, x, w, layer)
        else:
            self.map_slots(st)
            self.cache_update(st, x, w, layer)
        self.attention(st, layer, with_mass=with_mass, mass_overwrite=mass_overwrite)
