"""Thin Python binding of libdllm.so (the C ABI in include/dllm.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the path runs in the library's HIP kernels.  There
is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libdllm.so")

F32, BF16, BF16_E4M3KV = 0, 1, 2
PAGE = 16

# names in include/dllm.h, in declaration order
EXPORTS = (
    "dllm_status_string", "dllm_version", "dllm_build_block_table", "dllm_map_slots",
    "dllm_qkv_rope_cachewrite_workspace", "dllm_qkv_rope_cachewrite", "dllm_qkv_rope_cachewrite_paged",
    "dllm_qkv_project", "dllm_rope_apply", "dllm_cache_write",
    "dllm_sched_attention_workspace", "dllm_sched_attention", "dllm_topk_tracked",
    "dllm_confidence_workspace", "dllm_confidence_argmax", "dllm_confidence_commit", "dllm_verify_accept",
    "dllm_decode_commit", "dllm_decode_verify", "dllm_set_tuning", "dllm_sched_attention_noalloc",
)
NOALLOC_SCRATCH_BYTES = 64 << 20     # DLLM_NOALLOC_SCRATCH_BYTES


class DllmError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {code} ({text})")
        self.code = code


_lib = None
_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is missing: build it with `python -m io_aware_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dllm_status_string.argtypes = [_i32]
    lib.dllm_status_string.restype = ctypes.c_char_p
    lib.dllm_version.argtypes = []
    lib.dllm_version.restype = _i32
    lib.dllm_build_block_table.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
    lib.dllm_map_slots.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.dllm_qkv_rope_cachewrite_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.dllm_qkv_rope_cachewrite_workspace.restype = _sz
    lib.dllm_qkv_rope_cachewrite.argtypes = [_i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _vp, _i64, _vp, _sz, _vp]
    lib.dllm_qkv_rope_cachewrite_paged.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                                   _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i64,
                                                   _vp, _sz, _vp]
    lib.dllm_qkv_project.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.dllm_rope_apply.argtypes = [_i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp]
    lib.dllm_cache_write.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp]
    lib.dllm_sched_attention_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.dllm_sched_attention_workspace.restype = _sz
    lib.dllm_sched_attention.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                         _i64, _vp, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _i32,
                                         _i32, _vp, _vp, _sz, _vp]
    lib.dllm_topk_tracked.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp]
    lib.dllm_confidence_workspace.argtypes = [_i32, _i32]
    lib.dllm_confidence_workspace.restype = _sz
    lib.dllm_confidence_argmax.argtypes = [_i32, _i32, _i32, _vp, _i64, _vp, _vp, _vp, _sz, _vp]
    lib.dllm_confidence_commit.argtypes = [_i32, _i32, _vp, _vp, _f32, _vp, _vp, _vp]
    lib.dllm_verify_accept.argtypes = [_i32, _i32, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp]
    lib.dllm_decode_commit.argtypes = [_i32, _i32, _i32, _vp, _i32, _vp, _i64, _f32, _vp, _vp, _vp, _vp,
                                       _vp, _sz, _vp]
    lib.dllm_decode_verify.argtypes = [_i32, _i32, _i32, _vp, _i32, _vp, _i64, _vp, _f32, _vp, _vp, _vp,
                                       _vp, _vp, _sz, _vp]
    lib.dllm_set_tuning.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
    lib.dllm_sched_attention_noalloc.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                                 _i64, _vp, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _i32,
                                                 _i32, _vp, _vp]
    for name in ("dllm_set_tuning", "dllm_sched_attention_noalloc", "dllm_build_block_table", "dllm_map_slots", "dllm_qkv_rope_cachewrite",
                 "dllm_qkv_rope_cachewrite_paged", "dllm_qkv_project", "dllm_rope_apply", "dllm_cache_write",
                 "dllm_sched_attention", "dllm_topk_tracked", "dllm_confidence_argmax", "dllm_confidence_commit",
                 "dllm_verify_accept", "dllm_decode_commit", "dllm_decode_verify"):
        getattr(lib, name).restype = _i32
    _lib = lib
    return lib


def set_tuning(knob: str, value: Optional[str]) -> None:
    """Process-wide tuning override: knob "attn_splits" (a split count as
    text) or "qkv_kernel" (a projection kernel name); None restores the
    automatic choice."""
    _check("dllm_set_tuning", load().dllm_set_tuning(knob.encode(), None if value is None else str(value).encode()))


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise DllmError(fn, rc, load().dllm_status_string(rc).decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def cache_dtype_code(t, k_cache) -> int:
    """The dtype code of a call that takes caches: one-byte (uint8) caches
    hold E4M3 codes next to bf16 activations."""
    import torch
    if k_cache is not None and k_cache.dtype == torch.uint8:
        if t.dtype != torch.bfloat16:
            raise TypeError("E4M3 caches go with bf16 activations")
        return BF16_E4M3KV
    return dtype_code(t)


def version() -> int:
    return load().dllm_version()


def status_string(code: int) -> str:
    return load().dllm_status_string(code).decode()


# ---------------------------------------------------------------------------

def build_block_table(seq_pages, pool_perm, pool_pages: int, max_pages: int, page_table,
                      cu_q=None, q_logical=None, slot=None, page_size: int = PAGE, stream=None) -> None:
    """dllm_build_block_table: host seq_pages / pool_perm (/ cu_q, q_logical),
    device page_table int32[n_seq*max_pages] (and slot int32[n_rows])."""
    sp = np.ascontiguousarray(seq_pages, dtype=np.int32)
    perm = np.ascontiguousarray(pool_perm, dtype=np.int32)
    cu = None if cu_q is None else np.ascontiguousarray(cu_q, dtype=np.int32)
    lg = None if q_logical is None else np.ascontiguousarray(q_logical, dtype=np.int32)
    n_rows = 0 if cu is None else int(cu[-1])
    _check("dllm_build_block_table", load().dllm_build_block_table(
        len(sp), page_size, pool_pages, max_pages, _ptr(sp), _ptr(perm), _ptr(page_table),
        n_rows, _ptr(cu), _ptr(lg), _ptr(slot), _stream(stream)))


def map_slots(cu_q, q_logical, page_table, slot, max_pages: int, pool_pages: int,
              page_size: int = PAGE, stream=None) -> None:
    n_seq = cu_q.numel() - 1
    _check("dllm_map_slots", load().dllm_map_slots(
        n_seq, q_logical.numel(), page_size, max_pages, pool_pages, _ptr(cu_q), _ptr(q_logical),
        _ptr(page_table), _ptr(slot), _stream(stream)))


def qkv_rope_cachewrite_workspace(dt: int, n_rows: int, d_model: int, n_heads: int, head_dim: int) -> int:
    return int(load().dllm_qkv_rope_cachewrite_workspace(dt, n_rows, d_model, n_heads, head_dim))


def qkv_rope_cachewrite(x, w_qkv, pos, slot, q_out, k_cache, v_cache, n_heads: int, head_dim: int,
                        rope_base: float, workspace=None, stream=None) -> None:
    dt = cache_dtype_code(x, k_cache)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dllm_qkv_rope_cachewrite", load().dllm_qkv_rope_cachewrite(
        dt, x.shape[0], x.shape[1], n_heads, head_dim, float(rope_base), _ptr(x), _ptr(w_qkv),
        _ptr(pos), _ptr(slot), _ptr(q_out), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
        _ptr(workspace), ws_bytes, _stream(stream)))


def qkv_rope_cachewrite_paged(x, w_qkv, pos, cu_q, q_logical, page_table, max_pages: int, slot, q_out,
                              k_cache, v_cache, n_heads: int, head_dim: int, rope_base: float,
                              workspace=None, page_size: int = PAGE, stream=None) -> None:
    """qkv_rope_cachewrite with each row's cache slot formed from its logical
    position and the block table (written to slot as well)."""
    dt = cache_dtype_code(x, k_cache)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dllm_qkv_rope_cachewrite_paged", load().dllm_qkv_rope_cachewrite_paged(
        dt, cu_q.shape[0] - 1, x.shape[0], x.shape[1], n_heads, head_dim, float(rope_base), _ptr(x),
        _ptr(w_qkv), _ptr(pos), _ptr(cu_q), _ptr(q_logical), _ptr(page_table), max_pages, page_size,
        _ptr(slot), _ptr(q_out), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _ptr(workspace),
        ws_bytes, _stream(stream)))


def qkv_project(x, w_qkv, qkv_out, n_heads: int, head_dim: int, workspace=None, stream=None) -> None:
    """Unfused arm: unrotated q|k|v rows [R, 3*H*D]."""
    dt = dtype_code(x)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dllm_qkv_project", load().dllm_qkv_project(
        dt, x.shape[0], x.shape[1], n_heads, head_dim, _ptr(x), _ptr(w_qkv), _ptr(qkv_out),
        _ptr(workspace), ws_bytes, _stream(stream)))


def rope_apply(qkv, pos, q_out, n_heads: int, head_dim: int, rope_base: float, stream=None) -> None:
    """Unfused arm: q rotated into q_out, k rotated in place inside qkv."""
    _check("dllm_rope_apply", load().dllm_rope_apply(
        dtype_code(qkv), qkv.shape[0], n_heads, head_dim, float(rope_base), _ptr(pos), _ptr(qkv),
        _ptr(q_out), _stream(stream)))


def cache_write(qkv, slot, k_cache, v_cache, n_heads: int, head_dim: int, stream=None) -> None:
    """Unfused arm: qkv's k|v parts to their cache slots."""
    _check("dllm_cache_write", load().dllm_cache_write(
        dtype_code(qkv), qkv.shape[0], n_heads, head_dim, _ptr(qkv), _ptr(slot), _ptr(k_cache),
        _ptr(v_cache), k_cache.shape[0], _stream(stream)))


def sched_attention_workspace(dt: int, n_seq: int, n_rows: int, n_heads: int, head_dim: int,
                              max_kv: int, n_cap: int, max_mass_rows: int = 0) -> int:
    return int(load().dllm_sched_attention_workspace(dt, n_seq, n_rows, n_heads, head_dim, max_kv, n_cap,
                                                     max_mass_rows))


def sched_attention(q, cu_q, k_cache, v_cache, page_table, max_pages: int, kv_len, o, workspace,
                    n_heads: int, head_dim: int, max_kv: int, mask_bits=None, mask_off=None,
                    mass_count=None, max_mass_rows: int = 0, mass_accum=None, n_cap: int = 0,
                    page_size: int = PAGE, mass_overwrite: bool = False, stream=None) -> None:
    dt = cache_dtype_code(q, k_cache)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    mask_words = 0 if mask_bits is None else mask_bits.numel()
    _check("dllm_sched_attention", load().dllm_sched_attention(
        dt, cu_q.numel() - 1, q.shape[0], n_heads, head_dim, page_size, max_kv, _ptr(q), _ptr(cu_q),
        _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _ptr(page_table), max_pages, _ptr(kv_len),
        _ptr(mask_bits), _ptr(mask_off), mask_words, _ptr(mass_count), max_mass_rows,
        _ptr(mass_accum), int(bool(mass_overwrite)), n_cap, _ptr(o), _ptr(workspace), ws_bytes, _stream(stream)))


def sched_attention_noalloc(q, cu_q, k_cache, v_cache, page_table, max_pages: int, kv_len, o,
                            n_heads: int, head_dim: int, max_kv: int, mask_bits=None, mask_off=None,
                            mass_count=None, max_mass_rows: int = 0, mass_accum=None, n_cap: int = 0,
                            page_size: int = PAGE, mass_overwrite: bool = False, stream=None) -> None:
    """sched_attention with the library's static scratch array in place of a
    workspace (no device allocation by the call)."""
    dt = cache_dtype_code(q, k_cache)
    mask_words = 0 if mask_bits is None else mask_bits.numel()
    _check("dllm_sched_attention_noalloc", load().dllm_sched_attention_noalloc(
        dt, cu_q.numel() - 1, q.shape[0], n_heads, head_dim, page_size, max_kv, _ptr(q), _ptr(cu_q),
        _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _ptr(page_table), max_pages, _ptr(kv_len),
        _ptr(mask_bits), _ptr(mask_off), mask_words, _ptr(mass_count), max_mass_rows,
        _ptr(mass_accum), int(bool(mass_overwrite)), n_cap, _ptr(o), _stream(stream)))


def topk_tracked(mass, eligible, k: int, idx, val, count, clear_mass: bool = False, stream=None) -> None:
    """mass: float32 [n_seq, n_heads, n_cap] per-head scores."""
    n_seq, n_heads, n_cap = mass.shape
    _check("dllm_topk_tracked", load().dllm_topk_tracked(
        n_seq, n_heads, n_cap, k, _ptr(mass), _ptr(eligible), _ptr(idx), _ptr(val), _ptr(count),
        1 if clear_mass else 0, _stream(stream)))


def pack_mask(visible: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Boolean [rows_b, kv_b] matrices -> (uint32 words, int64 word offset per
    sequence) in the layout dllm_sched_attention reads: bit j%32 of word
    off[b] + i*ceil(kv_b/32) + j/32 is row i's visibility of key j."""
    words: List[np.ndarray] = []
    offs = []
    total = 0
    for v in visible:
        v = np.asarray(v, dtype=bool)
        rows, kv = v.shape
        w = (kv + 31) // 32
        pad = np.zeros((rows, w * 32), dtype=bool)
        pad[:, :kv] = v
        packed = np.packbits(pad.reshape(rows, w, 32), axis=2, bitorder="little")
        words.append(packed.reshape(rows, w, 4).view(np.uint32).reshape(-1))
        offs.append(total)
        total += rows * w
    return np.concatenate(words).astype(np.uint32), np.asarray(offs, dtype=np.int64)


# ---------------------------------------------------------------------------
# Decode side: logits rows [R, >= vocab] (bf16 or fp32, rows may be strided).

def confidence_workspace(n_rows: int, vocab: int) -> int:
    return int(load().dllm_confidence_workspace(n_rows, vocab))


def _logits_args(logits, vocab: Optional[int]):
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-d with unit column stride")
    v = logits.shape[1] if vocab is None else int(vocab)
    return dtype_code(logits), logits.shape[0], v, logits.stride(0)


def confidence_argmax(logits, token, conf, workspace, vocab: Optional[int] = None, stream=None) -> None:
    """Per row: argmax token (lowest id on ties) and max softmax probability."""
    dt, R, V, stride = _logits_args(logits, vocab)
    _check("dllm_confidence_argmax", load().dllm_confidence_argmax(
        dt, R, V, _ptr(logits), stride, _ptr(token), _ptr(conf), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))


def confidence_commit(cu_rows, conf, eps: float, commit, n_commit, stream=None) -> None:
    _check("dllm_confidence_commit", load().dllm_confidence_commit(
        cu_rows.numel() - 1, conf.numel(), _ptr(cu_rows), _ptr(conf), float(eps), _ptr(commit), _ptr(n_commit),
        _stream(stream)))


def verify_accept(cu_rows, draft, token, conf, gamma: float, accept, n_accept, stream=None) -> None:
    _check("dllm_verify_accept", load().dllm_verify_accept(
        cu_rows.numel() - 1, conf.numel(), _ptr(cu_rows), _ptr(draft), _ptr(token), _ptr(conf), float(gamma),
        _ptr(accept), _ptr(n_accept), _stream(stream)))


def decode_commit(logits, cu_rows, eps: float, token, conf, commit, n_commit, workspace,
                  vocab: Optional[int] = None, stream=None) -> None:
    dt, R, V, stride = _logits_args(logits, vocab)
    _check("dllm_decode_commit", load().dllm_decode_commit(
        dt, cu_rows.numel() - 1, R, _ptr(cu_rows), V, _ptr(logits), stride, float(eps), _ptr(token), _ptr(conf),
        _ptr(commit), _ptr(n_commit), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_verify(logits, cu_rows, draft, gamma: float, token, conf, accept, n_accept, workspace,
                  vocab: Optional[int] = None, stream=None) -> None:
    dt, R, V, stride = _logits_args(logits, vocab)
    _check("dllm_decode_verify", load().dllm_decode_verify(
        dt, cu_rows.numel() - 1, R, _ptr(cu_rows), V, _ptr(logits), stride, _ptr(draft), float(gamma),
        _ptr(token), _ptr(conf), _ptr(accept), _ptr(n_accept), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
