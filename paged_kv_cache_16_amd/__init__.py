"""paged_kv_cache_16_amd — Python binding of libpagedkv.so (MI355X / gfx950).

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. Importing this
package fails loudly when the library has not been built; there is no fallback.

Cache tensors are allocated by the caller as ``[num_blocks, num_kv_heads, block_size,
head_dim]`` of the cache dtype; the library stores elements inside each page in its own
"lane-chunk" order (documented in include/pagedkv.h), so the tensor is a byte container:
only ``kv_cache_append`` writes it and only the attention calls read it.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

__all__ = [
    "kv_cache_append", "paged_decode_attention", "paged_decode_append_attention", "paged_decode_attention_noalloc",
    "paged_decode_attention_partial",
    "paged_decode_combine", "workspace_size", "num_splits", "kv_cache_bytes", "status_string",
    "select_pages", "new_cache", "BlockManager", "ring_pages", "policy_blocks", "device_errors",
    "read_probe", "profile_events", "prepare_decode_append_attention", "PreparedCall",
    "PagedKVError", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_cache_16_amd/build.py` "
                      "(hipcc, gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", _i32), ("block_size", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("dtype", ctypes.c_int), ("input_dtype", ctypes.c_int)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("window", _i32), ("num_sinks", _i32), ("page_list", _vp),
                ("pages_per_seq", _i32), ("split_tokens", _i32), ("score_acc", _vp), ("score_stride", _i32),
                ("score_block", _i32), ("ring_pages", _i32)]


class LayerGroup(ctypes.Structure):
    _fields_ = [("window", _i32), ("num_sinks", _i32), ("ring_pages", _i32), ("num_blocks", _i32)]


_P_DESC = ctypes.POINTER(CacheDesc)
_P_OPTS = ctypes.POINTER(DecodeOpts)

_lib.kv_cache_append.restype = ctypes.c_int
_lib.kv_cache_append.argtypes = [_P_DESC, _vp, _vp, _vp, _vp, _vp, _i32, _vp]
_lib.paged_decode_attention.restype = ctypes.c_int
_lib.paged_decode_attention.argtypes = [_P_DESC, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                                        _P_OPTS, _vp, ctypes.c_int, _vp, _vp, _sz, _vp]
_lib.paged_decode_append_attention.restype = ctypes.c_int
_lib.paged_decode_append_attention.argtypes = [_P_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                               _i32, _i32, _f32, _P_OPTS, _vp, ctypes.c_int, _vp, _vp, _sz,
                                               _vp]
_lib.paged_decode_attention_noalloc.restype = ctypes.c_int
_lib.paged_decode_attention_noalloc.argtypes = [_P_DESC, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                                                _P_OPTS, _vp, ctypes.c_int, _vp, _vp]
_lib.paged_decode_attention_workspace_size.restype = _sz
_lib.paged_decode_attention_workspace_size.argtypes = [_P_DESC, _i32, _i32, _i32, _P_OPTS]
_lib.paged_decode_attention_num_splits.restype = _i32
_lib.paged_decode_attention_num_splits.argtypes = [_P_DESC, _i32, _i32, _P_OPTS]
_lib.paged_decode_attention_partial.restype = ctypes.c_int
_lib.paged_decode_attention_partial.argtypes = [_P_DESC, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                                _f32, _P_OPTS, _vp, _vp, _vp, _i32, _vp]
_lib.paged_decode_combine.restype = ctypes.c_int
_lib.paged_decode_combine.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, ctypes.c_int, _vp, _vp]
_lib.paged_select_pages.restype = ctypes.c_int
_lib.paged_select_pages.argtypes = [_vp, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp]
_lib.pkv_kv_cache_bytes.restype = ctypes.c_uint64
_lib.pkv_kv_cache_bytes.argtypes = [_i64] * 7
_lib.pkv_ring_pages.restype = _i32
_lib.pkv_ring_pages.argtypes = [_i32, _i32]
_lib.pkv_policy_blocks.restype = _i64
_lib.pkv_policy_blocks.argtypes = [_i64, _i32, _i32, _i32, _i32]
_lib.pkv_bm_create.restype = ctypes.c_int
_lib.pkv_bm_create.argtypes = [_i32, _i32, _i32, ctypes.POINTER(LayerGroup), _i32, ctypes.POINTER(_vp)]
_lib.pkv_bm_destroy.restype = None
_lib.pkv_bm_destroy.argtypes = [_vp]
_lib.pkv_bm_table_cols.restype = _i32
_lib.pkv_bm_table_cols.argtypes = [_vp, _i32]
_lib.pkv_bm_ring_pages.restype = _i32
_lib.pkv_bm_ring_pages.argtypes = [_vp, _i32]
_lib.pkv_bm_append.restype = ctypes.c_int
_lib.pkv_bm_append.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp]
_lib.pkv_bm_release.restype = ctypes.c_int
_lib.pkv_bm_release.argtypes = [_vp, _i32]
_lib.pkv_bm_block_tables.restype = ctypes.c_int
_lib.pkv_bm_block_tables.argtypes = [_vp, _i32, _vp, _i32, _vp]
_lib.pkv_bm_context_len.restype = _i64
_lib.pkv_bm_context_len.argtypes = [_vp, _i32]
_lib.pkv_bm_blocks_in_use.restype = _i64
_lib.pkv_bm_blocks_in_use.argtypes = [_vp, _i32]
_lib.pkv_device_errors.restype = ctypes.c_int
_lib.pkv_device_errors.argtypes = [_vp, _i32, _vp]
_lib.pkv_read_probe.restype = ctypes.c_int
_lib.pkv_read_probe.argtypes = [_vp, ctypes.c_size_t, _i32, _vp, ctypes.c_size_t, _vp, _vp]
_lib.pkv_profile_events.restype = ctypes.c_int
_lib.pkv_profile_events.argtypes = [_vp, _vp]
_lib.pkv_status_string.restype = ctypes.c_char_p
_lib.pkv_status_string.argtypes = [ctypes.c_int]

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return _lib.pkv_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(fn, status)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


# Shape checks. The C ABI takes raw pointers and sizes, so a tensor smaller than the call
# implies would be read or written past its end; every wrapper checks the tensors it passes
# against the sizes it passes before anything is enqueued (ValueError, nothing launched).
def _need(ok: bool, msg: str) -> None:
    if not ok:
        raise ValueError(msg)


def _shape(t, name: str, shape) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(tuple(t.shape) == tuple(shape), f"{name} must be shaped {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t, name: str, ndim: int, rows: int) -> None:
    """t has ndim dimensions and at least `rows` rows (entries past them are never read)."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.dim() == ndim, f"{name} must have {ndim} dimension(s), got {t.dim()}")
    _need(t.shape[0] >= rows, f"{name} must have at least {rows} rows, got {t.shape[0]}")


def _cache_pair(k_cache, v_cache) -> None:
    _need(isinstance(k_cache, torch.Tensor) and isinstance(v_cache, torch.Tensor), "caches must be tensors")
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype,
          f"k_cache and v_cache must match, got {tuple(k_cache.shape)} {k_cache.dtype} and "
          f"{tuple(v_cache.shape)} {v_cache.dtype}")


def _decode_shapes(desc, q, k_cache, v_cache, block_table, context_lens, page_list, out, lse, scores):
    """Checks of a decode call's tensors against (B, Hq, d) taken from q."""
    _cache_pair(k_cache, v_cache)
    _need(isinstance(q, torch.Tensor) and q.dim() == 3, "q must be [batch, num_q_heads, head_dim]")
    B, Hq, d = q.shape
    _need(d == desc.head_dim, f"q's head_dim {d} differs from the cache's {desc.head_dim}")
    _rows(block_table, "block_table", 2, B)
    _need(block_table.shape[1] >= 1 or B == 0, "block_table needs at least one column")
    _rows(context_lens, "context_lens", 1, B)
    if page_list is not None:
        _rows(page_list, "page_list", 2, B)
        _need(page_list.shape[1] >= 1, "page_list needs at least one column")
    if out is not None:
        _shape(out, "out", (B, Hq, d))
    if lse is not None:
        _shape(lse, "lse", (B, Hq))
    if scores is not None:
        _need(isinstance(scores, torch.Tensor) and scores.dim() == 3,
              "scores must be a [batch, num_kv_heads, stride] tensor")
        _need(scores.shape[0] >= B and scores.shape[1] == desc.num_kv_heads,
              f"scores must be [>= {B}, {desc.num_kv_heads}, stride], got {tuple(scores.shape)}")
    return B, Hq, d


def cache_desc(k_cache: torch.Tensor, input_dtype=None) -> CacheDesc:
    """Descriptor of a cache tensor. An INT8 cache is a torch.int8 tensor
    [num_blocks, num_kv_heads, block_size, head_dim + 4] holding the int8 data plane followed
    by the fp32 scale plane (see new_cache); input_dtype is then the type of q and of the
    appended rows (bf16 by default)."""
    if k_cache.dim() != 4:
        raise ValueError("cache tensors are [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, P, d = k_cache.shape
    if k_cache.dtype == torch.int8:
        ind = DTYPE_CODE.get(input_dtype or torch.bfloat16)
        if ind not in (1, 2):
            raise ValueError("an INT8 cache takes bf16 or fp16 inputs")
        return CacheDesc(nb, P, hkv, d - 4, 3, ind)
    if k_cache.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    return CacheDesc(nb, P, hkv, d, DTYPE_CODE[k_cache.dtype], 0)


def input_dtype_of(k_cache: torch.Tensor, other: torch.Tensor | None = None):
    """Type of q / appended rows for this cache (the cache's own, or other's for INT8)."""
    if k_cache.dtype == torch.int8:
        return other.dtype if other is not None else torch.bfloat16
    return k_cache.dtype


def new_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype, device="cuda"):
    """An uninitialised cache tensor. dtype torch.int8 gives an INT8 cache: int8 data plane
    plus fp32 scale plane, shaped [num_blocks, num_kv_heads, block_size, head_dim + 4]."""
    if dtype == torch.int8:
        return torch.empty((num_blocks, num_kv_heads, block_size, head_dim + 4), dtype=torch.int8, device=device)
    return torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)


def _opts(window=0, num_sinks=0, page_list=None, split_tokens=0, scores=None,
          score_block=1, ring_pages=0) -> DecodeOpts:
    o = DecodeOpts(int(window), int(num_sinks), None, 0, int(split_tokens), None, 0,
                   int(score_block), int(ring_pages))
    if page_list is not None:
        o.page_list = _dev(page_list, "page_list", torch.int32)
        o.pages_per_seq = page_list.shape[1]
    if scores is not None:
        # [B, Hkv, stride] fp32, accumulated in place
        if scores.dim() != 3 or scores.dtype != torch.float32 or not scores.is_contiguous():
            raise ValueError("scores must be a contiguous [batch, num_kv_heads, stride] float32 tensor")
        o.score_acc = _dev(scores, "scores", torch.float32)
        o.score_stride = scores.shape[2]
    return o


def profile_events(start=None, stop=None) -> None:
    """Profiling hook: raw hipEvent_t handles (ints) that this thread's later decode calls record
    around their main attention kernel; profile_events() clears them."""
    _lib.pkv_profile_events(None if start is None else int(start), None if stop is None else int(stop))


def _set_timing(timing) -> None:
    # a call's timing=(start, stop) sets the thread's hook for that call; timing=None clears it
    if timing is None:
        _lib.pkv_profile_events(None, None)
    else:
        _lib.pkv_profile_events(int(timing[0]), int(timing[1]))


def kv_cache_append(k_cache, v_cache, k_new, v_new, slot_mapping) -> None:
    """Scatter k_new/v_new [N, Hkv, d] into the pools at slot_mapping[N] (int32, <0 = skip)."""
    desc = cache_desc(k_cache, k_new.dtype)
    _cache_pair(k_cache, v_cache)
    _need(isinstance(slot_mapping, torch.Tensor) and slot_mapping.dim() == 1, "slot_mapping must be [N]")
    n = slot_mapping.numel()
    _shape(k_new, "k_new", (n, desc.num_kv_heads, desc.head_dim))
    _shape(v_new, "v_new", (n, desc.num_kv_heads, desc.head_dim))
    _check("kv_cache_append", _lib.kv_cache_append(
        ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(k_new, "k_new", input_dtype_of(k_cache, k_new)), _dev(v_new, "v_new", input_dtype_of(k_cache, k_new)),
        _dev(slot_mapping, "slot_mapping", torch.int32), n, _stream(k_cache)))


def workspace_size(k_cache, batch: int, num_q_heads: int, max_context_len: int, *, window=0,
                   num_sinks=0, page_list=None, split_tokens=0, scores=False, score_block=1, ring_pages=0) -> int:
    """scores: True (or the score tensor) when the calls export scores, with entries of
    score_block tokens (the path, and so the size, can depend on it)."""
    desc = cache_desc(k_cache)
    o = _opts(window, num_sinks, None, split_tokens, score_block=score_block, ring_pages=ring_pages)
    if page_list is not None:
        o.page_list = ctypes.c_void_p(1)  # only its presence matters to the size
        o.pages_per_seq = page_list.shape[1]
    if scores is not None and scores is not False:
        o.score_acc = ctypes.c_void_p(1)
    return int(_lib.paged_decode_attention_workspace_size(ctypes.byref(desc), batch, num_q_heads,
                                                          max_context_len, ctypes.byref(o)))


def num_splits(k_cache, batch: int, max_context_len: int, *, window=0, num_sinks=0, page_list=None,
               split_tokens: int = 0, ring_pages: int = 0) -> int:
    desc = cache_desc(k_cache)
    o = _opts(window, num_sinks, None, split_tokens, ring_pages=ring_pages)
    if page_list is not None:
        o.page_list = ctypes.c_void_p(1)
        o.pages_per_seq = page_list.shape[1]
    return int(_lib.paged_decode_attention_num_splits(ctypes.byref(desc), batch, max_context_len,
                                                      ctypes.byref(o)))


def paged_decode_attention(q, k_cache, v_cache, block_table, context_lens, *, max_context_len: int,
                           scale: float = 0.0, window: int = 0, num_sinks: int = 0, page_list=None,
                           split_tokens: int = 0, out=None, out_dtype=None, lse=None, workspace=None,
                           want_lse: bool = True, timing=None, scores=None, score_block: int = 1,
                           ring_pages: int = 0):
    """One decode query per sequence over its paged cache. Returns (out, lse).

    ring_pages > 0: block_table holds a window layer's ring rows (BlockManager.block_table of a
    window group, with window/num_sinks of that group).

    timing: optional pair of raw hipEvent_t handles recorded around the main kernel (the
    library's per-thread profiling hook, set for this call).
    scores: optional [B, Hkv, stride] float32 tensor; every attended token's softmax
    probability, summed over the query heads of its kv head, is added into entry
    t // score_block (score_block = 1: per token; = the page size: per page)."""
    desc = cache_desc(k_cache, q.dtype)
    B, Hq, d = _decode_shapes(desc, q, k_cache, v_cache, block_table, context_lens, page_list, out, lse, scores)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    o = _opts(window, num_sinks, page_list, split_tokens, scores, score_block, ring_pages)
    ws_bytes = int(_lib.paged_decode_attention_workspace_size(ctypes.byref(desc), B, Hq, max_context_len,
                                                              ctypes.byref(o)))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _set_timing(timing)
    _check("paged_decode_attention", _lib.paged_decode_attention(
        ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(q, "q", input_dtype_of(k_cache, q)), _dev(block_table, "block_table", torch.int32),
        block_table.shape[1], _dev(context_lens, "context_lens", torch.int32), B, Hq,
        int(max_context_len), float(scale), ctypes.byref(o), _dev(out, "out"), DTYPE_CODE[out.dtype],
        _dev(lse, "lse", torch.float32) if lse is not None else None, ws_ptr, ws_n, _stream(q)))
    return out, lse


NOALLOC_SCRATCH_BYTES = 32 << 20  # the library's per-device scratch for paged_decode_attention_noalloc


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_table, context_lens, *, max_context_len: int,
                                   out, lse=None, scale: float = 0.0, window: int = 0, num_sinks: int = 0,
                                   page_list=None, split_tokens: int = 0, scores=None, score_block: int = 1,
                                   ring_pages: int = 0):
    """paged_decode_attention without a workspace: the library's own per-device scratch serves
    instead, so the call allocates nothing (out, and lse if wanted, are the caller's). Calls that
    overlap in time on one device race on that scratch. Returns (out, lse)."""
    desc = cache_desc(k_cache, q.dtype)
    B, Hq, d = _decode_shapes(desc, q, k_cache, v_cache, block_table, context_lens, page_list, out, lse, scores)
    _need(out is not None, "out is required (the call allocates nothing)")
    o = _opts(window, num_sinks, page_list, split_tokens, scores, score_block, ring_pages)
    _check("paged_decode_attention_noalloc", _lib.paged_decode_attention_noalloc(
        ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(q, "q", input_dtype_of(k_cache, q)), _dev(block_table, "block_table", torch.int32),
        block_table.shape[1], _dev(context_lens, "context_lens", torch.int32), B, Hq,
        int(max_context_len), float(scale), ctypes.byref(o), _dev(out, "out"), DTYPE_CODE[out.dtype],
        _dev(lse, "lse", torch.float32) if lse is not None else None, _stream(q)))
    return out, lse


def _fused_args(q, k_cache, v_cache, k_new, v_new, slot_mapping, block_table, context_lens, max_context_len,
                scale, window, num_sinks, page_list, split_tokens, out, out_dtype, lse, workspace, want_lse, scores,
                score_block, ring_pages):
    """Checks and marshals a paged_decode_append_attention call: (C arguments, out, lse, tensors
    to keep alive)."""
    desc = cache_desc(k_cache, q.dtype)
    B, Hq, d = _decode_shapes(desc, q, k_cache, v_cache, block_table, context_lens, page_list, out, lse, scores)
    # one new token per sequence
    _shape(k_new, "k_new", (B, desc.num_kv_heads, desc.head_dim))
    _shape(v_new, "v_new", (B, desc.num_kv_heads, desc.head_dim))
    _need(isinstance(slot_mapping, torch.Tensor) and slot_mapping.dim() == 1 and slot_mapping.numel() == B,
          f"slot_mapping must be [{B}]")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    o = _opts(window, num_sinks, page_list, split_tokens, scores, score_block, ring_pages)
    ws_bytes = int(_lib.paged_decode_attention_workspace_size(ctypes.byref(desc), B, Hq, max_context_len,
                                                              ctypes.byref(o)))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(k_new, "k_new", input_dtype_of(k_cache, k_new)), _dev(v_new, "v_new", input_dtype_of(k_cache, k_new)),
            _dev(slot_mapping, "slot_mapping", torch.int32), _dev(q, "q", input_dtype_of(k_cache, q)),
            _dev(block_table, "block_table", torch.int32), block_table.shape[1],
            _dev(context_lens, "context_lens", torch.int32), B, Hq, int(max_context_len), float(scale),
            ctypes.byref(o), _dev(out, "out"), DTYPE_CODE[out.dtype],
            _dev(lse, "lse", torch.float32) if lse is not None else None, ws_ptr, ws_n, _stream(q))
    keep = (desc, o, q, k_cache, v_cache, k_new, v_new, slot_mapping, block_table, context_lens, page_list, scores,
            workspace)
    return args, out, lse, keep


def paged_decode_append_attention(q, k_cache, v_cache, k_new, v_new, slot_mapping, block_table,
                                  context_lens, *, max_context_len: int, scale: float = 0.0,
                                  window: int = 0, num_sinks: int = 0, page_list=None,
                                  split_tokens: int = 0, out=None, out_dtype=None, lse=None,
                                  workspace=None, want_lse: bool = True, timing=None, scores=None,
                                  score_block: int = 1, ring_pages: int = 0):
    """One decode step of one layer: append of row b of k_new/v_new ([B, Hkv, d]) at
    slot_mapping[b] (position context_lens[b] - 1), then attention. Returns (out, lse).
    scores: as in paged_decode_attention."""
    args, out, lse, _ = _fused_args(q, k_cache, v_cache, k_new, v_new, slot_mapping, block_table, context_lens,
                                    max_context_len, scale, window, num_sinks, page_list, split_tokens, out,
                                    out_dtype, lse, workspace, want_lse, scores, score_block, ring_pages)
    _set_timing(timing)
    _check("paged_decode_append_attention", _lib.paged_decode_append_attention(*args))
    return out, lse


class PreparedCall:
    """A decode call checked and marshalled once, for loops that repeat it: each call makes the
    one library call again, with the same tensors (their contents at that time) on the stream
    that was current when it was prepared, and returns (out, lse). It holds its tensors (and the
    workspace) alive."""
    __slots__ = ("_fn", "_args", "_name", "out", "lse", "_keep")

    def __init__(self, name, fn, args, out, lse, keep):
        self._name, self._fn, self._args, self.out, self.lse, self._keep = name, fn, args, out, lse, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise PagedKVError(self._name, st)
        return self.out, self.lse


def prepare_decode_append_attention(q, k_cache, v_cache, k_new, v_new, slot_mapping, block_table, context_lens,
                                    *, max_context_len: int, scale: float = 0.0, window: int = 0,
                                    num_sinks: int = 0, page_list=None, split_tokens: int = 0, out=None,
                                    out_dtype=None, lse=None, workspace=None, want_lse: bool = True, scores=None,
                                    score_block: int = 1, ring_pages: int = 0) -> PreparedCall:
    """paged_decode_append_attention checked and marshalled once (same arguments); calling the
    result runs the step. The workspace, out and lse are allocated here when not given."""
    args, out, lse, keep = _fused_args(q, k_cache, v_cache, k_new, v_new, slot_mapping, block_table, context_lens,
                                       max_context_len, scale, window, num_sinks, page_list, split_tokens, out,
                                       out_dtype, lse, workspace, want_lse, scores, score_block, ring_pages)
    return PreparedCall("paged_decode_append_attention", _lib.paged_decode_append_attention, args, out, lse, keep)


def paged_decode_attention_partial(q, k_cache, v_cache, block_table, context_lens, *,
                                   max_context_len: int, split_tokens: int = 0, scale: float = 0.0,
                                   window: int = 0, num_sinks: int = 0, page_list=None,
                                   o_part=None, m_part=None, l_part=None, ring_pages: int = 0):
    """Split-K partials (o [B,Hq,S,d], m [B,Hq,S], l [B,Hq,S], fp32) over explicit partitions."""
    desc = cache_desc(k_cache, q.dtype)
    B, Hq, d = _decode_shapes(desc, q, k_cache, v_cache, block_table, context_lens, page_list, None, None, None)
    o = _opts(window, num_sinks, page_list, split_tokens, ring_pages=ring_pages)
    S = int(_lib.paged_decode_attention_num_splits(ctypes.byref(desc), B, max_context_len, ctypes.byref(o)))
    if S <= 0:
        raise ValueError("invalid partition request")
    if o_part is None and m_part is None and l_part is None:
        o_part = torch.empty((B, Hq, S, d), dtype=torch.float32, device=q.device)
        m_part = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
        l_part = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _shape(o_part, "o_part", (B, Hq, S, d))
    _shape(m_part, "m_part", (B, Hq, S))
    _shape(l_part, "l_part", (B, Hq, S))
    _check("paged_decode_attention_partial", _lib.paged_decode_attention_partial(
        ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(q, "q", input_dtype_of(k_cache, q)), _dev(block_table, "block_table", torch.int32),
        block_table.shape[1], _dev(context_lens, "context_lens", torch.int32), B, Hq,
        int(max_context_len), float(scale), ctypes.byref(o), _dev(o_part, "o_part", torch.float32),
        _dev(m_part, "m_part", torch.float32), _dev(l_part, "l_part", torch.float32), S, _stream(q)))
    return o_part, m_part, l_part


def paged_decode_combine(o_part, m_part, l_part, *, out=None, out_dtype=torch.float32, lse=None,
                         want_lse: bool = True):
    """Log-sum-exp merge of split partials into (out [B,Hq,d], lse [B,Hq])."""
    _need(isinstance(o_part, torch.Tensor) and o_part.dim() == 4, "o_part must be [batch, num_q_heads, splits, d]")
    B, Hq, S, d = o_part.shape
    _shape(m_part, "m_part", (B, Hq, S))
    _shape(l_part, "l_part", (B, Hq, S))
    if out is not None:
        _shape(out, "out", (B, Hq, d))
    if lse is not None:
        _shape(lse, "lse", (B, Hq))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=o_part.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=o_part.device)
    _check("paged_decode_combine", _lib.paged_decode_combine(
        _dev(o_part, "o_part", torch.float32), _dev(m_part, "m_part", torch.float32),
        _dev(l_part, "l_part", torch.float32), B, Hq, S, d, _dev(out, "out"), DTYPE_CODE[out.dtype],
        _dev(lse, "lse", torch.float32) if lse is not None else None, _stream(o_part)))
    return out, lse


def select_pages(scores, context_lens, *, block_size: int, k: int, recent: int = 1, page_list=None):
    """Next step's page lists [B, k] int32 from page scores [B, heads, stride] float32: the
    newest `recent` pages plus the k - recent older pages of largest weight (sum over heads),
    ascending, -1 padded."""
    if scores.dim() != 3 or scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous [batch, heads, stride] float32 tensor")
    B, H, stride = scores.shape
    _rows(context_lens, "context_lens", 1, B)
    if page_list is None:
        page_list = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    _shape(page_list, "page_list", (B, k))
    _check("paged_select_pages", _lib.paged_select_pages(
        _dev(scores, "scores", torch.float32), H, stride, _dev(context_lens, "context_lens", torch.int32), B,
        int(block_size), int(k), int(recent), _dev(page_list, "page_list", torch.int32), _stream(scores)))
    return page_list


def ring_pages(window: int, block_size: int) -> int:
    """Least ring size of a window layer: the most pages `window` consecutive tokens touch."""
    return int(_lib.pkv_ring_pages(int(window), int(block_size)))


def policy_blocks(context_len: int, block_size: int, window: int = 0, num_sinks: int = 0,
                  ring_pages: int = 0) -> int:
    """Blocks one sequence holds in one layer under its policy (full: one per page)."""
    n = int(_lib.pkv_policy_blocks(int(context_len), int(block_size), int(window), int(num_sinks),
                                   int(ring_pages)))
    if n < 0:
        raise ValueError("policy_blocks: bad arguments")
    return n


def _host_i32(a, name):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if a.ndim != 1:
        raise ValueError(f"{name} must be one-dimensional")
    return a


class BlockManager:
    """Host block manager of the per-layer memory policy (pkv_bm_* in libpagedkv): per group of
    layers sharing a policy, a free list of block ids and one block-table row per sequence
    (a ring for window groups). groups: dicts with window (0: full cache), num_sinks, ring_pages
    (0: the least size) and num_blocks."""

    def __init__(self, block_size: int, max_seqs: int, max_pages_per_seq: int, groups):
        arr = (LayerGroup * len(groups))()
        for i, g in enumerate(groups):
            arr[i] = LayerGroup(int(g.get("window", 0)), int(g.get("num_sinks", 0)), int(g.get("ring_pages", 0)),
                                int(g["num_blocks"]))
        h = _vp()
        _check("pkv_bm_create", _lib.pkv_bm_create(int(block_size), int(max_seqs), int(max_pages_per_seq), arr,
                                                   len(groups), ctypes.byref(h)))
        self._h = h
        self.block_size = int(block_size)
        self.num_groups = len(groups)

    def close(self, _destroy=_lib.pkv_bm_destroy) -> None:
        # the destroy function is bound at definition time: __del__ may run at interpreter exit
        if getattr(self, "_h", None):
            _destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def table_cols(self, group: int) -> int:
        return int(_lib.pkv_bm_table_cols(self._h, int(group)))

    def ring_pages(self, group: int) -> int:
        return int(_lib.pkv_bm_ring_pages(self._h, int(group)))

    def append(self, seq_ids, num_new=None):
        """Adds num_new[i] tokens (default 1) to sequence seq_ids[i]. Returns (slots
        [num_groups, T] int32 — -1 for a window group's tokens already out of its window —, new
        context lengths [n] int32), numpy arrays."""
        ids = _host_i32(seq_ids, "seq_ids")
        cnt = None if num_new is None else _host_i32(num_new, "num_new")
        if cnt is not None and cnt.size != ids.size:
            raise ValueError("num_new must match seq_ids")
        T = ids.size if cnt is None else int(cnt.astype(np.int64).sum())
        slots = np.empty((self.num_groups, max(T, 0)), np.int32)
        lens = np.empty(ids.size, np.int32)
        _check("pkv_bm_append", _lib.pkv_bm_append(
            self._h, ids.ctypes.data if ids.size else None, None if cnt is None else cnt.ctypes.data, ids.size,
            slots.ctypes.data if slots.size else None, lens.ctypes.data if lens.size else None))
        return slots, lens

    def release(self, seq_id: int) -> None:
        _check("pkv_bm_release", _lib.pkv_bm_release(self._h, int(seq_id)))

    def block_table(self, group: int, seq_ids):
        """[n, table_cols(group)] int32 numpy rows (-1 where no block is held)."""
        ids = _host_i32(seq_ids, "seq_ids")
        out = np.empty((ids.size, self.table_cols(group)), np.int32)
        _check("pkv_bm_block_tables", _lib.pkv_bm_block_tables(
            self._h, int(group), ids.ctypes.data if ids.size else None, ids.size,
            out.ctypes.data if out.size else None))
        return out

    def context_len(self, seq_id: int) -> int:
        return int(_lib.pkv_bm_context_len(self._h, int(seq_id)))

    def blocks_in_use(self, group: int) -> int:
        return int(_lib.pkv_bm_blocks_in_use(self._h, int(group)))


DEV_BLOCK_ID, DEV_SLOT, DEV_CONTEXT, DEV_PAGES = 1, 2, 4, 8


def device_errors(clear: bool = True, stream=None) -> int:
    """The current device's error word (an OR of the DEV_* bits the kernels set when they skip a
    violated device-side precondition); waits for the stream (default: torch's current one)."""
    flags = ctypes.c_uint32(0)
    st = torch.cuda.current_stream().cuda_stream if stream is None else int(stream)
    _check("pkv_device_errors", _lib.pkv_device_errors(ctypes.byref(flags), 1 if clear else 0, st))
    return int(flags.value)


def read_probe(buf, waves_per_simd: int, sink) -> int:
    """Enqueues the read-rate probe over the device tensor `buf` on torch's current stream
    (sink: a device int32/uint32 tensor of at least CUs * 4 * waves_per_simd entries); returns
    the number of bytes the launch reads."""
    if not buf.is_cuda or not sink.is_cuda or sink.dtype not in (torch.int32, torch.uint32):
        raise ValueError("buf and sink must be device tensors, sink 32-bit")
    n = ctypes.c_size_t(0)
    _check("pkv_read_probe", _lib.pkv_read_probe(
        ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), int(waves_per_simd),
        ctypes.c_void_p(sink.data_ptr()), sink.numel(), ctypes.byref(n), _stream(buf)))
    return int(n.value)


def kv_cache_bytes(batch, layers, kv_heads, head_dim, seq_len, dtype_bytes, block_size=0) -> int:
    return int(_lib.pkv_kv_cache_bytes(batch, layers, kv_heads, head_dim, seq_len, dtype_bytes,
                                       block_size))


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
