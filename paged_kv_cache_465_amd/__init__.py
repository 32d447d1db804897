"""Paged KV cache and paged decode attention for AMD MI355X (gfx950).

A thin Python binding over libkvp.so, whose C ABI (include/kvp.h) holds the
whole path: the host page pool, kv_append and paged_attention_decode with
their HIP kernels.  The functions below carry the C entry points' names and
only marshal arguments: torch tensors supply device pointers and the current
HIP stream.  There is no fallback: if libkvp.so is missing, import fails.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import DecodePlan, PoolDesc, ScheduleInfo

_L = _lib.load()

KVP_OK, KVP_E_INVAL, KVP_E_NOPAGES, KVP_E_UNSUPPORTED, KVP_E_HIP, KVP_E_SCRATCH = range(6)
KVP_BF16, KVP_INT8, KVP_INT4, KVP_FP8 = 0, 1, 2, 3
_DTYPES = {"bf16": KVP_BF16, "int8": KVP_INT8, "int4": KVP_INT4, "fp8": KVP_FP8}
_DTYPE_NAMES = {v: k for k, v in _DTYPES.items()}


class KvpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvp_status_string(status)} (status {status})")


def _check(status: int, where: str) -> None:
    if status != KVP_OK:
        raise KvpError(status, where)


def kvp_status_string(status: int) -> str:
    return _L.kvp_status_string(status).decode()


def make_desc(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
              dtype="bf16") -> PoolDesc:
    return PoolDesc(num_pages, page_size, num_kv_heads, head_dim,
                    _DTYPES.get(dtype, dtype) if isinstance(dtype, str) else int(dtype))


class Pool:
    """Owner of one host pool object (kvp_pool_create / kvp_pool_destroy)."""

    def __init__(self, handle: int, desc: PoolDesc):
        self.handle = ctypes.c_void_p(handle)
        self.desc = desc

    @property
    def dtype(self) -> str:
        return _DTYPE_NAMES[self.desc.dtype]

    @property
    def elem_bytes(self) -> int:
        """Element size of the device tensors that hold the K/V pools: bfloat16
        pools are 2-byte words, code pools are bytes."""
        return 2 if self.desc.dtype == KVP_BF16 else 1

    def close(self) -> None:
        if self.handle:
            _L.kvp_pool_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- host pool ------------------------------------------------------------------
def kvp_pool_bytes(desc: PoolDesc):
    kv, meta = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_L.kvp_pool_bytes(ctypes.byref(desc), ctypes.byref(kv), ctypes.byref(meta)),
           "kvp_pool_bytes")
    return kv.value, meta.value


def kvp_pool_create(desc: PoolDesc) -> Pool:
    h = ctypes.c_void_p()
    _check(_L.kvp_pool_create(ctypes.byref(desc), ctypes.byref(h)), "kvp_pool_create")
    return Pool(h.value, desc)


def kvp_pool_destroy(pool: Pool) -> None:
    pool.close()


def kvp_pool_get_desc(pool: Pool) -> PoolDesc:
    d = PoolDesc()
    _check(_L.kvp_pool_get_desc(pool.handle, ctypes.byref(d)), "kvp_pool_get_desc")
    return d


def kvp_pool_free_count(pool: Pool) -> int:
    return int(_L.kvp_pool_free_count(pool.handle))


def kvp_pool_refcount(pool: Pool, page: int) -> int:
    return int(_L.kvp_pool_refcount(pool.handle, int(page)))


def _i32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.int32 or not a.flags.c_contiguous:
        raise ValueError("expected a C-contiguous int32 array")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_lib.P_int32)


def kvp_pages_alloc(pool: Pool, n: int) -> np.ndarray:
    out = np.empty(int(n), dtype=np.int32)
    _check(_L.kvp_pages_alloc(pool.handle, int(n), _ptr(out)), "kvp_pages_alloc")
    return out


def kvp_pages_ref(pool: Pool, ids) -> None:
    ids = _i32(np.ascontiguousarray(ids, dtype=np.int32))
    _check(_L.kvp_pages_ref(pool.handle, ids.size, _ptr(ids)), "kvp_pages_ref")


def kvp_pages_free(pool: Pool, ids) -> None:
    ids = _i32(np.ascontiguousarray(ids, dtype=np.int32))
    _check(_L.kvp_pages_free(pool.handle, ids.size, _ptr(ids)), "kvp_pages_free")


def kvp_seq_grow(pool: Pool, row: np.ndarray, cur_len: int, new_len: int) -> None:
    """Allocate pages so that ``row`` (int32 host array, edited in place) covers new_len."""
    row = _i32(row)
    _check(_L.kvp_seq_grow(pool.handle, _ptr(row), row.size, int(cur_len), int(new_len)),
           "kvp_seq_grow")


def kvp_seq_share(pool: Pool, src_row: np.ndarray, dst_row: np.ndarray, n_blocks: int) -> None:
    src_row, dst_row = _i32(src_row), _i32(dst_row)
    if n_blocks > min(src_row.size, dst_row.size):
        raise ValueError("n_blocks exceeds a row")
    _check(_L.kvp_seq_share(pool.handle, _ptr(src_row), _ptr(dst_row), int(n_blocks)),
           "kvp_seq_share")


def kvp_seq_release(pool: Pool, row: np.ndarray, n_blocks: int) -> None:
    row = _i32(row)
    if n_blocks > row.size:
        raise ValueError("n_blocks exceeds the row")
    _check(_L.kvp_seq_release(pool.handle, _ptr(row), int(n_blocks)), "kvp_seq_release")


def kvp_seq_evict_window(pool: Pool, row: np.ndarray, ctx_len: int, sink_tokens: int,
                         window_tokens: int) -> None:
    """Release the pages of ``row`` that hold only tokens outside sinks + window."""
    row = _i32(row)
    _check(_L.kvp_seq_evict_window(pool.handle, _ptr(row), row.size, int(ctx_len),
                                   int(sink_tokens), int(window_tokens)), "kvp_seq_evict_window")


class PrefixCache:
    """Owner of one host prefix cache (kvp_prefix_cache_create / _destroy)."""

    def __init__(self, pool: Pool):
        h = ctypes.c_void_p()
        _check(_L.kvp_prefix_cache_create(pool.handle, ctypes.byref(h)), "kvp_prefix_cache_create")
        self.handle = h
        self.pool = pool   # the pool must outlive the cache

    def close(self) -> None:
        if self.handle:
            _L.kvp_prefix_cache_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kvp_prefix_cache_create(pool: Pool) -> PrefixCache:
    return PrefixCache(pool)


def kvp_prefix_cache_pages(cache: PrefixCache) -> int:
    return int(_L.kvp_prefix_cache_pages(cache.handle))


def kvp_prefix_match(cache: PrefixCache, tokens, max_pages: int = None) -> np.ndarray:
    """Pages of the longest cached whole-block prefix of ``tokens`` (each with a
    reference added for the caller)."""
    tokens = _i32(np.ascontiguousarray(tokens, dtype=np.int32))
    P = cache.pool.desc.page_size
    cap = tokens.size // P if max_pages is None else int(max_pages)
    out = np.empty(max(cap, 1), dtype=np.int32)
    n = ctypes.c_int32()
    _check(_L.kvp_prefix_match(cache.handle, _ptr(tokens), tokens.size, _ptr(out), cap,
                               ctypes.byref(n)), "kvp_prefix_match")
    return out[:n.value].copy()


def kvp_prefix_insert(cache: PrefixCache, tokens, pages) -> None:
    tokens = _i32(np.ascontiguousarray(tokens, dtype=np.int32))
    pages = _i32(np.ascontiguousarray(pages, dtype=np.int32))
    if pages.size < tokens.size // cache.pool.desc.page_size:
        raise ValueError("one page per full block of tokens is needed")
    _check(_L.kvp_prefix_insert(cache.handle, _ptr(tokens), tokens.size, _ptr(pages)),
           "kvp_prefix_insert")


def kvp_prefix_evict(cache: PrefixCache, n_pages: int) -> int:
    n = ctypes.c_int32()
    _check(_L.kvp_prefix_evict(cache.handle, int(n_pages), ctypes.byref(n)), "kvp_prefix_evict")
    return int(n.value)


def kvp_seq_prepare_append(pool: Pool, row: np.ndarray, cur_len: int, new_len: int):
    """Private pages for appending cur_len..new_len-1; returns [(src, dst)] copies to run."""
    row = _i32(row)
    src = np.full(1, -1, dtype=np.int32)
    dst = np.full(1, -1, dtype=np.int32)
    n = ctypes.c_int32()
    _check(_L.kvp_seq_prepare_append(pool.handle, _ptr(row), row.size, int(cur_len),
                                     int(new_len), _ptr(src), _ptr(dst), ctypes.byref(n)),
           "kvp_seq_prepare_append")
    return [(int(src[0]), int(dst[0]))] if n.value else []


def kvp_copy_pages(pool: Pool, k_pool, v_pool, k_meta, v_meta, src_dst, stream=None) -> None:
    """Copy pages on the device; src_dst is an int32 device tensor [n, 2]."""
    eb = pool.elem_bytes
    n = int(src_dst.shape[0]) if src_dst.dim() == 2 else 0
    if src_dst.dim() != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be [n, 2]")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "kvp_copy_pages")
    _check(_L.kvp_copy_pages(pool.handle, _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
                             _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2),
                             _dev(src_dst, "src_dst", 4), n, _stream(stream)), "kvp_copy_pages")


def kvp_decode_plan(desc: PoolDesc, num_seqs: int, num_q_heads: int, max_context_len: int,
                    num_splits_req: int = 0, num_cus: int = 256) -> dict:
    p = DecodePlan()
    _check(_L.kvp_decode_plan(ctypes.byref(desc), int(num_seqs), int(num_q_heads),
                              int(max_context_len), int(num_splits_req), int(num_cus),
                              ctypes.byref(p)), "kvp_decode_plan")
    return {"num_splits": p.num_splits, "pages_per_split": p.pages_per_split,
            "waves_per_group": p.waves_per_group, "use_mfma": bool(p.use_mfma),
            "workspace_bytes": int(p.workspace_bytes)}


# ---- device entry points ------------------------------------------------------------
def _dev(t, name, elem_size=None):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    return 0 if t is None else int(t.numel()) * int(t.element_size())


def _check_pools(pool: Pool, k_pool, v_pool, k_meta, v_meta, where: str) -> None:
    """The K/V (and metadata) tensors hold at least one layer's pool bytes."""
    kv_bytes, meta_bytes = kvp_pool_bytes(pool.desc)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if t is None or _nbytes(t) < kv_bytes:
            raise ValueError(f"{where}: {name} must hold the pool's {kv_bytes} bytes")
    for name, t in (("k_meta", k_meta), ("v_meta", v_meta)):
        if meta_bytes and (t is None or _nbytes(t) < meta_bytes):
            raise ValueError(f"{where}: {name} must hold the pool's {meta_bytes} metadata bytes")
        if not meta_bytes and t is not None:
            raise ValueError(f"{where}: bfloat16 pools take no {name}")


def _check_queries(pool: Pool, q, out, where: str) -> None:
    """q and out are [rows, H_q, D] with the pool's head dim and whole groups."""
    D, Hkv = pool.desc.head_dim, pool.desc.num_kv_heads
    if q.dim() != 3 or int(q.shape[2]) != D:
        raise ValueError(f"{where}: q must be [rows, H_q, {D}]")
    if int(q.shape[1]) % Hkv:
        raise ValueError(f"{where}: H_q must be a multiple of the pool's {Hkv} KV heads")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"{where}: out must have q's shape")


def _check_batch(block_tables, context_lens, B: int, where: str) -> None:
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != B or context_lens.numel() != B:
        raise ValueError(f"{where}: block_tables [B, max_blocks] and context_lens [B] "
                         "must cover the batch")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def kvp_kv_append(pool: Pool, k_pool, v_pool, k_meta, v_meta, k_new, v_new, seq_idx, pos,
                  block_tables, stream=None) -> None:
    """Write k_new/v_new [N, H_kv, D] (bf16) into the slots the tables name."""
    eb = pool.elem_bytes
    n = int(seq_idx.numel())
    rows = (n, pool.desc.num_kv_heads, pool.desc.head_dim)
    if pos.numel() != n or tuple(k_new.shape) != rows or tuple(v_new.shape) != rows:
        raise ValueError(f"kvp_kv_append: seq_idx and pos [N], k_new and v_new {list(rows)}")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "kvp_kv_append")
    _check(_L.kvp_kv_append(pool.handle, _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
                            _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2),
                            _dev(k_new, "k_new", 2), _dev(v_new, "v_new", 2),
                            _dev(seq_idx, "seq_idx", 4), _dev(pos, "pos", 4), n,
                            _dev(block_tables, "block_tables", 4), int(block_tables.shape[0]),
                            int(block_tables.shape[1]), _stream(stream)), "kvp_kv_append")


def kvp_decode_workspace_bytes(pool: Pool, num_seqs: int, num_q_heads: int,
                               max_context_len: int, num_splits_req: int = 0) -> int:
    b = ctypes.c_size_t()
    _check(_L.kvp_decode_workspace_bytes(pool.handle, int(num_seqs), int(num_q_heads),
                                         int(max_context_len), int(num_splits_req),
                                         ctypes.byref(b)), "kvp_decode_workspace_bytes")
    return int(b.value)


def kvp_paged_attention_decode(pool: Pool, q, k_pool, v_pool, k_meta, v_meta, block_tables,
                               context_lens, max_context_len: int, scale: float, out,
                               num_splits_req: int = 0, workspace=None,
                               stream=None) -> None:
    """out[b, j] = softmax(scale * q[b, j] K_b^T) V_b over the sequence's pages."""
    eb = pool.elem_bytes
    _check_queries(pool, q, out, "decode")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check_batch(block_tables, context_lens, B, "decode")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "decode")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_L.kvp_paged_attention_decode(
        pool.handle, _dev(q, "q", 2), _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
        _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2), _dev(block_tables, "block_tables", 4),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", 4), B, Hq,
        int(max_context_len), float(scale), _dev(out, "out", 2), int(num_splits_req),
        _dev(workspace, "workspace"), ws_bytes, _stream(stream)), "kvp_paged_attention_decode")


def kvp_paged_attention_decode_noalloc(pool: Pool, q, k_pool, v_pool, k_meta, v_meta,
                                       block_tables, context_lens, max_context_len: int,
                                       scale: float, out, num_splits_req: int = 0,
                                       stream=None) -> None:
    """kvp_paged_attention_decode with the split partials in the library's
    fixed device buffer (no workspace argument, no device allocation)."""
    eb = pool.elem_bytes
    _check_queries(pool, q, out, "decode")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check_batch(block_tables, context_lens, B, "decode")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "decode")
    _check(_L.kvp_paged_attention_decode_noalloc(
        pool.handle, _dev(q, "q", 2), _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
        _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2), _dev(block_tables, "block_tables", 4),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", 4), B, Hq,
        int(max_context_len), float(scale), _dev(out, "out", 2), int(num_splits_req),
        _stream(stream)), "kvp_paged_attention_decode_noalloc")


def kvp_decode_window_workspace_bytes(pool: Pool, num_seqs: int, num_q_heads: int,
                                      max_context_len: int, sink_tokens: int, window_tokens: int,
                                      num_splits_req: int = 0) -> int:
    b = ctypes.c_size_t()
    _check(_L.kvp_decode_window_workspace_bytes(pool.handle, int(num_seqs), int(num_q_heads),
                                                int(max_context_len), int(sink_tokens),
                                                int(window_tokens), int(num_splits_req),
                                                ctypes.byref(b)),
           "kvp_decode_window_workspace_bytes")
    return int(b.value)


def kvp_paged_attention_decode_window(pool: Pool, q, k_pool, v_pool, k_meta, v_meta,
                                      block_tables, context_lens, max_context_len: int,
                                      scale: float, sink_tokens: int, window_tokens: int, out,
                                      num_splits_req: int = 0, workspace=None,
                                      stream=None) -> None:
    """Decode attending only to the first sink_tokens and the last window_tokens tokens."""
    eb = pool.elem_bytes
    _check_queries(pool, q, out, "decode")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check_batch(block_tables, context_lens, B, "decode")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "decode")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_L.kvp_paged_attention_decode_window(
        pool.handle, _dev(q, "q", 2), _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
        _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2), _dev(block_tables, "block_tables", 4),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", 4), B, Hq,
        int(max_context_len), float(scale), int(sink_tokens), int(window_tokens),
        _dev(out, "out", 2), int(num_splits_req), _dev(workspace, "workspace"), ws_bytes,
        _stream(stream)), "kvp_paged_attention_decode_window")


def kvp_decode_schedule_bounds(pool: Pool, num_seqs: int, num_q_heads: int,
                               max_bins: int) -> tuple:
    """(schedule bytes, workspace bytes) upper bounds for any lengths."""
    sb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_L.kvp_decode_schedule_bounds(pool.handle, int(num_seqs), int(num_q_heads),
                                         int(max_bins), ctypes.byref(sb), ctypes.byref(wb)),
           "kvp_decode_schedule_bounds")
    return int(sb.value), int(wb.value)


class Schedule:
    """A balanced decode schedule built on the host (kvp_decode_schedule):
    ``words`` is the int32 host array, ``info`` the ScheduleInfo."""

    def __init__(self, words: np.ndarray, info: ScheduleInfo):
        self.words = words
        self.info = info

    @property
    def used(self) -> np.ndarray:
        return self.words[: self.info.sched_words]


def kvp_decode_schedule(pool: Pool, context_lens, num_q_heads: int, max_blocks: int,
                        max_bins: int, sink_tokens: int = 0, window_tokens: int = 0) -> Schedule:
    """Balanced schedule for host context lengths (numpy int32 array); at most
    max_bins bins (kvp_decode_schedule_bins gives the count that fills the
    device)."""
    ctx = _i32(np.ascontiguousarray(context_lens, dtype=np.int32))
    sb, _ = kvp_decode_schedule_bounds(pool, ctx.size, num_q_heads, max_bins)
    words = np.zeros(sb // 4, dtype=np.int32)
    info = ScheduleInfo()
    _check(_L.kvp_decode_schedule(pool.handle, _ptr(ctx), ctx.size, int(num_q_heads),
                                  int(max_blocks), int(sink_tokens), int(window_tokens),
                                  int(max_bins), _ptr(words), words.nbytes, ctypes.byref(info)),
           "kvp_decode_schedule")
    return Schedule(words, info)


def kvp_decode_schedule_bins(pool: Pool, num_q_heads: int) -> int:
    """Bins that keep every compute unit of the current device busy along a
    schedule for this pool (four per compute unit, eight for quantized pools
    on the matrix-core path with up to 16 query heads per KV head)."""
    n = ctypes.c_int32()
    _check(_L.kvp_decode_schedule_bins(pool.handle, int(num_q_heads), ctypes.byref(n)),
           "kvp_decode_schedule_bins")
    return int(n.value)


def kvp_paged_attention_decode_scheduled(pool: Pool, q, k_pool, v_pool, k_meta, v_meta,
                                         block_tables, context_lens, max_context_len: int,
                                         scale: float, sched_dev, schedule: Schedule, out,
                                         workspace=None, stream=None) -> None:
    """Decode along a balanced schedule; sched_dev is the device copy (int32)
    of schedule.used."""
    eb = pool.elem_bytes
    _check_queries(pool, q, out, "decode")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check_batch(block_tables, context_lens, B, "decode")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "decode")
    if sched_dev.numel() < schedule.info.sched_words:
        raise ValueError("sched_dev must hold the schedule's used words")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_L.kvp_paged_attention_decode_scheduled(
        pool.handle, _dev(q, "q", 2), _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
        _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2), _dev(block_tables, "block_tables", 4),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", 4), B, Hq,
        int(max_context_len), float(scale), _dev(sched_dev, "sched", 4),
        ctypes.byref(schedule.info), _dev(out, "out", 2), _dev(workspace, "workspace"), ws_bytes,
        _stream(stream)), "kvp_paged_attention_decode_scheduled")


def kvp_paged_attention_prefill(pool: Pool, q, q_start, k_pool, v_pool, k_meta, v_meta,
                                block_tables, context_lens, max_q_len: int,
                                max_context_len: int, scale: float, out, stream=None) -> None:
    """Causal multi-query attention: q/out [N, H_q, D], rows q_start[b]..q_start[b+1]-1
    are sequence b's chunk (its last positions)."""
    eb = pool.elem_bytes
    B = int(context_lens.numel())
    if q_start.numel() != B + 1 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("q_start must have B+1 entries and block_tables B rows")
    _check_queries(pool, q, out, "prefill")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "prefill")
    _check(_L.kvp_paged_attention_prefill(
        pool.handle, _dev(q, "q", 2), _dev(q_start, "q_start", 4), _dev(k_pool, "k_pool", eb),
        _dev(v_pool, "v_pool", eb), _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2),
        _dev(block_tables, "block_tables", 4), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", 4), B, int(q.shape[1]), int(max_q_len),
        int(max_context_len), float(scale), _dev(out, "out", 2), _stream(stream)),
        "kvp_paged_attention_prefill")


def kvp_prefill_schedule_bound(pool: Pool, num_seqs: int, num_q_heads: int, max_blocks: int,
                               max_q_len: int, max_context_len: int) -> int:
    """Upper bound of a multi-query order's length for these arguments."""
    n = ctypes.c_int64()
    _check(_L.kvp_prefill_schedule_bound(pool.handle, int(num_seqs), int(num_q_heads),
                                         int(max_blocks), int(max_q_len), int(max_context_len),
                                         ctypes.byref(n)), "kvp_prefill_schedule_bound")
    return int(n.value)


def kvp_prefill_schedule(pool: Pool, q_start, context_lens, num_q_heads: int, max_blocks: int,
                         max_q_len: int, max_context_len: int) -> np.ndarray:
    """Longest-first workgroup order (int32 host array, -1 = padding) of the
    multi-query call for these host chunk offsets and lengths."""
    qs = _i32(np.ascontiguousarray(q_start, dtype=np.int32))
    ctx = _i32(np.ascontiguousarray(context_lens, dtype=np.int32))
    if qs.size != ctx.size + 1:
        raise ValueError("q_start must have B+1 entries")
    cap = kvp_prefill_schedule_bound(pool, ctx.size, num_q_heads, max_blocks, max_q_len,
                                     max_context_len)
    buf = np.zeros(max(cap, 1), dtype=np.int32)
    n = ctypes.c_int64()
    _check(_L.kvp_prefill_schedule(pool.handle, _ptr(qs), _ptr(ctx), ctx.size, int(num_q_heads),
                                   int(max_blocks), int(max_q_len), int(max_context_len),
                                   _ptr(buf), cap, ctypes.byref(n)), "kvp_prefill_schedule")
    return buf[: n.value].copy()


def kvp_paged_attention_prefill_scheduled(pool: Pool, q, q_start, k_pool, v_pool, k_meta, v_meta,
                                          block_tables, context_lens, max_q_len: int,
                                          max_context_len: int, scale: float, sched_dev, out,
                                          stream=None) -> None:
    """kvp_paged_attention_prefill with its workgroups in the order sched_dev
    (device int32 copy of kvp_prefill_schedule's result)."""
    eb = pool.elem_bytes
    B = int(context_lens.numel())
    if q_start.numel() != B + 1 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("q_start must have B+1 entries and block_tables B rows")
    _check_queries(pool, q, out, "prefill")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "prefill")
    _check(_L.kvp_paged_attention_prefill_scheduled(
        pool.handle, _dev(q, "q", 2), _dev(q_start, "q_start", 4), _dev(k_pool, "k_pool", eb),
        _dev(v_pool, "v_pool", eb), _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2),
        _dev(block_tables, "block_tables", 4), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", 4), B, int(q.shape[1]), int(max_q_len),
        int(max_context_len), float(scale), _dev(sched_dev, "sched", 4), int(sched_dev.numel()),
        _dev(out, "out", 2), _stream(stream)), "kvp_paged_attention_prefill_scheduled")


def kvp_decode_partials_bytes(pool: Pool, num_seqs: int, num_q_heads: int,
                              max_context_len: int, num_splits_req: int = 0):
    """(num_splits, bytes) of the partials buffer the split kernel writes."""
    b = ctypes.c_size_t()
    s = ctypes.c_int32()
    _check(_L.kvp_decode_partials_bytes(pool.handle, int(num_seqs), int(num_q_heads),
                                        int(max_context_len), int(num_splits_req),
                                        ctypes.byref(s), ctypes.byref(b)),
           "kvp_decode_partials_bytes")
    return int(s.value), int(b.value)


def kvp_paged_attention_decode_partials(pool: Pool, q, k_pool, v_pool, k_meta, v_meta,
                                        block_tables, context_lens, max_context_len: int,
                                        scale: float, partials, num_splits_req: int = 0,
                                        stream=None) -> int:
    """Split kernel only: per-split (o, m, l) partials into ``partials``; returns S."""
    eb = pool.elem_bytes
    if q.dim() != 3 or int(q.shape[2]) != pool.desc.head_dim:
        raise ValueError(f"decode partials: q must be [B, H_q, {pool.desc.head_dim}]")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check_batch(block_tables, context_lens, B, "decode partials")
    _check_pools(pool, k_pool, v_pool, k_meta, v_meta, "decode partials")
    nbytes = partials.numel() * partials.element_size()
    s = ctypes.c_int32()
    _check(_L.kvp_paged_attention_decode_partials(
        pool.handle, _dev(q, "q", 2), _dev(k_pool, "k_pool", eb), _dev(v_pool, "v_pool", eb),
        _dev(k_meta, "k_meta", 2), _dev(v_meta, "v_meta", 2), _dev(block_tables, "block_tables", 4),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", 4), B, Hq,
        int(max_context_len), float(scale), int(num_splits_req), _dev(partials, "partials"),
        nbytes, ctypes.byref(s), _stream(stream)), "kvp_paged_attention_decode_partials")
    return int(s.value)


def kvp_lse_merge(partials, rows: int, num_splits: int, head_dim: int, out, stream=None) -> None:
    """Merge per-split partials by log-sum-exp into ``out`` ([rows, D] bfloat16 bits)."""
    if out.numel() != int(rows) * int(head_dim):
        raise ValueError("out must hold rows * head_dim elements")
    parts = int(rows) * int(num_splits)
    need = (parts * int(head_dim) * 4 + 255) // 256 * 256 + parts * 2 * 4
    if parts > 0 and _nbytes(partials) < need:
        raise ValueError(f"partials must hold {need} bytes for {rows} rows x {num_splits} splits")
    _check(_L.kvp_lse_merge(_dev(partials, "partials"), int(rows), int(num_splits),
                            int(head_dim), _dev(out, "out", 2), _stream(stream)),
           "kvp_lse_merge")


def kvp_probe_read_chunks(pool_a, pool_b, chunk_ids, chunk_bytes: int, num_waves: int, sink,
                          chunks_in_flight: int = 2, stream=None) -> None:
    """Read chunk chunk_ids[i] of both device buffers for every i (the decode
    kernels' page-streaming pattern with no arithmetic); sink receives
    num_waves * 64 words."""
    pool_bytes = min(_nbytes(pool_a), _nbytes(pool_b))
    if _nbytes(sink) < int(num_waves) * 64 * 4:
        raise ValueError("sink must hold num_waves * 64 uint32 words")
    _check(_L.kvp_probe_read_chunks(_dev(pool_a, "pool_a"), _dev(pool_b, "pool_b"), pool_bytes,
                                    _dev(chunk_ids, "chunk_ids", 4), int(chunk_ids.numel()),
                                    int(chunk_bytes), int(chunks_in_flight), int(num_waves),
                                    _dev(sink, "sink", 4),
                                    _stream(stream)), "kvp_probe_read_chunks")


__all__ = [
    "KVP_OK", "KVP_E_INVAL", "KVP_E_NOPAGES", "KVP_E_UNSUPPORTED", "KVP_E_HIP", "KVP_E_SCRATCH",
    "KVP_BF16",
    "KVP_INT8", "KVP_INT4", "KVP_FP8", "KvpError", "Pool", "PoolDesc", "make_desc", "kvp_status_string",
    "kvp_pool_bytes", "kvp_pool_create", "kvp_pool_destroy", "kvp_pool_get_desc",
    "kvp_pool_free_count", "kvp_pool_refcount", "kvp_pages_alloc", "kvp_pages_ref",
    "kvp_pages_free", "kvp_seq_grow", "kvp_seq_share", "kvp_seq_release", "kvp_decode_plan",
    "kvp_kv_append", "kvp_decode_workspace_bytes", "kvp_paged_attention_decode",
    "kvp_paged_attention_decode_noalloc",
    "kvp_decode_partials_bytes", "kvp_paged_attention_decode_partials", "kvp_lse_merge",
    "kvp_decode_schedule_bounds", "kvp_decode_schedule", "kvp_decode_schedule_bins",
    "kvp_paged_attention_decode_scheduled",
    "Schedule", "ScheduleInfo",
    "kvp_seq_evict_window", "kvp_decode_window_workspace_bytes",
    "kvp_paged_attention_decode_window", "kvp_paged_attention_prefill",
    "kvp_prefill_schedule_bound", "kvp_prefill_schedule", "kvp_paged_attention_prefill_scheduled",
    "PrefixCache",
    "kvp_prefix_cache_create", "kvp_prefix_cache_pages", "kvp_prefix_match",
    "kvp_prefix_insert", "kvp_prefix_evict", "kvp_seq_prepare_append", "kvp_copy_pages",
    "kvp_probe_read_chunks",
]
