"""Paged decode attention -- plain float64 CPU oracle (test infrastructure only).

What it computes ("KV-Cache Optimization Techniques", section "PagedAttention",
eq. 1): for the new query token q_t of a sequence, gather the sequence's K and
V pages in logical order through its page table, concatenate them, and take
softmax(q_t K^T / sqrt(d_k)) V.  Paging moves where the rows live, not the
result ("Understanding KV-Cache Optimization in Modern LLM Serving", section
"PagedAttention Solution": the block table maps logical blocks to scattered
physical blocks without changing model output), so this is the definition of
attention applied to the gathered rows.

Several new tokens per sequence ("KV-Cache Optimization Techniques", section
"Cache-Aware Scheduling": chunked prefill processes a prompt in chunks against
the cache): a sequence holding n tokens whose last q_len are the chunk's own
(already written to its pages) has query row i at position n - q_len + i, and
that row attends to positions 0 .. n - q_len + i (causal; eq. 1 over those
rows).

Sinks and a recent window ("KV-Cache Optimization Techniques", section "Token
Eviction Strategies", eq. 5, StreamingLLM: the cache keeps tokens 1..s and
t-w+1..t; section "Sliding Window Cache", eq. 6, the window alone): the query
of a sequence of n tokens attends to positions 0..s-1 and n-w..n-1 (0-based),
or to all n when s + w >= n.

Readings taken where the pages leave a step open:
* the scale is an explicit float32 argument (1/sqrt(D) in every workload);
* query head j uses KV head j // g with g = H_q / H_kv ("Multi-Query and
  Grouped-Query Caching", eq. 7, gives only the group count);
* a sequence of length 0 attends to nothing and yields 0;
* rows past a sequence's length in its last page are never read.

The pool layout is the library header's contract, written out here from its
text: K[page][h][t][d], V stored transposed per (page, head) as [d][t],
float16 (scale, zero) pairs per token per head for INT8 pools.  INT4 pools
hold two channels per byte (even channel in the low nibble, code + 8):
K bytes [page][h][t][d/2], V bytes [page][h][d/2][t].  FP8 pools hold one
e4m3 code per byte in the INT8 layout, with (scale, 0) metadata.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .quantize import (bf16_bits_to_f32, dequantize, dequantize_fp8, quantize_rows,
                       quantize_rows_fp8, quantize_rows_int4)


@dataclass(frozen=True)
class PoolLayout:
    num_pages: int
    page_size: int      # P
    num_kv_heads: int   # H_kv
    head_dim: int       # D
    dtype: str = "bf16"  # "bf16" | "int8" | "int4" | "fp8"

    @property
    def elems(self) -> int:
        """Elements of one K (or V) array."""
        return self.num_pages * self.num_kv_heads * self.page_size * self.head_dim

    @property
    def quantized(self) -> bool:
        return self.dtype != "bf16"

    @property
    def meta_elems(self) -> int:
        """float16 elements of one INT8 metadata array."""
        return self.num_pages * self.num_kv_heads * self.page_size * 2

    def empty_pools(self, k_fill: int, meta_fill: int):
        """Host pools filled with a poison pattern: (k, v, k_meta, v_meta)."""
        if self.dtype == "bf16":
            k = np.full(self.elems, k_fill, dtype=np.uint16)
            v = np.full(self.elems, k_fill, dtype=np.uint16)
            return k, v, None, None
        if self.dtype in ("int4", "fp8"):
            nbytes = self.elems // 2 if self.dtype == "int4" else self.elems
            k = np.full(nbytes, k_fill, dtype=np.uint8)
            v = np.full(nbytes, k_fill, dtype=np.uint8)
            km = np.full(self.meta_elems, meta_fill, dtype=np.uint16)
            vm = np.full(self.meta_elems, meta_fill, dtype=np.uint16)
            return k, v, km, vm
        k = np.full(self.elems, k_fill, dtype=np.uint8).view(np.int8)
        v = np.full(self.elems, k_fill, dtype=np.uint8).view(np.int8)
        km = np.full(self.meta_elems, meta_fill, dtype=np.uint16)
        vm = np.full(self.meta_elems, meta_fill, dtype=np.uint16)
        return k, v, km, vm


def slot(block_table_row: np.ndarray, pos: int, page_size: int):
    """Physical (page, in-page row) of token position ``pos``: the page table
    entry of logical block pos // P, row pos % P ("PagedAttention": each
    request's page table maps logical KV positions to physical pages)."""
    return int(block_table_row[pos // page_size]), pos % page_size


def _to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def gather_sequence(layout: PoolLayout, k_pool, v_pool, k_meta, v_meta,
                    block_table_row: np.ndarray, ctx: int):
    """K and V of one sequence in logical order: float64 [H_kv, ctx, D] each."""
    P, H, D = layout.page_size, layout.num_kv_heads, layout.head_dim
    if ctx == 0:
        z = np.zeros((H, 0, D))
        return z, z.copy()
    nb = -(-ctx // P)
    pages = np.asarray(block_table_row[:nb], dtype=np.int64)
    if (pages < 0).any() or (pages >= layout.num_pages).any():
        raise ValueError("block table names a page outside the pool")
    if layout.dtype in ("int4", "fp8"):
        return gather_positions(layout, k_pool, v_pool, k_meta, v_meta, block_table_row,
                                np.arange(ctx))
    kp = np.asarray(k_pool).reshape(layout.num_pages, H, P, D)[pages]      # [nb,H,P,D]
    vp = np.asarray(v_pool).reshape(layout.num_pages, H, D, P)[pages]      # [nb,H,D,P]
    if layout.dtype == "bf16":
        K = _to_f64(kp)
        V = _to_f64(vp)
    else:
        km = np.asarray(k_meta).reshape(layout.num_pages, H, P, 2)[pages]  # [nb,H,P,2]
        vm = np.asarray(v_meta).reshape(layout.num_pages, H, P, 2)[pages]
        K = dequantize(kp, km[..., 0], km[..., 1])                          # [nb,H,P,D]
        # V tile is [D][P]; move the token axis next to the head axis first.
        V = dequantize(np.swapaxes(vp, -1, -2), vm[..., 0], vm[..., 1])    # [nb,H,P,D]
        vp = None
    K = K.transpose(1, 0, 2, 3).reshape(H, nb * P, D)[:, :ctx]
    if layout.dtype == "bf16":
        V = V.transpose(1, 0, 3, 2).reshape(H, nb * P, D)[:, :ctx]
    else:
        V = V.transpose(1, 0, 2, 3).reshape(H, nb * P, D)[:, :ctx]
    return K, V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V per query head, float64.

    q: [H_q, D]; K, V: [H_kv, n, D]; query head j reads KV head j // (H_q/H_kv).
    """
    Hq, D = q.shape
    Hkv, n, _ = K.shape
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    g = Hq // Hkv
    out = np.zeros((Hq, D))
    if n == 0:
        return out
    for j in range(Hq):
        h = j // g
        s = (K[h] @ q[j]) * scale
        p = np.exp(s - s.max())
        out[j] = (p @ V[h]) / p.sum()
    return out


def _unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """Bytes holding channel pairs (even channel low, code + 8) -> codes [..., 2n]."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = (b & 0xF).astype(np.int64) - 8
    out[..., 1::2] = (b >> 4).astype(np.int64) - 8
    return out


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Codes in -8..7 [..., 2n] -> bytes [..., n] (even channel in the low nibble)."""
    c = (np.asarray(codes, dtype=np.int64) + 8).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def kept_positions(n: int, sink: int, window: int) -> np.ndarray:
    """Positions a sequence of n tokens attends to with s sink tokens and a
    recent window of w tokens (eq. 5; eq. 6 when s = 0).  w = 0: no window."""
    if window <= 0 or sink + window >= n:
        return np.arange(n)
    return np.concatenate([np.arange(sink), np.arange(n - window, n)])


def gather_positions(layout: PoolLayout, k_pool, v_pool, k_meta, v_meta,
                     block_table_row: np.ndarray, positions: np.ndarray):
    """K and V rows of the listed token positions, in that order: float64
    [H_kv, len, D] each.  Only the pages holding those positions are read."""
    P, H, D = layout.page_size, layout.num_kv_heads, layout.head_dim
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size == 0:
        z = np.zeros((H, 0, D))
        return z, z.copy()
    pages = np.asarray(block_table_row, dtype=np.int64)[positions // P]
    rows = positions % P
    if (pages < 0).any() or (pages >= layout.num_pages).any():
        raise ValueError("a kept position lies in a page outside the pool")
    hh = np.arange(H)[None, :]
    if layout.dtype in ("int4", "fp8"):
        km = np.asarray(k_meta).reshape(layout.num_pages, H, P, 2)[pages[:, None], hh,
                                                                   rows[:, None]]  # [len, H, 2]
        vm = np.asarray(v_meta).reshape(layout.num_pages, H, P, 2)[pages[:, None], hh,
                                                                   rows[:, None]]
        if layout.dtype == "fp8":
            kb = np.asarray(k_pool).reshape(layout.num_pages, H, P, D)[pages[:, None], hh,
                                                                       rows[:, None], :]
            vb = np.asarray(v_pool).reshape(layout.num_pages, H, D, P)[pages[:, None], hh, :,
                                                                       rows[:, None]]
            K = dequantize_fp8(kb, km[..., 0])
            V = dequantize_fp8(vb, vm[..., 0])
        else:
            kb = np.asarray(k_pool).reshape(layout.num_pages, H, P, D // 2)[pages[:, None], hh,
                                                                            rows[:, None], :]
            vb = np.asarray(v_pool).reshape(layout.num_pages, H, D // 2, P)[pages[:, None], hh,
                                                                            :, rows[:, None]]
            K = dequantize(_unpack_nibbles(kb), km[..., 0], km[..., 1])
            V = dequantize(_unpack_nibbles(vb), vm[..., 0], vm[..., 1])
        return K.transpose(1, 0, 2), V.transpose(1, 0, 2)
    kp = np.asarray(k_pool).reshape(layout.num_pages, H, P, D)
    vp = np.asarray(v_pool).reshape(layout.num_pages, H, D, P)
    kr = kp[pages[:, None], hh, rows[:, None], :]    # [len, H, D]
    vr = vp[pages[:, None], hh, :, rows[:, None]]    # [len, H, D] (V tile is [D][P])
    if layout.dtype == "bf16":
        K, V = _to_f64(kr), _to_f64(vr)
    else:
        km = np.asarray(k_meta).reshape(layout.num_pages, H, P, 2)[pages[:, None], hh,
                                                                   rows[:, None]]  # [len, H, 2]
        vm = np.asarray(v_meta).reshape(layout.num_pages, H, P, 2)[pages[:, None], hh,
                                                                   rows[:, None]]
        K = dequantize(kr, km[..., 0], km[..., 1])
        V = dequantize(vr, vm[..., 0], vm[..., 1])
    return K.transpose(1, 0, 2), V.transpose(1, 0, 2)


def paged_decode_window(layout: PoolLayout, q_bits: np.ndarray, k_pool, v_pool, k_meta, v_meta,
                        block_tables: np.ndarray, context_lens: np.ndarray, scale, sink: int,
                        window: int, seqs=None) -> np.ndarray:
    """Eq. 1 over the kept positions of eq. 5 / eq. 6: float64 [B, H_q, D]."""
    q = _to_f64(q_bits)
    B = q.shape[0]
    sel = range(B) if seqs is None else seqs
    out = np.zeros(q.shape)
    sc = float(np.float32(scale))
    for b in sel:
        pos = kept_positions(int(context_lens[b]), sink, window)
        K, V = gather_positions(layout, k_pool, v_pool, k_meta, v_meta, block_tables[b], pos)
        out[b] = attend(q[b], K, V, sc)
    return out


def paged_prefill(layout: PoolLayout, q_bits: np.ndarray, q_start: np.ndarray, k_pool, v_pool,
                  k_meta, v_meta, block_tables: np.ndarray, context_lens: np.ndarray, scale,
                  seqs=None) -> np.ndarray:
    """Causal multi-query attention over pages: float64 [N, H_q, D].

    q_bits: bfloat16 bits [N, H_q, D]; rows q_start[b] .. q_start[b+1]-1 are
    sequence b's chunk, in position order.  A row whose position would be
    negative (chunk longer than the sequence) attends to nothing and gives 0."""
    q = _to_f64(q_bits)
    out = np.zeros(q.shape)
    B = len(q_start) - 1
    sc = float(np.float32(scale))
    sel = range(B) if seqs is None else seqs
    for b in sel:
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = int(context_lens[b])
        K, V = gather_sequence(layout, k_pool, v_pool, k_meta, v_meta, block_tables[b], n)
        for i in range(r1 - r0):
            pos = n - (r1 - r0) + i
            if pos < 0:
                continue
            out[r0 + i] = attend(q[r0 + i], K[:, :pos + 1], V[:, :pos + 1], sc)
    return out


def paged_decode(layout: PoolLayout, q_bits: np.ndarray, k_pool, v_pool, k_meta, v_meta,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale,
                 seqs=None) -> np.ndarray:
    """Eq. 1 for every sequence (or the listed ``seqs``): float64 [B, H_q, D]."""
    q = _to_f64(q_bits)
    B = q.shape[0]
    sel = range(B) if seqs is None else seqs
    out = np.zeros(q.shape)
    sc = float(np.float32(scale))
    for b in sel:
        K, V = gather_sequence(layout, k_pool, v_pool, k_meta, v_meta,
                               block_tables[b], int(context_lens[b]))
        out[b] = attend(q[b], K, V, sc)
    return out


def append(layout: PoolLayout, k_pool, v_pool, k_meta, v_meta, k_rows, v_rows,
           seq_idx, pos, block_tables) -> None:
    """Write new K/V rows into their pages in place ("PagedAttention": pages
    hold the sequence's rows at the positions the page table gives).

    k_rows, v_rows: bfloat16 bits [N, H_kv, D]; seq_idx, pos: [N].
    INT8 pools store each (token, head) row quantized (``quantize_rows``);
    INT4 and FP8 pools with ``quantize_rows_int4`` / ``quantize_rows_fp8``.
    Rows are written in order, so a later row wins a shared slot.
    """
    P, H, D = layout.page_size, layout.num_kv_heads, layout.head_dim
    seq_idx = np.asarray(seq_idx, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    pages = np.asarray(block_tables, dtype=np.int64)[seq_idx, pos // P]
    if (pages < 0).any() or (pages >= layout.num_pages).any():
        raise ValueError("append names a page outside the pool")
    t = pos % P
    hh = np.arange(H)
    if layout.dtype in ("bf16", "int8"):
        kp = np.asarray(k_pool).reshape(layout.num_pages, H, P, D)
        vp = np.asarray(v_pool).reshape(layout.num_pages, H, D, P)
    if layout.dtype == "bf16":
        kp[pages[:, None], hh[None, :], t[:, None], :] = k_rows
        vp[pages[:, None], hh[None, :], :, t[:, None]] = v_rows
        return
    km = np.asarray(k_meta).reshape(layout.num_pages, H, P, 2)
    vm = np.asarray(v_meta).reshape(layout.num_pages, H, P, 2)
    if layout.dtype in ("int4", "fp8"):
        kb = np.asarray(k_pool).reshape(layout.num_pages, H, P, -1)          # [.., t, bytes]
        vb = np.asarray(v_pool).reshape(layout.num_pages, H, -1, P)          # [.., bytes, t]
        quant = quantize_rows_int4 if layout.dtype == "int4" else quantize_rows_fp8
        for rows, pool, meta, transposed in ((k_rows, kb, km, False), (v_rows, vb, vm, True)):
            codes, s16, z16 = quant(rows)
            stored = _pack_nibbles(codes) if layout.dtype == "int4" else codes
            if transposed:
                pool[pages[:, None], hh[None, :], :, t[:, None]] = stored
            else:
                pool[pages[:, None], hh[None, :], t[:, None], :] = stored
            meta[pages[:, None], hh[None, :], t[:, None], 0] = s16
            meta[pages[:, None], hh[None, :], t[:, None], 1] = z16
        return
    for rows, pool, meta, transposed in ((k_rows, kp, km, False), (v_rows, vp, vm, True)):
        codes, s16, z16 = quantize_rows(rows)
        if transposed:
            pool[pages[:, None], hh[None, :], :, t[:, None]] = codes
        else:
            pool[pages[:, None], hh[None, :], t[:, None], :] = codes
        meta[pages[:, None], hh[None, :], t[:, None], 0] = s16
        meta[pages[:, None], hh[None, :], t[:, None], 1] = z16
