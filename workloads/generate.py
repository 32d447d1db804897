"""Seeded synthetic inputs for paged decode attention.

Both the GPU path and the CPU oracle take their inputs from here.  This module
draws random numbers and rounds them to the storage type; it holds none of the
method's arithmetic (no slot indexing, no attention, no quantization).

Recipe (host configs), one ``numpy.random.Generator(PCG64(seed))`` per case,
draws taken in this order:

1. ``ctx``: explicit, or ``integers(ctx_lo, ctx_hi, endpoint=True)`` per sequence;
2. ``perm = permutation(num_pages)``: physical page ids, consumed in order by
   the shared prefix (if any) and then by each sequence's own blocks;
3. outlier channel sets for K and then V: ``choice(H_kv*D, n, replace=False)``;
4. ``q``: standard normal ``[B, H_q, D]`` times ``q_gain``;
5. history K rows then history V rows: standard normal ``[T, H_kv, D]``, drawn
   in chunks of 65,536 rows in order, outlier channels times ``outlier_gain``;
6. the new token's K then V rows: standard normal ``[B, H_kv, D]`` (outliers too).
   V rows (history and new) are multiplied by ``v_gain`` before the outliers.

Every float32 draw is rounded to bfloat16 (round to nearest even) and kept as
its raw 16-bit pattern.  The config with ``device_data`` draws q and K/V on the
GPU with ``torch.Generator`` seeded ``seed*100 + layer``, in the order q,
history K, history V, new K, new V, as float32 rounded to bfloat16; its block
table still comes from the numpy generator (one table for all layers).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import DecodeConfig

# Poison patterns for storage the decode must never read: free pages, the
# unused tail of a sequence's last page.
POISON_BF16 = 0x7FC0   # bfloat16 quiet NaN
POISON_F16 = 0x7E00    # float16 quiet NaN
POISON_I8 = 0x7F       # int8 code 127 (codes have no NaN; the metadata carries it)

_CHUNK = 65536


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class DecodeCase:
    cfg: DecodeConfig
    ctx: np.ndarray            # int32 [B] tokens attended (new token included)
    num_pages: int
    max_blocks: int
    block_tables: np.ndarray   # int32 [B, max_blocks], -1 where unused
    scale: np.float32
    q: Optional[np.ndarray] = None        # uint16 [N, H_q, D] (one row per new token)
    hist_k: Optional[np.ndarray] = None   # uint16 [T, H_kv, D]
    hist_v: Optional[np.ndarray] = None
    hist_seq: Optional[np.ndarray] = None  # int32 [T]
    hist_pos: Optional[np.ndarray] = None  # int32 [T]
    new_k: Optional[np.ndarray] = None    # uint16 [N, H_kv, D] (N = sum of chunk lengths)
    new_v: Optional[np.ndarray] = None
    new_pos: Optional[np.ndarray] = None  # int32 [N]: the chunk's positions (ctx - q_len ..)
    new_seq: Optional[np.ndarray] = None  # int32 [N]: sequence of each new row
    q_start: Optional[np.ndarray] = None  # int32 [B+1]: rows q_start[b].. of q / new_* are b's

    @property
    def B(self) -> int:
        return int(self.ctx.shape[0])


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _context_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.ctx_fixed is not None:
        ctx = np.asarray(cfg.ctx_fixed, dtype=np.int64)
        assert ctx.shape[0] == cfg.batch
    else:
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi, size=cfg.batch, endpoint=True)
    return ctx.astype(np.int32)


def _history_ranges(cfg: DecodeConfig, ctx: np.ndarray):
    """First cached position each sequence owns (rows before it are the shared prefix)."""
    starts = np.zeros(cfg.batch, dtype=np.int64)
    if cfg.shared_prefix:
        assert cfg.shared_prefix % cfg.page_size == 0, "shared prefix must be page aligned"
        assert (ctx - 1 >= cfg.shared_prefix).all(), "new token must lie past the prefix"
        starts[1:] = cfg.shared_prefix
    return starts


def held_positions(cfg: DecodeConfig, n: int) -> np.ndarray:
    """Positions the workload's cache holds for a sequence of n tokens: all of
    them, or (window configs) those below sink_tokens and the last
    window_tokens."""
    if cfg.window_tokens <= 0 or cfg.sink_tokens + cfg.window_tokens >= n:
        return np.arange(n)
    return np.concatenate([np.arange(cfg.sink_tokens), np.arange(n - cfg.window_tokens, n)])


def _tables(cfg: DecodeConfig, ctx: np.ndarray, rng: np.random.Generator):
    P = cfg.page_size
    n_prefix = cfg.shared_prefix // P
    # blocks each sequence holds pages for (beyond the shared prefix)
    own_blocks = [np.unique(held_positions(cfg, int(n)) // P) for n in ctx]
    own_blocks = [blk[blk >= n_prefix] for blk in own_blocks]
    used = n_prefix + sum(len(o) for o in own_blocks)
    num_pages = cfg.pool_pages if cfg.pool_pages is not None else \
        int(np.ceil((1.0 + cfg.pool_slack) * used))
    assert num_pages >= used
    perm = rng.permutation(num_pages).astype(np.int32)
    max_blocks = max(_ceil_div(int(n), P) for n in ctx)
    bt = np.full((cfg.batch, max_blocks), -1, dtype=np.int32)
    cursor = n_prefix
    for b in range(cfg.batch):
        bt[b, :n_prefix] = perm[:n_prefix]
        k = len(own_blocks[b])
        bt[b, own_blocks[b]] = perm[cursor:cursor + k]
        cursor += k
    return num_pages, max_blocks, bt


def _normal_bf16(rng: np.random.Generator, shape, gain: float = 1.0,
                 outliers: Optional[np.ndarray] = None, gain_out: float = 1.0) -> np.ndarray:
    """Standard normal float32 draws -> bf16 bits, rows drawn in order in chunks."""
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    inner = int(np.prod(shape[1:]))
    flat = out.reshape(rows, inner)
    for r0 in range(0, rows, _CHUNK):
        r1 = min(rows, r0 + _CHUNK)
        x = rng.standard_normal((r1 - r0, inner), dtype=np.float32)
        if gain != 1.0:
            x *= np.float32(gain)
        if outliers is not None and len(outliers):
            x[:, outliers] *= np.float32(gain_out)
        flat[r0:r1] = f32_to_bf16_bits(x)
    return out


def make_case(cfg: DecodeConfig, with_data: bool = True) -> DecodeCase:
    """Build one host decode case of ``cfg`` (one layer's worth of K/V)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    ctx = _context_lengths(cfg, rng)
    if cfg.q_len_hi > cfg.q_len:
        qlens = rng.integers(cfg.q_len, cfg.q_len_hi, size=cfg.batch, endpoint=True)
    else:
        qlens = np.full(cfg.batch, cfg.q_len)
    qlens = np.minimum(qlens, np.maximum(ctx, 1)).astype(np.int64)
    num_pages, max_blocks, bt = _tables(cfg, ctx, rng)
    scale = np.float32(1.0 / np.sqrt(np.float64(cfg.head_dim)))
    case = DecodeCase(cfg=cfg, ctx=ctx, num_pages=num_pages, max_blocks=max_blocks,
                      block_tables=bt, scale=scale)
    case.q_start = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    case.new_seq = np.repeat(np.arange(cfg.batch, dtype=np.int32), qlens)
    case.new_pos = np.concatenate([np.arange(int(ctx[b]) - int(qlens[b]), int(ctx[b]))
                                   for b in range(cfg.batch)]).astype(np.int32)
    if not with_data or cfg.device_data:
        return case
    Hkv, D, Hq, B = cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads, cfg.batch
    out_k = out_v = None
    if cfg.outlier_channels:
        out_k = np.sort(rng.choice(Hkv * D, cfg.outlier_channels, replace=False))
        out_v = np.sort(rng.choice(Hkv * D, cfg.outlier_channels, replace=False))
    N = int(case.q_start[-1])
    case.q = _normal_bf16(rng, (N, Hq, D), gain=cfg.q_gain)
    starts = _history_ranges(cfg, ctx)
    seqs, poss = [], []
    for b in range(B):
        p = held_positions(cfg, int(ctx[b])).astype(np.int32)
        p = p[(p >= starts[b]) & (p < ctx[b] - qlens[b])]
        poss.append(p)
        seqs.append(np.full(p.shape, b, dtype=np.int32))
    case.hist_seq = np.concatenate(seqs) if seqs else np.zeros(0, np.int32)
    case.hist_pos = np.concatenate(poss) if poss else np.zeros(0, np.int32)
    T = int(case.hist_pos.shape[0])
    case.hist_k = _normal_bf16(rng, (T, Hkv, D), outliers=out_k, gain_out=cfg.outlier_gain)
    case.hist_v = _normal_bf16(rng, (T, Hkv, D), gain=cfg.v_gain, outliers=out_v,
                               gain_out=cfg.outlier_gain)
    case.new_k = _normal_bf16(rng, (N, Hkv, D), outliers=out_k, gain_out=cfg.outlier_gain)
    case.new_v = _normal_bf16(rng, (N, Hkv, D), gain=cfg.v_gain, outliers=out_v,
                              gain_out=cfg.outlier_gain)
    return case


def history_rows_device(cfg: DecodeConfig, case: DecodeCase, layer: int, device):
    """Device draws for one layer of a ``device_data`` config (torch tensors, bf16).

    Returns (q, hist_k, hist_v, hist_seq, hist_pos, new_k, new_v, new_pos)."""
    import torch
    assert cfg.q_len == 1 and cfg.q_len_hi <= 1, "device draws cover one new token per sequence"
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 100 + layer)
    Hkv, D, Hq, B = cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads, cfg.batch

    def draw(shape):
        return torch.randn(shape, generator=g, device=device,
                           dtype=torch.float32).to(torch.bfloat16)

    starts = _history_ranges(cfg, case.ctx)
    counts = (case.ctx.astype(np.int64) - 1 - starts)
    hist_seq = np.repeat(np.arange(B, dtype=np.int32), counts)
    hist_pos = np.concatenate([np.arange(starts[b], case.ctx[b] - 1, dtype=np.int32)
                               for b in range(B)])
    T = int(hist_pos.shape[0])
    q = draw((B, Hq, D))
    hk = draw((T, Hkv, D))
    hv = draw((T, Hkv, D))
    nk = draw((B, Hkv, D))
    nv = draw((B, Hkv, D))
    t_seq = torch.from_numpy(hist_seq).to(device)
    t_pos = torch.from_numpy(hist_pos).to(device)
    new_pos = torch.from_numpy((case.ctx - 1).astype(np.int32)).to(device)
    return q, hk, hv, t_seq, t_pos, nk, nv, new_pos
