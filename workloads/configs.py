"""Synthetic workload shapes for paged decode attention.

Each config describes one decode step: every sequence appends one new token
(its K/V row is written into the page the block table names) and then its
single query token attends over all ``ctx`` tokens of that sequence, the new
one included.  ``ctx`` therefore counts the tokens attended in the step; the
cache holds ``ctx - 1`` of them before the step starts.

The shapes follow the worked examples and models named on the pages
("Understanding KV-Cache Optimization in Modern LLM Serving", section
"Concrete Example: Llama-3-70B": L=80, H_kv=8, D=128, 8,192 tokens, 32
requests; "KV-Cache Optimization Techniques", sections "PagedAttention",
"Prefix Caching", "KV-Cache Quantization", "Multi-Query and Grouped-Query
Caching").  This module holds shapes only; it computes nothing of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

BASE_SEED = 465


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str = "bf16"          # "bf16", "int8", "int4" or "fp8"
    ctx_fixed: Optional[Tuple[int, ...]] = None   # explicit per-sequence ctx
    ctx_lo: int = 0                 # else ctx ~ U{ctx_lo..ctx_hi} (inclusive)
    ctx_hi: int = 0
    shared_prefix: int = 0          # tokens of a prefix every sequence shares (page aligned)
    pool_pages: Optional[int] = None  # fixed pool size; else ceil((1+slack) * used)
    pool_slack: float = 0.10
    outlier_channels: int = 0       # channels (of H_kv*D) scaled by outlier_gain, K and V drawn separately
    outlier_gain: float = 1.0
    q_gain: float = 1.0
    v_gain: float = 1.0             # V rows (history and new) times v_gain (small or large V scales)
    q_len: int = 1                  # new query tokens per sequence (chunked prefill / verification)
    q_len_hi: int = 0               # > q_len: per-sequence chunk lengths ~ U{q_len..q_len_hi}
    sink_tokens: int = 0            # with window_tokens > 0: the cache holds only positions
    window_tokens: int = 0          #   < sink_tokens and the last window_tokens positions
    device_data: bool = False       # draw K/V/q on the GPU with torch's generator (too big for host)
    seed: int = BASE_SEED

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# C1: tiny case, small enough for brute force everywhere.
TINY = DecodeConfig(
    name="tiny", layers=1, batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
    page_size=16, ctx_fixed=(37, 100), pool_pages=16, seed=465001)

# C2: one Llama-3-8B-shaped attention layer, medium mixed context lengths.
LLAMA3_8B_LAYER = DecodeConfig(
    name="llama3_8b_layer", layers=1, batch=64, num_q_heads=32, num_kv_heads=8,
    head_dim=128, page_size=16, ctx_lo=512, ctx_hi=4096, seed=465002)

# C3: Llama-3-70B-shaped full cache, 80 layers x 32 sequences x 8192 tokens
# (85,899,345,920 bytes of bf16 K+V).
LLAMA3_70B_FULL = DecodeConfig(
    name="llama3_70b_full_cache", layers=80, batch=32, num_q_heads=64,
    num_kv_heads=8, head_dim=128, page_size=16, ctx_fixed=(8192,) * 32,
    pool_pages=32 * 512, device_data=True, seed=465003)

# C4: INT8 KV cache (per token, per KV head scale and zero point), long contexts,
# 10 of the 1024 (head, dim) channels scaled x8 as persistent outliers.
INT8_LONG = DecodeConfig(
    name="int8_long", layers=1, batch=16, num_q_heads=32, num_kv_heads=8,
    head_dim=128, page_size=32, kv_dtype="int8", ctx_lo=16385, ctx_hi=32769,
    outlier_channels=10, outlier_gain=8.0, seed=465004)

# C5: 100 sequences sharing one 2000-token prefix (125 pages of 16), each with
# its own 500-token suffix; multi-query attention (one KV head for 32 q heads).
SHARED_PREFIX_MQA = DecodeConfig(
    name="shared_prefix_mqa", layers=1, batch=100, num_q_heads=32, num_kv_heads=1,
    head_dim=128, page_size=16, ctx_fixed=(2500,) * 100, shared_prefix=2000,
    seed=465005)

CONFIGS = {c.name: c for c in (TINY, LLAMA3_8B_LAYER, LLAMA3_70B_FULL, INT8_LONG,
                               SHARED_PREFIX_MQA)}

# Streaming decode with attention sinks and a recent window ("KV-Cache
# Optimization Techniques", section "Token Eviction Strategies", eq. 5): a
# Llama-3-8B-shaped layer, 64 sequences that have reached 32,768 tokens, of
# which the cache still holds the first 4 and the last 4,096.
STREAMING_WINDOW = DecodeConfig(
    name="streaming_window", layers=1, batch=64, num_q_heads=32, num_kv_heads=8,
    head_dim=128, page_size=16, ctx_fixed=(32768,) * 64, sink_tokens=4, window_tokens=4096,
    seed=465006)

# Several new tokens per sequence against the paged cache ("KV-Cache
# Optimization Techniques", section "Cache-Aware Scheduling": chunked prefill).
# Verification of 4 drafted tokens per sequence on a Llama-3-70B-shaped layer:
SPEC_VERIFY = DecodeConfig(
    name="spec_verify", layers=1, batch=32, num_q_heads=64, num_kv_heads=8, head_dim=128,
    page_size=16, ctx_fixed=(4096,) * 32, q_len=4, seed=465007)

# A 512-token prompt chunk per sequence on a Llama-3-8B-shaped layer, the cache
# already holding 1.5k-7.5k tokens of each prompt (context incl. the chunk):
CHUNKED_PREFILL = DecodeConfig(
    name="chunked_prefill", layers=1, batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
    page_size=16, ctx_lo=2048, ctx_hi=8192, q_len=512, seed=465008)

# The long-context quantized cache with 4-bit codes (two per byte, same row
# contract with 16 levels) and with FP8 e4m3 values under a per-token scale
# ("KV-Cache Optimization Techniques", section "KV-Cache Quantization").
INT4_LONG = replace(INT8_LONG, name="int4_long", kv_dtype="int4", seed=465009)
FP8_LONG = replace(INT8_LONG, name="fp8_long", kv_dtype="fp8", seed=465010)

EXTRA_CONFIGS = {c.name: c for c in (STREAMING_WINDOW, SPEC_VERIFY, CHUNKED_PREFILL, INT4_LONG,
                                     FP8_LONG)}


def variant(cfg: DecodeConfig, **kw) -> DecodeConfig:
    """A copy of ``cfg`` with some fields changed (smaller parity shapes, g=1/2 ...)."""
    return replace(cfg, **kw)
