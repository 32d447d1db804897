"""CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library never does, and this
package imports nothing from the library.  Everything here is plain numpy,
float64 for attention, float32 where the quantization contract fixes it.

Modules:
  paged_attention  eq. 1 over gathered pages; causal multi-query chunks;
                   sinks + window (eq. 5, eq. 6);
                   append (slot write / quantize)
  quantize         eq. 3 per-token INT8 rows
  accounting       memory closed forms (memory formula, eq. 2, eq. 7, waste)
  allocator        page allocator semantics (parity unpinned for id order)
  prefix           prefix caching: longest cached whole-block prefix (eq. 2)
"""
from .accounting import (alloc_tokens, bytes_per_token, gqa_ratio, int8_row_ratio, kv_bytes,
                         paged_bytes, prefix_cached_bytes, waste, window_cache_elems)
from .allocator import AllocError, NoPages, PoolModel, window_evicted_blocks
from .paged_attention import (PoolLayout, append, attend, gather_positions, gather_sequence,
                              kept_positions, paged_decode, paged_decode_window, paged_prefill,
                              slot)
from .prefix import PrefixModel
from .quantize import dequantize, quantize_rows

__all__ = [
    "alloc_tokens", "bytes_per_token", "gqa_ratio", "int8_row_ratio", "kv_bytes", "paged_bytes",
    "prefix_cached_bytes", "waste", "window_cache_elems", "AllocError", "NoPages", "PoolModel",
    "window_evicted_blocks", "PoolLayout", "append", "attend", "gather_positions",
    "gather_sequence", "kept_positions", "paged_decode", "paged_decode_window", "paged_prefill",
    "slot",
    "dequantize", "quantize_rows", "PrefixModel",
]
