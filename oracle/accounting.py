"""Memory accounting closed forms -- CPU oracle (test infrastructure only).

* ``kv_bytes``: "Understanding KV-Cache Optimization in Modern LLM Serving",
  section "The Memory Math Behind KV-Cache": K plus V of one request take
  2 * L * H_kv * D * N * (bytes per element).  That page writes P for the
  bytes per element; here it is ``elem_bytes`` because P is the page size.
* ``paged_bytes`` / ``prefix_cached_bytes``: "KV-Cache Optimization
  Techniques", section "Prefix Caching", eq. 2, with c the bytes per token
  (c is not defined on the page; read as kv_bytes with N = 1).
* ``alloc_tokens`` / ``waste``: section "PagedAttention": a request holds
  ceil(n / P) pages, so at most P - 1 slots of its last page are unused.
* ``gqa_ratio``: section "Multi-Query and Grouped-Query Caching", eq. 7, the
  GQA/MHA cache-size ratio G / H with G the number of KV heads.
* ``window_cache_elems``: section "Sliding Window Cache", eq. 6: a window of
  w tokens holds w * 2 * L * d_k values per KV head, whatever the context.
"""
from __future__ import annotations


def kv_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, elem_bytes: float) -> float:
    return 2 * layers * kv_heads * head_dim * tokens * elem_bytes


def bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    """c of eq. 2: K+V bytes one token adds to the cache."""
    return kv_bytes(layers, kv_heads, head_dim, 1, elem_bytes)


def paged_bytes(requests: int, tokens: int, c: float) -> float:
    return requests * tokens * c


def prefix_cached_bytes(requests: int, tokens: int, shared: int, c: float) -> float:
    return shared * c + requests * (tokens - shared) * c


def alloc_tokens(n: int, page_size: int) -> int:
    return -(-n // page_size) * page_size


def waste(n: int, page_size: int) -> int:
    return alloc_tokens(n, page_size) - n


def gqa_ratio(kv_heads: int, q_heads: int) -> float:
    return kv_heads / q_heads


def int4_row_ratio(head_dim: int) -> float:
    """Bytes of an INT4 row (D/2 code bytes + float16 scale + zero) over bfloat16."""
    return (head_dim / 2 + 4) / (2 * head_dim)


def int8_row_ratio(head_dim: int) -> float:
    """Bytes of an INT8 row (D codes + float16 scale + float16 zero) over its
    bfloat16 size: the "2x" of section "KV-Cache Quantization" less metadata."""
    return (head_dim + 4) / (2 * head_dim)


def window_cache_elems(window: int, layers: int, head_dim: int) -> int:
    """Eq. 6: K and V values a w-token window keeps per KV head."""
    return window * 2 * layers * head_dim
