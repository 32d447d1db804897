"""Page allocator semantics -- CPU oracle (test infrastructure only).

"KV-Cache Optimization Techniques", section "PagedAttention": physical memory
is divided into pages, each request has a page table, pages are allocated
only when needed and freed when the request completes; pages may be shared
by requests with a common prefix.  This model keeps what is unique about any
correct allocator -- which pages are in use, their reference counts, the free
count and which calls must fail -- and leaves the choice of page ids open
(any free page is a correct answer).  Parity unpinned for the id order.
"""
from __future__ import annotations

from collections import Counter
from typing import Dict, List


class AllocError(Exception):
    pass


class NoPages(AllocError):
    pass


class PoolModel:
    def __init__(self, num_pages: int):
        if num_pages <= 0:
            raise AllocError("empty pool")
        self.num_pages = num_pages
        self.ref: Dict[int, int] = {}

    @property
    def free_count(self) -> int:
        return self.num_pages - len(self.ref)

    def refcount(self, page: int) -> int:
        return self.ref.get(page, 0)

    def check_alloc(self, n: int, ids: List[int]) -> None:
        """Accept the ids an allocator returned for alloc(n), then record them."""
        if n < 0:
            raise AllocError("negative count")
        if n > self.free_count:
            raise NoPages()
        if len(ids) != n or len(set(ids)) != n:
            raise AssertionError("alloc must return n distinct ids")
        for p in ids:
            if not 0 <= p < self.num_pages or p in self.ref:
                raise AssertionError(f"alloc returned page {p} that is not free")
        for p in ids:
            self.ref[p] = 1

    def share(self, ids: List[int]) -> None:
        for p in ids:
            if p not in self.ref:
                raise AllocError(f"page {p} is not in use")
        for p in ids:
            self.ref[p] += 1

    def free(self, ids: List[int]) -> None:
        counts = Counter(ids)
        for p, c in counts.items():
            if self.ref.get(p, 0) < c:
                raise AllocError(f"page {p} freed more often than referenced")
        for p, c in counts.items():
            self.ref[p] -= c
            if self.ref[p] == 0:
                del self.ref[p]


def window_evicted_blocks(n: int, page_size: int, sink: int, window: int):
    """Logical blocks of a sequence of n tokens that hold no position a sink +
    window decode attends to ("KV-Cache Optimization Techniques", section
    "Token Eviction Strategies", eq. 5): every block of the sequence minus the
    blocks of the kept positions."""
    from .paged_attention import kept_positions
    nblk = -(-n // page_size)
    kept = set((kept_positions(n, sink, window) // page_size).tolist())
    return sorted(set(range(nblk)) - kept)
