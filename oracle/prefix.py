"""Prefix caching semantics -- CPU oracle (test infrastructure only).

"KV-Cache Optimization Techniques", section "Prefix Caching": requests that
share a prefix reuse its KV-cache; memory for N requests of T tokens sharing
P_shared of them is P_shared*c + N*(T - P_shared)*c (eq. 2); cached prefixes
are looked up by longest-prefix match.  Written here as the plainest model:
every cached block is keyed by the whole token prefix up to and including it
(a tuple of token ids), so "the longest cached prefix" is the largest k whose
first k blocks are all keys.  The hash function and tree structure of an
implementation are its own choices: parity unpinned for them; what is pinned
is which blocks match and which pages they name.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple


class PrefixModel:
    def __init__(self, page_size: int):
        self.page_size = page_size
        self.blocks: Dict[Tuple[int, ...], int] = {}   # prefix (whole blocks) -> page of its last block

    def insert(self, tokens: Sequence[int], pages: Sequence[int]) -> None:
        """Cache every full block of a sequence whose K/V sit in ``pages``;
        blocks already cached keep their page."""
        P = self.page_size
        for k in range(1, len(tokens) // P + 1):
            key = tuple(int(t) for t in tokens[:k * P])
            if key not in self.blocks:
                self.blocks[key] = int(pages[k - 1])

    def match(self, tokens: Sequence[int]) -> List[int]:
        """Pages of the longest cached prefix of whole blocks."""
        P = self.page_size
        pages = []
        k = 1
        while k * P <= len(tokens):
            key = tuple(int(t) for t in tokens[:k * P])
            if key not in self.blocks:
                break
            pages.append(self.blocks[key])
            k += 1
        return pages

    def unique_pages(self) -> int:
        return len(set(self.blocks.values()))
