"""Page-pool ledger (write-side bookkeeping) -- TEST INFRASTRUCTURE ONLY.

Models the page pool and the per-request paged cache of anllm "Tutorial 13:
Paged Attention and Memory Management" (section 3 "The Page Pool", section 4
"The Request Cache", section 5 "Reading Pages for Attention") and the decode
rules of tiny-llm "Week 3 Day 4" ("Decode Metadata" and the invariants list in
"What Must Hold, and What Breaks If It Doesn't").  It tracks token *positions*,
not values: each appended token is given a (page, slot) and the ledger can
export the block_table row / context_len that the read path consumes.

Readings taken where the pages are open or inconsistent:

* Fresh page ids.  The printed allocate_page names an attribute it never
  defines; the plainest reading that matches the walkthrough's ids 0, 1, 2 is
  "fresh id = number of pages allocated so far", then increment.  Reuse pops
  the most recently freed id (a LIFO free list); freeing an id that is not in
  use raises (the pool's "already free" error on double release).
* Append policy.  The printed _append_chunk fills the partial tail page before
  opening new ones ("fill_tail"), which turns 3+2+4 tokens at page size 4 into
  page_lens [4, 4, 1].  The printed walkthrough of the same section instead
  opens new pages on every append and shows page_lens [3, 2, 4], offset 9.
  Both are modelled: ``policy="fill_tail"`` (the default; it is also what the
  decode rule "allocate a new page only if the tail page is full" requires) and
  ``policy="walkthrough"``.
* A block table plus one context length can only describe a request whose
  pages are all full except the last.  ``block_table_row`` therefore refuses a
  layout with a hole (a non-full page that is not the last one); the read path
  never sees such layouts.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


class DoubleFreeError(KeyError):
    pass


class HoleLayoutError(ValueError):
    pass


class PagePool:
    """Physical page ids of one layer's shared pool."""

    def __init__(self, page_size: int = 128):
        if page_size <= 0:
            raise ValueError("page_size must be positive")
        self.page_size = page_size
        self.free_page_ids: List[int] = []
        self.used_page_ids = set()
        self.num_allocated_pages = 0

    def allocate_page(self) -> int:
        if self.free_page_ids:
            page_id = self.free_page_ids.pop()
        else:
            page_id = self.num_allocated_pages
            self.num_allocated_pages += 1
        self.used_page_ids.add(page_id)
        return page_id

    def free_page(self, page_id: int) -> None:
        if page_id not in self.used_page_ids:
            raise DoubleFreeError(f"page {page_id} is already free")
        self.used_page_ids.remove(page_id)
        self.free_page_ids.append(page_id)


class PagedCache:
    """One request's page list in one layer: page_ids, page_lens, offset."""

    POLICIES = ("fill_tail", "walkthrough")

    def __init__(self, pool: PagePool, policy: str = "fill_tail"):
        if policy not in self.POLICIES:
            raise ValueError(f"unknown policy {policy!r}")
        self.pool = pool
        self.policy = policy
        self.page_ids: List[int] = []
        self.page_lens: List[int] = []
        self.offset = 0
        # placement[t] = (page, slot) of logical token t
        self.placement: List[Tuple[int, int]] = []

    def append(self, n_tokens: int) -> List[Tuple[int, int]]:
        """Write ``n_tokens`` new tokens; returns their (page, slot)s in order
        (the flat slot of each is page * page_size + slot)."""
        if n_tokens < 0:
            raise ValueError("n_tokens must be non-negative")
        ps = self.pool.page_size
        written: List[Tuple[int, int]] = []
        start = 0
        if (self.policy == "fill_tail" and self.page_ids and self.page_lens[-1] < ps
                and n_tokens > 0):
            page = self.page_ids[-1]
            take = min(ps - self.page_lens[-1], n_tokens)
            for k in range(take):
                written.append((page, self.page_lens[-1] + k))
            self.page_lens[-1] += take
            start = take
        while start < n_tokens:
            end = min(start + ps, n_tokens)
            page = self.pool.allocate_page()
            for k in range(end - start):
                written.append((page, k))
            self.page_ids.append(page)
            self.page_lens.append(end - start)
            start = end
        self.offset += n_tokens
        self.placement.extend(written)
        return written

    def slot_mapping(self, written: Sequence[Tuple[int, int]]) -> List[int]:
        ps = self.pool.page_size
        return [p * ps + s for p, s in written]

    def gather_order(self) -> List[Tuple[int, int]]:
        """(page, slot) of every stored token in logical order, reading only
        the valid prefix of each page (the gather_dense rule)."""
        out = []
        for page, n in zip(self.page_ids, self.page_lens):
            out.extend((page, s) for s in range(n))
        return out

    def has_hole(self) -> bool:
        ps = self.pool.page_size
        return any(n < ps for n in self.page_lens[:-1])

    def context_len(self) -> int:
        return self.offset

    def block_table_row(self, max_pages: int) -> List[int]:
        if self.has_hole():
            raise HoleLayoutError("a non-final page is not full; a block table plus a "
                                  "context length cannot describe this layout")
        if len(self.page_ids) > max_pages:
            raise ValueError("more pages than max_pages")
        return list(self.page_ids) + [-1] * (max_pages - len(self.page_ids))

    def release(self) -> None:
        for page in self.page_ids:
            self.pool.free_page(page)
        self.page_ids, self.page_lens, self.offset, self.placement = [], [], 0, []
