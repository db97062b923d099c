"""Page-pool ledger (write-side bookkeeping) -- TEST INFRASTRUCTURE ONLY.

A model of where the tokens of each request land in a shared page pool, as
anllm "Tutorial 13: Paged Attention and Memory Management" describes it
(section 3, the page pool; section 4, the per-request cache and its append;
section 5, reading the valid part of each page back for attention) and as
tiny-llm "Week 3 Day 4" states the decode-side rules (section "Decode
Metadata" and the invariants of "What Must Hold, and What Breaks If It
Doesn't").  Only positions are tracked: every appended token gets a physical
(page, slot), and a request can be exported as the block-table row and the
context length that the read path takes.

Readings where the pages leave a step open or disagree with themselves:

* Which id a new page gets.  The printed allocator refers to a pool size it
  never sets; the reading that reproduces the walkthrough's ids 0, 1, 2 is
  that never-used ids are handed out in increasing order starting at 0, and
  that a released id is reused before any never-used one, the most recently
  released first.  Releasing an id that is not in use is an error.
* Where an append starts.  The printed append code first tops up the
  request's last page if it has room, and only then opens new pages; with
  pages of 4 slots, appends of 3, 2 and 4 tokens then fill pages of 4, 4 and
  1 tokens.  The walkthrough printed next to it instead begins every append
  on a new page and shows pages of 3, 2 and 4 tokens with 9 tokens stored.
  Both are modelled: ``policy="fill_tail"`` (default; it is also what the
  decode rule needs, under which a request opens a page only once its last
  page has no free slot) and ``policy="walkthrough"``.
* A block-table row plus one context length can only describe a request
  whose pages are all full except possibly the last; exporting a layout with
  a partly filled page before the last one is refused.  The read path never
  sees such layouts.
"""
from __future__ import annotations

from typing import List, Sequence, Set, Tuple

Placement = Tuple[int, int]  # (physical page, slot in the page)


class DoubleFreeError(KeyError):
    pass


class HoleLayoutError(ValueError):
    pass


class PageAllocator:
    """The physical page ids of one layer's pool: never-used ids in
    increasing order, released ids reused most recent first."""

    def __init__(self, page_size: int = 128):
        if page_size <= 0:
            raise ValueError("page_size must be positive")
        self.page_size = page_size
        self.fresh_count = 0            # ids 0 .. fresh_count - 1 have been handed out
        self.recycled: List[int] = []   # released ids; the end of the list is reused first
        self.in_use: Set[int] = set()

    def take(self) -> int:
        pid = self.recycled.pop() if self.recycled else self._fresh()
        self.in_use.add(pid)
        return pid

    def _fresh(self) -> int:
        pid = self.fresh_count
        self.fresh_count += 1
        return pid

    def give_back(self, pid: int) -> None:
        if pid not in self.in_use:
            raise DoubleFreeError(f"page {pid} is not in use")
        self.in_use.discard(pid)
        self.recycled.append(pid)


class RequestPages:
    """The pages one request holds in one layer: `pages` (physical ids in
    logical order), `fill` (tokens stored in each) and `length` (tokens
    stored in all), plus `placement[t]`, the (page, slot) of token t."""

    POLICIES = ("fill_tail", "walkthrough")

    def __init__(self, alloc: PageAllocator, policy: str = "fill_tail"):
        if policy not in self.POLICIES:
            raise ValueError(f"unknown policy {policy!r}")
        self.alloc = alloc
        self.policy = policy
        self.pages: List[int] = []
        self.fill: List[int] = []
        self.length = 0
        self.placement: List[Placement] = []

    def _needs_new_page(self, first_of_append: bool) -> bool:
        if not self.pages or self.fill[-1] == self.alloc.page_size:
            return True
        return first_of_append and self.policy == "walkthrough"

    def append(self, n_tokens: int) -> List[Placement]:
        """Store `n_tokens` new tokens one by one; returns their placements in
        order (token t's flat slot is page * page_size + slot)."""
        if n_tokens < 0:
            raise ValueError("n_tokens must be non-negative")
        placed: List[Placement] = []
        for k in range(n_tokens):
            if self._needs_new_page(k == 0):
                self.pages.append(self.alloc.take())
                self.fill.append(0)
            placed.append((self.pages[-1], self.fill[-1]))
            self.fill[-1] += 1
        self.length += n_tokens
        self.placement.extend(placed)
        return placed

    def slot_mapping(self, placed: Sequence[Placement]) -> List[int]:
        return [page * self.alloc.page_size + slot for page, slot in placed]

    def gather_order(self) -> List[Placement]:
        """(page, slot) of every stored token in logical order, reading only
        the filled part of each page."""
        return [(page, slot) for page, used in zip(self.pages, self.fill)
                for slot in range(used)]

    def has_hole(self) -> bool:
        return any(used < self.alloc.page_size for used in self.fill[:-1])

    def context_len(self) -> int:
        return self.length

    def block_table_row(self, max_pages: int) -> List[int]:
        if self.has_hole():
            raise HoleLayoutError("a page before the last is only partly filled; a block "
                                  "table plus a context length cannot describe it")
        if len(self.pages) > max_pages:
            raise ValueError("more pages than max_pages")
        return self.pages + [-1] * (max_pages - len(self.pages))

    def release(self) -> None:
        for pid in self.pages:
            self.alloc.give_back(pid)
        self.pages, self.fill, self.length, self.placement = [], [], 0, []
