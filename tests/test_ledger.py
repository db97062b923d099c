"""Pins of the write-side ledger (page pool + request cache)."""
import json
import os

import pytest

from oracle.ledger import DoubleFreeError, HoleLayoutError, PageAllocator, RequestPages


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "anllm_append_walkthrough.json")) as f:
        return json.load(f)


def test_p2_walkthrough_policy_reproduces_printed_states(golden_dir):
    g = _golden(golden_dir)
    cache = RequestPages(PageAllocator(g["page_size"]), policy="walkthrough")
    for n, want in zip(g["appends"], g["expected_after_each"]):
        cache.append(n)
        assert cache.pages == want["page_ids"]
        assert cache.fill == want["page_lens"]
        assert cache.length == want["offset"]
    assert [list(p) for p in cache.placement] == g["expected_token_placement"]
    assert [list(p) for p in cache.gather_order()] == g["expected_token_placement"]
    # a hole (page 0 holds 3 of 4 slots) cannot be expressed by a block table
    with pytest.raises(HoleLayoutError):
        cache.block_table_row(4)


def test_p2_fill_tail_policy_packs_pages(golden_dir):
    g = _golden(golden_dir)
    cache = RequestPages(PageAllocator(g["page_size"]), policy="fill_tail")
    for n in g["appends"]:
        cache.append(n)
    want = g["fill_tail_expected"]
    assert (cache.pages, cache.fill, cache.length) == (
        want["page_ids"], want["page_lens"], want["offset"])
    # packed layout: token t sits at (page t // 4, slot t % 4) of the list
    assert cache.gather_order() == [(t // 4, t % 4) for t in range(9)]
    assert cache.block_table_row(4) == [0, 1, 2, -1]
    assert cache.context_len() == 9


def test_decode_allocates_only_on_tail_overflow():
    pool = PageAllocator(4)
    cache = RequestPages(pool)
    cache.append(6)                          # pages [0, 1], tail holds 2
    allocs = []
    for _ in range(7):
        before = pool.fresh_count
        cache.append(1)
        allocs.append(pool.fresh_count - before)
    # tokens 7, 8 fill page 1; token 9 opens page 2; 10-12 fill it; 13 opens page 3
    assert allocs == [0, 0, 1, 0, 0, 0, 1]
    assert cache.fill == [4, 4, 4, 1]


def test_pool_reuses_freed_pages_lifo_and_rejects_double_free():
    pool = PageAllocator(2)
    a, b = RequestPages(pool), RequestPages(pool)
    a.append(5)                              # pages 0, 1, 2
    b.append(2)                              # page 3
    assert a.pages == [0, 1, 2] and b.pages == [3]
    a.release()
    assert sorted(pool.recycled) == [0, 1, 2] and pool.in_use == {3}
    c = RequestPages(pool)
    c.append(4)                              # reuses the last freed ids first
    assert c.pages == [2, 1]
    with pytest.raises(DoubleFreeError):
        pool.give_back(0)
    with pytest.raises(DoubleFreeError):
        pool.give_back(1) or pool.give_back(1)


def test_release_returns_every_page_exactly_once():
    pool = PageAllocator(3)
    caches = [RequestPages(pool) for _ in range(4)]
    for k, c in enumerate(caches):
        for n in (2, 5, 1, k + 1):
            c.append(n)
    owned = [p for c in caches for p in c.pages]
    assert len(owned) == len(set(owned)) == len(pool.in_use)   # no aliasing
    for c in caches:
        c.release()
    assert pool.in_use == set()
    assert sorted(pool.recycled) == sorted(owned)


def test_slot_mapping_is_flat_page_slot():
    pool = PageAllocator(16)
    cache = RequestPages(pool)
    cache.append(20)
    written = cache.append(14)
    assert cache.slot_mapping(written) == [1 * 16 + 4 + k for k in range(12)] + [2 * 16, 2 * 16 + 1]
