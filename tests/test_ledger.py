"""Pins of the write-side ledger (page pool + request cache)."""
import json
import os

import pytest

from oracle.ledger import DoubleFreeError, HoleLayoutError, PagePool, PagedCache


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "anllm_append_walkthrough.json")) as f:
        return json.load(f)


def test_p2_walkthrough_policy_reproduces_printed_states(golden_dir):
    g = _golden(golden_dir)
    cache = PagedCache(PagePool(g["page_size"]), policy="walkthrough")
    for n, want in zip(g["appends"], g["expected_after_each"]):
        cache.append(n)
        assert cache.page_ids == want["page_ids"]
        assert cache.page_lens == want["page_lens"]
        assert cache.offset == want["offset"]
    assert [list(p) for p in cache.placement] == g["expected_token_placement"]
    assert [list(p) for p in cache.gather_order()] == g["expected_token_placement"]
    # a hole (page 0 holds 3 of 4 slots) cannot be expressed by a block table
    with pytest.raises(HoleLayoutError):
        cache.block_table_row(4)


def test_p2_fill_tail_policy_packs_pages(golden_dir):
    g = _golden(golden_dir)
    cache = PagedCache(PagePool(g["page_size"]), policy="fill_tail")
    for n in g["appends"]:
        cache.append(n)
    want = g["fill_tail_expected"]
    assert (cache.page_ids, cache.page_lens, cache.offset) == (
        want["page_ids"], want["page_lens"], want["offset"])
    # packed layout: token t sits at (page t // 4, slot t % 4) of the list
    assert cache.gather_order() == [(t // 4, t % 4) for t in range(9)]
    assert cache.block_table_row(4) == [0, 1, 2, -1]
    assert cache.context_len() == 9


def test_decode_allocates_only_on_tail_overflow():
    pool = PagePool(4)
    cache = PagedCache(pool)
    cache.append(6)                          # pages [0, 1], tail holds 2
    allocs = []
    for _ in range(7):
        before = pool.num_allocated_pages
        cache.append(1)
        allocs.append(pool.num_allocated_pages - before)
    # tokens 7, 8 fill page 1; token 9 opens page 2; 10-12 fill it; 13 opens page 3
    assert allocs == [0, 0, 1, 0, 0, 0, 1]
    assert cache.page_lens == [4, 4, 4, 1]


def test_pool_reuses_freed_pages_lifo_and_rejects_double_free():
    pool = PagePool(2)
    a, b = PagedCache(pool), PagedCache(pool)
    a.append(5)                              # pages 0, 1, 2
    b.append(2)                              # page 3
    assert a.page_ids == [0, 1, 2] and b.page_ids == [3]
    a.release()
    assert sorted(pool.free_page_ids) == [0, 1, 2] and pool.used_page_ids == {3}
    c = PagedCache(pool)
    c.append(4)                              # reuses the last freed ids first
    assert c.page_ids == [2, 1]
    with pytest.raises(DoubleFreeError):
        pool.free_page(0)
    with pytest.raises(DoubleFreeError):
        pool.free_page(1) or pool.free_page(1)


def test_release_returns_every_page_exactly_once():
    pool = PagePool(3)
    caches = [PagedCache(pool) for _ in range(4)]
    for k, c in enumerate(caches):
        for n in (2, 5, 1, k + 1):
            c.append(n)
    owned = [p for c in caches for p in c.page_ids]
    assert len(owned) == len(set(owned)) == len(pool.used_page_ids)   # no aliasing
    for c in caches:
        c.release()
    assert pool.used_page_ids == set()
    assert sorted(pool.free_page_ids) == sorted(owned)


def test_slot_mapping_is_flat_page_slot():
    pool = PagePool(16)
    cache = PagedCache(pool)
    cache.append(20)
    written = cache.append(14)
    assert cache.slot_mapping(written) == [1 * 16 + 4 + k for k in range(12)] + [2 * 16, 2 * 16 + 1]
