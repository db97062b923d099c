"""Pins of the write-side oracle (oracle/scatter.py): the K/V scatter that
fills the page pool.  Each pin is a fact fixed by the pages or by the
definition of paging, not a retyping of the scatter:

* the printed page contents of anllm "Tutorial 13" (section 4, Example
  Walkthrough): after appending 3, 2 and 4 tokens at page size 4 (each append
  opening new pages), page 0 holds t0 t1 t2 and one empty slot, page 1 holds
  t3 t4 and two empty slots, page 2 holds t5..t8;
* paging is exact ("Reading vLLM's PagedAttention Kernel", section 3.2: the
  read path gathers back exactly what the write path scattered): reading every
  request's slots in logical order returns its tokens, for interleaved decode
  steps and chunks of several requests sharing one pool;
* nothing else is written: free pages and unused tail slots keep their bytes,
  and negative (padding) or out-of-pool slots change nothing.
The pin functions take the scatter as an argument, so that planted mistakes
(test_mutants) can be run through them.
"""
import inspect
import json
import os
import textwrap

import numpy as np
import pytest

from oracle import scatter as oracle_scatter
from oracle.ledger import PageAllocator, RequestPages

GARBAGE = 1.0e4


def _tokens(rng, T, Hkv, D):
    return (rng.standard_normal((T, Hkv, D)).astype(np.float32),
            rng.standard_normal((T, Hkv, D)).astype(np.float32))


def pin_walkthrough_pages(scatter, golden_dir):
    with open(os.path.join(golden_dir, "anllm_append_walkthrough.json")) as f:
        g = json.load(f)
    ps, Hkv, D = g["page_size"], 2, 8
    kp = np.full((4, Hkv, ps, D), GARBAGE, np.float32)
    vp = kp.copy()
    cache = RequestPages(PageAllocator(ps), policy="walkthrough")
    rng = np.random.default_rng(11)
    k_all, v_all = [], []
    for n in g["appends"]:
        written = cache.append(n)
        k, v = _tokens(rng, n, Hkv, D)
        kp, vp = scatter(kp, vp, k, v, cache.slot_mapping(written))
        k_all.append(k)
        v_all.append(v)
    k_all, v_all = np.concatenate(k_all), np.concatenate(v_all)
    # the printed figure: token t at (page, slot) = expected_token_placement[t]
    for t, (page, slot) in enumerate(g["expected_token_placement"]):
        assert np.array_equal(kp[page, :, slot, :], k_all[t])
        assert np.array_equal(vp[page, :, slot, :], v_all[t])
    # the empty slots it prints: page 0 slot 3, page 1 slots 2 and 3; page 3 unused
    for page, slot in [(0, 3), (1, 2), (1, 3)]:
        assert np.all(kp[page, :, slot, :] == GARBAGE) and np.all(vp[page, :, slot, :] == GARBAGE)
    assert np.all(kp[3] == GARBAGE) and np.all(vp[3] == GARBAGE)


def pin_gather_returns_tokens(scatter, seed=0):
    rng = np.random.default_rng(seed)
    ps, Hkv, D, P = 4, 3, 8, 40
    pool = PageAllocator(ps)
    caches = [RequestPages(pool) for _ in range(3)]
    kp = np.full((P, Hkv, ps, D), GARBAGE, np.float32)
    vp = kp.copy()
    hist = {i: ([], []) for i in range(3)}
    # chunked prefills, then decode steps, then a second chunk, interleaved
    for step in [(0, 7), (1, 3), (2, 9), (0, 1), (1, 1), (2, 1), (0, 5), (1, 6), (2, 1), (0, 1)]:
        r, n = step
        written = caches[r].append(n)
        k, v = _tokens(rng, n, Hkv, D)
        kp, vp = scatter(kp, vp, k, v, caches[r].slot_mapping(written))
        hist[r][0].append(k)
        hist[r][1].append(v)
    used = set()
    for r, cache in enumerate(caches):
        order = cache.gather_order()
        got_k = np.stack([kp[p, :, s, :] for p, s in order])
        got_v = np.stack([vp[p, :, s, :] for p, s in order])
        assert np.array_equal(got_k, np.concatenate(hist[r][0]))
        assert np.array_equal(got_v, np.concatenate(hist[r][1]))
        used.update(order)
    for p in range(P):
        for s in range(ps):
            if (p, s) not in used:
                assert np.all(kp[p, :, s, :] == GARBAGE) and np.all(vp[p, :, s, :] == GARBAGE)


def pin_skipped_slots(scatter):
    rng = np.random.default_rng(3)
    ps, Hkv, D, P = 4, 2, 8, 3
    kp = rng.standard_normal((P, Hkv, ps, D)).astype(np.float32)
    vp = rng.standard_normal((P, Hkv, ps, D)).astype(np.float32)
    k, v = _tokens(rng, 4, Hkv, D)
    k2, v2 = scatter(kp, vp, k, v, [-1, P * ps, P * ps + 5, -7])
    assert np.array_equal(k2, kp) and np.array_equal(v2, vp)
    # a mixed mapping writes exactly the valid slots
    k3, v3 = scatter(kp, vp, k, v, [5, -1, 11, P * ps])
    assert np.array_equal(k3[1, :, 1, :], k[0]) and np.array_equal(k3[2, :, 3, :], k[2])
    assert np.array_equal(v3[1, :, 1, :], v[0]) and np.array_equal(v3[2, :, 3, :], v[2])
    mask = np.ones((P, ps), bool)
    mask[1, 1] = mask[2, 3] = False
    assert np.array_equal(k3.transpose(0, 2, 1, 3)[mask], kp.transpose(0, 2, 1, 3)[mask])


def test_walkthrough_pages(golden_dir):
    pin_walkthrough_pages(oracle_scatter.scatter_tokens, golden_dir)


@pytest.mark.parametrize("seed", [0, 1])
def test_gather_returns_tokens(seed):
    pin_gather_returns_tokens(oracle_scatter.scatter_tokens, seed)


def test_skipped_slots():
    pin_skipped_slots(oracle_scatter.scatter_tokens)


MUTANTS = {
    "page_offset_swapped": ("page, off = s // ps, s % ps", "off, page = s // ps, s % ps"),
    "page_from_pool_size": ("page, off = s // ps, s % ps", "page, off = s // P, s % ps"),
    "head_ignored": ("kp[page, h, off, :] = key[t, h, :]", "kp[page, 0, off, :] = key[t, h, :]"),
    "value_from_keys": ("vp[page, h, off, :] = value[t, h, :]", "vp[page, h, off, :] = key[t, h, :]"),
    "skip_only_negative": ("if s < 0 or s >= P * ps:", "if s < 0:"),
    "last_token_dropped": ("for t in range(T):", "for t in range(T - 1):"),
}


def _mutant(name):
    src = textwrap.dedent(inspect.getsource(oracle_scatter.scatter_tokens))
    a, b = MUTANTS[name]
    assert src.count(a) == 1, name
    ns = {"np": np}
    exec(src.replace(a, b), ns)  # noqa: S102 - a planted mistake in a copy of the oracle
    return ns["scatter_tokens"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, golden_dir):
    fn = _mutant(name)
    caught = False
    for pin in (lambda: pin_walkthrough_pages(fn, golden_dir), lambda: pin_gather_returns_tokens(fn),
                lambda: pin_skipped_slots(fn)):
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught = True
    assert caught, f"no pin rejects the planted mistake {name}"


@pytest.mark.parametrize("ps,pad", [(16, 0), (4, 3), (128, 1)])
def test_generated_slots_are_the_read_path_translation(ps, pad):
    # The write workloads place new token t of request b at position
    # ctx_old[b] + i; the read-side oracle's address translation of that
    # position must name the same (page, slot) -- the two directions of the
    # same indirection (section 3.2 of the vLLM reading).
    import oracle
    from workloads import make_append
    a = make_append(40 + ps, B=3, H_kv=2, D=64, page_size=ps, ctx_old=[0, ps + 1, 3 * ps],
                    n_new=[ps // 2 + 1, 1, 2 * ps + 3], dtype="bf16", pad_tokens=pad)
    p = a.paged
    tr = oracle.translate_of(p)
    want = []
    for b in range(p.B):
        for pos in range(int(a.ctx_old[b]), int(a.ctx_old[b] + a.n_new[b])):
            page, slot = tr[b, pos]
            want.append(int(page) * ps + int(slot))
    got = [int(s) for s in a.slot_mapping if s >= 0]
    assert got == want and int((a.slot_mapping < 0).sum()) == pad
    # and scattering then gathering through the block table returns the tokens
    kp, vp = oracle_scatter.scatter_tokens(p.key_pages, p.value_pages, a.key, a.value,
                                           a.slot_mapping)
    live = np.flatnonzero(a.slot_mapping >= 0)
    for i, t in enumerate(live):
        page, slot = divmod(want[i], ps)
        assert np.array_equal(kp[page, :, slot, :], a.key[t])
        assert np.array_equal(vp[page, :, slot, :], a.value[t])
