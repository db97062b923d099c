"""Checks of the seeded workload generator (inputs only, no GPU)."""
import numpy as np
import pytest

from workloads import (bf16_bits_to_f32, f32_to_bf16_bits, make_c1, make_c3, make_random)


def _visited(x):
    """(page, slot) pairs that hold live tokens, from the generator's tables."""
    live = set()
    for b in range(x.B):
        for j in range(int(x.context_lens[b])):
            live.add((int(x.block_table[b, j // x.page_size]), j % x.page_size))
    return live


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.01171875, -2.5, 1e4, 3.0e38], np.float32)
    bits = f32_to_bf16_bits(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert bf16_bits_to_f32(bits).tolist()[:4] == [1.0, 1.0, 1.015625, -2.5]
    assert bf16_bits_to_f32(bits)[4] == 9984.0


def test_c1_shape_and_planted_garbage():
    x = make_c1()
    assert (x.B, x.H_q, x.H_kv, x.D, x.L, x.page_size, x.num_pages) == (2, 4, 4, 64, 1, 4, 16)
    assert x.context_lens.tolist() == [10, 7]
    assert x.block_table[0].tolist() == [12, 5, 3]
    assert x.block_table[1, 2] == -1 and len(set(x.block_table[1, :2]) & {12, 5, 3}) == 0
    live = _visited(x)
    assert len(live) == 17
    for p in range(16):
        for s in range(4):
            if (p, s) not in live:
                assert (x.key_pages[p, :, s] == 1e4).all() and (x.value_pages[p, :, s] == 1e4).all()
            else:
                assert np.abs(x.key_pages[p, :, s]).max() < 10


def test_same_seed_same_bytes():
    a = make_random(7, B=3, H_q=4, H_kv=2, L=2, D=8, page_size=4, ctx=(1, 20))
    b = make_random(7, B=3, H_q=4, H_kv=2, L=2, D=8, page_size=4, ctx=(1, 20))
    for f in ("query", "key_pages", "value_pages", "block_table", "context_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_c3_causal_chunk_shape():
    x = make_c3()
    assert (x.B, x.H_q, x.H_kv, x.L, x.D, x.page_size) == (4, 28, 4, 512, 128, 16)
    assert ((x.context_lens >= 512) & (x.context_lens <= 2560)).all()
    assert x.num_pages >= x.meta["live_pages"] * 1.1 - 1
    ids = x.block_table[x.block_table >= 0]
    assert len(ids) == len(set(ids.tolist())) == x.meta["live_pages"]


@pytest.mark.slow
def test_c5_shared_prefix_aliasing():
    from workloads import make_c5
    m = make_c5()
    bt = np.concatenate([m.decode.block_table, m.prefill.block_table])
    cl = np.concatenate([m.decode.context_lens, m.prefill.context_lens])
    shared = m.meta["shared_page_ids"]
    for r in m.meta["sharers"]:
        assert bt[r, :16].tolist() == shared and cl[r] >= 2048
    non = [r for r in range(56) if r not in m.meta["sharers"]]
    ids = [p for r in non for p in bt[r][bt[r] >= 0].tolist()]
    assert len(ids) == len(set(ids)) and not set(ids) & set(shared)
    assert (m.prefill.query_lens >= 64).all() and (m.prefill.query_lens <= 256).all()
    assert 0.85 <= m.meta["used_pages"] / m.decode.num_pages <= 0.9


def test_shared_groups_structure():
    """make_shared: groups of consecutive requests cover the batch; members'
    tables name the same physical pages below the group's prefix and distinct
    ones after it; every member row sees the whole prefix."""
    from workloads import make_shared
    sizes, pages = [3, 1, 2, 4], [4, 0, 2, 3]
    x, g = make_shared(21, H_q=8, H_kv=2, L=2, D=64, page_size=16, group_sizes=sizes,
                       prefix_pages=pages, suffix=(2, 50), query_lens=[2, 1, 0, 2, 2, 1, 2, 2, 1, 2])
    assert list(g.group_start) == [0, 3, 4, 6, 10] and g.max_group_size == 4
    assert list(g.prefix_lens) == [p * 16 for p in pages]
    for k in range(g.num_groups):
        s, e, P = g.group_start[k], g.group_start[k + 1], pages[k]
        for b in range(s, e):
            assert np.array_equal(x.block_table[b, :P], x.block_table[s, :P])
            assert x.context_lens[b] - x.rows_valid()[b] >= g.prefix_lens[k]
    own = [set(x.block_table[b, pages[next(k for k in range(4) if g.group_start[k + 1] > b)]:
                             (int(x.context_lens[b]) + 15) // 16].tolist()) for b in range(x.B)]
    for i in range(x.B):
        for j in range(i + 1, x.B):
            assert not (own[i] & own[j])


def test_c5_decode_grouped_is_a_permutation():
    from workloads import c5_decode_grouped, make_c5
    m = make_c5()
    x, g, order = c5_decode_grouped(m)
    dec = m.decode
    assert sorted(order.tolist()) == list(range(dec.B))
    assert np.array_equal(x.query, dec.query[order])
    assert np.array_equal(x.block_table, dec.block_table[order])
    assert np.array_equal(x.context_lens, dec.context_lens[order])
    n = int(g.group_start[1])
    assert n == sum(1 for b in m.meta["sharers"] if b < dec.B)
    shared = m.meta["shared_page_ids"]
    assert (x.block_table[:n, :len(shared)] == np.asarray(shared)).all()
    assert list(g.group_start) == [0, n] and list(g.prefix_lens) == [len(shared) * dec.page_size]
