"""Pins of the CPU oracle against facts the pages and the mathematics fix.

These run on the fp64 build at fp64 tolerances; tests/test_oracle_f32_pins.py
runs the same pins on the fp32 build with tolerances of fp32 rounding.
Each test names the pin it implements.  None of them re-types the oracle's
formula: expected values come from the pages' printed examples, from closed
forms, from library routines on dense data, or from invariances.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import OracleError
from tests._dense import dense_attention_rows, scatter_with_ledger
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_c1, make_random

LIB = oracle._LIB


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _as_f64(x, dtype):
    return bf16_bits_to_f32(x).astype(np.float64) if dtype == "bf16" else np.asarray(x, np.float64)


# --------------------------------------------------------------------------- P1
def test_p1_translate_tinyllm_block_table_example(golden_dir, lib_path=LIB):
    g = _golden(golden_dir, "tinyllm_block_table_example.json")
    ps, ctx = g["page_size"], g["context_len"]
    bt = np.array([g["page_ids"]], dtype=np.int32)
    tr = oracle.translate(bt, np.array([ctx], np.int32), ps, 16, lib_path=lib_path)
    assert tr.shape == (1, 3 * ps, 2)
    assert tr[0, :ctx, 0].tolist() == g["expected_page_of_token"]
    # slot = position within the page: 0..3, 0..3, 0..1
    assert tr[0, :ctx, 1].tolist() == [0, 1, 2, 3, 0, 1, 2, 3, 0, 1]
    assert (tr[0, ctx:] == -1).all()


def test_p1_translate_page_analogy(golden_dir, lib_path=LIB):
    g = _golden(golden_dir, "anllm_page_analogy.json")
    ps = 5
    bt = np.array([g["block_table"]], dtype=np.int32)
    ctx = ps * len(g["block_table"])
    tr = oracle.translate(bt, np.array([ctx], np.int32), ps, 8, lib_path=lib_path)
    pages_of_logical = [int(tr[0, lp * ps, 0]) for lp in range(len(g["block_table"]))]
    assert pages_of_logical == g["expected_physical_of_logical_page"]


def test_p1_translate_worked_example_placement(golden_dir, lib_path=LIB):
    g = _golden(golden_dir, "vllm_reading_worked_example.json")
    bt = np.array([g["block_table"]], dtype=np.int32)
    tr = oracle.translate(bt, np.array([g["seq_len"]], np.int32), g["block_size"], 5,
                          lib_path=lib_path)
    assert tr[0, :g["seq_len"]].tolist() == g["expected_token_location"]


def test_translate_rejects_bad_ids_but_ignores_padding(lib_path=LIB):
    bt = np.array([[2, -1, -1], [0, 1, 7]], dtype=np.int32)
    # request 0 needs one page; -1 padding after it is never read
    tr = oracle.translate(bt, np.array([3, 9], np.int32), 4, 8, lib_path=lib_path)
    assert (tr[0, :3, 0] == 2).all()
    with pytest.raises(OracleError) as e:
        oracle.translate(bt, np.array([5, 9], np.int32), 4, 8, lib_path=lib_path)
    assert e.value.code == 2
    with pytest.raises(OracleError) as e:
        oracle.translate(bt, np.array([3, 13], np.int32), 4, 8, lib_path=lib_path)
    assert e.value.code == 3


# --------------------------------------------------------------------------- P3
def _worked_example_inputs(g):
    D, bs, n = g["head_dim"], g["block_size"], g["seq_len"]
    bt = g["block_table"]
    P = max(bt) + 1
    kp = np.full((P, 1, bs, D), 1e4, dtype=np.float32)
    vp = np.full((P, 1, bs, D), -1e4, dtype=np.float32)
    for t, (page, slot) in enumerate(g["expected_token_location"]):
        kp[page, 0, slot] = g["K"][t]
        vp[page, 0, slot] = g["V"][t]
    q = np.array(g["q"], dtype=np.float32).reshape(1, 1, 1, D)
    return q, kp, vp, np.array([bt], np.int32), np.array([n], np.int32)


def test_p3_worked_example_matches_printed_output(golden_dir, lib_path=LIB):
    g = _golden(golden_dir, "vllm_reading_worked_example.json")
    q, kp, vp, bt, cl = _worked_example_inputs(g)
    # inputs are float32 copies of the printed decimals; float32 rounding of
    # them moves the result by < 1e-7, well inside the printed half-ulp
    out = oracle.attention(q, kp, vp, bt, cl, g["block_size"], dtype="f32", causal=True,
                           scale=g["scale"], lib_path=lib_path)
    got = out[0, 0, 0]
    tol = 0.5 * 10.0 ** (-g["printed_decimals"]) + 2e-7
    np.testing.assert_allclose(got, g["expected_output_6dp"], rtol=0, atol=tol)
    # scale 1/sqrt(head_dim) is what the example uses
    assert g["scale"] == pytest.approx(1 / math.sqrt(g["head_dim"]))


def test_p3_worked_example_paged_equals_dense(golden_dir, lib_path=LIB, atol=1e-15):
    g = _golden(golden_dir, "vllm_reading_worked_example.json")
    q, kp, vp, bt, cl = _worked_example_inputs(g)
    out = oracle.attention(q, kp, vp, bt, cl, g["block_size"], dtype="f32", causal=False,
                           scale=g["scale"], lib_path=lib_path)[0, 0, 0]
    dense = dense_attention_rows(q.reshape(1, -1).astype(np.float64),
                                 np.array(g["K"], np.float32), np.array(g["V"], np.float32),
                                 g["scale"], [g["seq_len"]])[0]
    assert np.max(np.abs(out - dense)) <= atol


# --------------------------------------------------------------------------- P4
@pytest.mark.parametrize("seed,ps,H_q,H_kv,L,causal", [
    (10, 1, 2, 1, 1, True), (11, 3, 4, 2, 1, True), (12, 4, 6, 2, 3, True),
    (13, 5, 3, 3, 4, False), (14, 8, 8, 2, 5, True), (15, 2, 1, 1, 2, True)])
def test_p4_brute_force_vs_dense_library_softmax(seed, ps, H_q, H_kv, L, causal, lib_path=LIB,
                                                 atol=1e-12):
    rng = np.random.default_rng(seed)
    B, D = 3, 8
    G = H_q // H_kv
    n_tok = [int(rng.integers(L, 4 * ps + L + 3)) for _ in range(B)]
    dk = [rng.standard_normal((H_kv, n, D)) for n in n_tok]
    dv = [rng.standard_normal((H_kv, n, D)) for n in n_tok]
    kp, vp, bt, cl = scatter_with_ledger(rng, dk, dv, ps, 3, 1e4)
    assert cl.tolist() == n_tok
    q = rng.standard_normal((B, H_q, L, D))
    scale = 0.37
    out = oracle.attention(q.astype(np.float32), kp.astype(np.float32), vp.astype(np.float32),
                           bt, cl, ps, dtype="f32", causal=causal, scale=scale, lib_path=lib_path)
    q32 = q.astype(np.float32).astype(np.float64)
    for b in range(B):
        n = n_tok[b]
        vis = [(n - L + i + 1) if causal else n for i in range(L)]
        for h in range(H_q):
            g = h // G
            ref = dense_attention_rows(q32[b, h], dk[b][g].astype(np.float32),
                                       dv[b][g].astype(np.float32), scale, vis)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=atol)


def test_p4_bf16_widening_is_exact(lib_path=LIB, atol=1e-12):
    x = make_random(21, B=2, H_q=2, H_kv=1, L=1, D=16, page_size=4, ctx=[5, 9],
                    dtype="bf16", causal=False)
    out = oracle.attention_of(x, lib_path=lib_path)
    # widen with an independent route: float32 view of the bits << 16
    k = x.key_pages.astype(np.uint32) << 16
    kf = k.view(np.float32).astype(np.float64)
    v = (x.value_pages.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qf = (x.query.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for b in range(2):
        n = int(x.context_lens[b])
        pages = x.block_table[b, :(n + 3) // 4]
        K = kf[pages, 0].reshape(-1, 16)[:n]
        V = v[pages, 0].reshape(-1, 16)[:n]
        for h in range(2):
            ref = dense_attention_rows(qf[b, h], K, V, x.scale, [n])
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=atol)


# --------------------------------------------------------------------------- P5
def test_p5_physical_relabel_is_bit_identical(lib_path=LIB):
    x = make_random(31, B=3, H_q=4, H_kv=2, L=3, D=16, page_size=4, ctx=(3, 30),
                    dtype="bf16", causal=True, extra_free_pages=5)
    ref = oracle.attention_of(x, lib_path=lib_path)
    rng = np.random.default_rng(5)
    pi = rng.permutation(x.num_pages)            # new id of old page p is pi[p]
    kp2 = np.empty_like(x.key_pages)
    vp2 = np.empty_like(x.value_pages)
    kp2[pi] = x.key_pages
    vp2[pi] = x.value_pages
    bt2 = np.where(x.block_table >= 0, pi[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    out = oracle.attention(x.query, kp2, vp2, bt2, x.context_lens, x.page_size, dtype="bf16",
                           causal=True, scale=x.scale, lib_path=lib_path)
    assert np.array_equal(out, ref)


# --------------------------------------------------------------------------- P6
@pytest.mark.parametrize("garbage", [1e4, -1e4, 0.0, "random", "nan"])
def test_p6_stale_data_is_ignored_bit_identically(garbage, lib_path=LIB):
    kw = dict(B=3, H_q=4, H_kv=2, L=2, D=16, page_size=4, ctx=[5, 8, 11], dtype="f32",
              causal=True, extra_free_pages=4)
    base = make_random(41, garbage=1e4, **kw)
    other = make_random(41, garbage=garbage, **kw)
    live = np.zeros(base.key_pages.shape[:1] + base.key_pages.shape[2:3], dtype=bool)
    for b in range(3):
        for j in range(int(base.context_lens[b])):
            live[base.block_table[b, j // 4], j % 4] = True
    # same live values, different stale values
    assert np.array_equal(base.key_pages[live.nonzero()[0], :, live.nonzero()[1]],
                          other.key_pages[live.nonzero()[0], :, live.nonzero()[1]])
    a = oracle.attention_of(base, lib_path=lib_path)
    b = oracle.attention_of(other, lib_path=lib_path)
    assert np.array_equal(a, b)
    assert np.isfinite(b).all()


# --------------------------------------------------------------------------- P7
def test_p7_logical_reorder(lib_path=LIB, atol=1e-13):
    rng = np.random.default_rng(71)
    ps, D, n_pages = 4, 8, 5
    n = ps * n_pages                                  # complete pages only
    K = rng.standard_normal((1, n, D)).astype(np.float32)
    V = rng.standard_normal((1, n, D)).astype(np.float32)
    perm = rng.permutation(n_pages)
    Kp = K.reshape(1, n_pages, ps, D)[:, perm].reshape(1, n, D)
    Vp = V.reshape(1, n_pages, ps, D)[:, perm].reshape(1, n, D)

    def run(Kd, Vd, q, L, causal):
        kp, vp, bt, cl = scatter_with_ledger(np.random.default_rng(1), [Kd], [Vd], ps, 2, 1e4,
                                             appends=[[ps] * n_pages])
        return oracle.attention(q, kp.astype(np.float32), vp.astype(np.float32), bt, cl, ps,
                                dtype="f32", causal=causal, scale=0.3, lib_path=lib_path)

    q1 = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    a, b = run(K, V, q1, 1, True), run(Kp, Vp, q1, 1, True)
    np.testing.assert_allclose(a, b, rtol=0, atol=atol)      # decode: order-free
    qL = rng.standard_normal((1, 1, 6, D)).astype(np.float32)
    a, b = run(K, V, qL, 6, True), run(Kp, Vp, qL, 6, True)
    assert np.max(np.abs(a - b)) > 1e-3                       # causal prefix: order matters


# --------------------------------------------------------------------------- P8
def test_p8_single_key_returns_its_value(lib_path=LIB):
    x = make_random(81, B=2, H_q=3, H_kv=3, L=1, D=16, page_size=4, ctx=[1, 1],
                    dtype="bf16", causal=True)
    out = oracle.attention_of(x, lib_path=lib_path)
    for b in range(2):
        p = x.block_table[b, 0]
        v = _as_f64(x.value_pages[p, :, 0, :], "bf16")      # [H_kv, D]
        assert np.array_equal(out[b, :, 0], v)


def test_p8_equal_keys_or_zero_query_give_mean_of_values(lib_path=LIB, atol=1e-13):
    x = make_random(82, B=2, H_q=2, H_kv=1, L=1, D=8, page_size=3, ctx=[7, 10],
                    dtype="f32", causal=True)
    kp = x.key_pages.copy()
    kp[:] = 0.25                                              # every key identical
    out = oracle.attention(x.query, kp, x.value_pages, x.block_table, x.context_lens, 3,
                           dtype="f32", causal=True, scale=x.scale, lib_path=lib_path)
    q0 = np.zeros_like(x.query)
    out0 = oracle.attention(q0, x.key_pages, x.value_pages, x.block_table, x.context_lens, 3,
                            dtype="f32", causal=True, scale=x.scale, lib_path=lib_path)
    for b in range(2):
        n = int(x.context_lens[b])
        rows = [x.value_pages[x.block_table[b, j // 3], 0, j % 3] for j in range(n)]
        mean = np.mean(np.array(rows, np.float64), axis=0)
        for h in range(2):
            np.testing.assert_allclose(out[b, h, 0], mean, rtol=0, atol=atol)
            np.testing.assert_allclose(out0[b, h, 0], mean, rtol=0, atol=atol)


def test_p8_full_causal_is_lower_triangular_textbook(lib_path=LIB, atol=1e-12):
    rng = np.random.default_rng(83)
    n, D, ps = 11, 8, 4
    K = rng.standard_normal((1, n, D))
    V = rng.standard_normal((1, n, D))
    kp, vp, bt, cl = scatter_with_ledger(rng, [K], [V], ps, 2, 1e4)
    q = rng.standard_normal((1, 1, n, D))
    out = oracle.attention(q.astype(np.float32), kp.astype(np.float32), vp.astype(np.float32),
                           bt, cl, ps, dtype="f32", causal=True, scale=0.5, lib_path=lib_path)
    q32, K32, V32 = (a.astype(np.float32).astype(np.float64) for a in (q[0, 0], K[0], V[0]))
    logits = q32 @ K32.T * 0.5
    logits[np.triu_indices(n, 1)] = -np.inf
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    ref = (w / w.sum(axis=1, keepdims=True)) @ V32
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=atol)


def test_p8_chunk_rows_equal_last_rows_of_full_causal(lib_path=LIB):
    """Bottom-right alignment: a chunk of the last L rows after a prefix is
    the same computation as those rows of causal attention over everything."""
    x = make_random(84, B=2, H_q=4, H_kv=2, L=9, D=16, page_size=4, ctx=[9, 9],
                    dtype="f32", causal=True)
    full = oracle.attention_of(x, lib_path=lib_path)
    for L in (1, 3, 5):
        q = np.ascontiguousarray(x.query[:, :, 9 - L:, :])
        out = oracle.attention(q, x.key_pages, x.value_pages, x.block_table, x.context_lens,
                               4, dtype="f32", causal=True, scale=x.scale, lib_path=lib_path)
        assert np.array_equal(out, full[:, :, 9 - L:, :])


def test_p8_gqa_equals_mha_on_repeated_kv(lib_path=LIB):
    G = 3
    x = make_random(85, B=2, H_q=6, H_kv=2, L=2, D=8, page_size=4, ctx=[6, 13],
                    dtype="f32", causal=True)
    out = oracle.attention_of(x, lib_path=lib_path)
    kp = np.repeat(x.key_pages, G, axis=1)       # head h of the MHA pool = kv head h // G
    vp = np.repeat(x.value_pages, G, axis=1)
    mha = oracle.attention(x.query, kp, vp, x.block_table, x.context_lens, 4, dtype="f32",
                           causal=True, scale=x.scale, lib_path=lib_path)
    assert np.array_equal(out, mha)


def test_p8_noncausal_rows_see_whole_context_and_qlen_padding_is_zero(lib_path=LIB,
                                                                      atol=1e-12):
    x = make_random(86, B=3, H_q=2, H_kv=1, L=4, D=8, page_size=4, ctx=[5, 10, 3],
                    dtype="f32", causal=False, query_lens=[4, 2, 0])
    out = oracle.attention_of(x, lib_path=lib_path)
    assert (out[1, :, 2:] == 0).all() and (out[2] == 0).all()
    # non-causal: every valid row of a request sees the same keys
    for b, n in ((0, 5), (1, 10)):
        pages = x.block_table[b]
        K = np.array([x.key_pages[pages[j // 4], 0, j % 4] for j in range(n)], np.float64)
        V = np.array([x.value_pages[pages[j // 4], 0, j % 4] for j in range(n)], np.float64)
        for h in range(2):
            ref = dense_attention_rows(x.query[b, h].astype(np.float64), K, V, x.scale, [n] * 4)
            rows = int(x.query_lens[b])
            np.testing.assert_allclose(out[b, h, :rows], ref[:rows], rtol=0, atol=atol)


def test_p8_empty_context_gives_zeros(lib_path=LIB):
    x = make_random(87, B=2, H_q=2, H_kv=2, L=1, D=8, page_size=4, ctx=[0, 6],
                    dtype="bf16", causal=False)
    out = oracle.attention_of(x, lib_path=lib_path)
    assert (out[0] == 0).all() and np.isfinite(out).all() and (out[1] != 0).any()


# --------------------------------------------------------------------------- P9
def _online_page_walk(q, pages_k, pages_v, valid, scale):
    """The per-tile online-softmax recurrence of tiny-llm "Task 2: Define
    paged_attention": running max, rescaled running sum and output, one page
    tile at a time; divide at the end."""
    m, l, acc = -math.inf, 0.0, np.zeros(q.shape[0])
    for K, V, n in zip(pages_k, pages_v, valid):
        if n == 0:
            continue
        s = (K[:n] @ q) * scale
        page_max = float(np.max(s))
        new_m = max(m, page_max)
        e = np.exp(s - new_m)
        corr = math.exp(m - new_m) if m != -math.inf else 0.0
        l = l * corr + float(e.sum())
        acc = acc * corr + e @ V[:n]
        m = new_m
    return acc / l if l > 0 else acc


def test_p9_online_page_walk_equals_two_pass(lib_path=LIB, rtol=1e-12, atol=1e-13):
    x = make_random(91, B=4, H_q=4, H_kv=2, L=1, D=16, page_size=5, ctx=(1, 40),
                    dtype="bf16", causal=True)
    out = oracle.attention_of(x, lib_path=lib_path)
    kf = _as_f64(x.key_pages, "bf16")
    vf = _as_f64(x.value_pages, "bf16")
    qf = _as_f64(x.query, "bf16")
    for b in range(4):
        n = int(x.context_lens[b])
        npg = (n + 4) // 5
        pages = x.block_table[b, :npg]
        valid = [min(5, n - 5 * i) for i in range(npg)]
        for h in range(4):
            g = h // 2
            ref = _online_page_walk(qf[b, h, 0], kf[pages, g], vf[pages, g], valid, x.scale)
            np.testing.assert_allclose(out[b, h, 0], ref, rtol=rtol, atol=atol)


# -------------------------------------------------------------------------- P10
@pytest.mark.parametrize("P_tok", [4, 8, 12, 64])
def test_p10_split_merge_equals_unsplit(P_tok, lib_path=LIB, atol=1e-13):
    x = make_random(101, B=3, H_q=4, H_kv=2, L=3, D=8, page_size=4, ctx=[3, 17, 40],
                    dtype="f32", causal=True)
    full = oracle.attention_of(x, lib_path=lib_path)
    S = (40 + P_tok - 1) // P_tok + 1                # one more than needed: always-empty tail
    po, pl = oracle.partials_of(x, P_tok, S, lib_path=lib_path)
    merged = oracle.merge(po, pl, lib_path=lib_path)
    np.testing.assert_allclose(merged, full, rtol=0, atol=atol)
    assert np.isneginf(pl[..., -1]).all()                  # empty partitions
    assert (po[..., -1, :] == 0).all()


def test_p10_single_partition_is_identity(lib_path=LIB):
    x = make_random(102, B=2, H_q=2, H_kv=1, L=2, D=8, page_size=4, ctx=[6, 13],
                    dtype="f32", causal=True)
    full = oracle.attention_of(x, lib_path=lib_path)
    po, pl = oracle.partials_of(x, 16, 1, lib_path=lib_path)
    assert np.array_equal(po[..., 0, :], full)
    assert np.array_equal(oracle.merge(po, pl, lib_path=lib_path), full)


def test_p10_merge_closed_form_two_halves(lib_path=LIB, atol=1e-15):
    # two partitions with equal lse get equal weight: out = (o1 + o2) / 2
    po = np.array([[[1.0, 2.0], [3.0, -2.0]]])
    pl = np.array([[0.7, 0.7]])
    np.testing.assert_allclose(oracle.merge(po, pl, lib_path=lib_path), [[2.0, 0.0]], atol=atol)
    # lse differing by ln 3: weights 3/4 and 1/4
    pl = np.array([[math.log(3.0), 0.0]])
    np.testing.assert_allclose(oracle.merge(po, pl, lib_path=lib_path), [[1.5, 1.0]], atol=atol)
    # all partitions empty -> zero row
    pl = np.array([[-np.inf, -np.inf]])
    assert (oracle.merge(po, pl, lib_path=lib_path) == 0).all()


# ------------------------------------------------------------------- contract
def test_oracle_validates_contract(lib_path=LIB):
    x = make_c1()
    ok = oracle.attention_of(x, lib_path=lib_path)
    assert np.isfinite(ok).all()
    bt = x.block_table.copy()
    bt[0, 2] = 16                                      # out of the 16-page pool
    with pytest.raises(OracleError) as e:
        oracle.attention(x.query, x.key_pages, x.value_pages, bt, x.context_lens, 4,
                         dtype="f32", causal=True, scale=x.scale, lib_path=lib_path)
    assert e.value.code == 2
    with pytest.raises(OracleError) as e:
        oracle.attention(x.query, x.key_pages, x.value_pages, x.block_table,
                         np.array([13, 7], np.int32), 4, dtype="f32", causal=True,
                         scale=x.scale, lib_path=lib_path)
    assert e.value.code == 3
    with pytest.raises(OracleError) as e:
        oracle.attention(x.query, x.key_pages[:, :3], x.value_pages[:, :3], x.block_table,
                         x.context_lens, 4, dtype="f32", causal=True, scale=x.scale,
                         lib_path=lib_path)
    assert e.value.code == 1
    y = make_random(3, B=1, H_q=1, H_kv=1, L=4, D=8, page_size=4, ctx=[2], dtype="f32",
                    causal=False)
    oracle.attention_of(y, lib_path=lib_path)        # non-causal: L > ctx is allowed
    y.causal = True
    with pytest.raises(OracleError) as e:
        oracle.attention_of(y, lib_path=lib_path)
    assert e.value.code == 4


def test_oracle_c1_request0_uses_worked_pages(lib_path=LIB):
    x = make_c1()
    tr = oracle.translate_of(x, lib_path=lib_path)
    assert tr[0, :10, 0].tolist() == [12] * 4 + [5] * 4 + [3] * 2
    assert x.key_pages[3, :, 2:].min() == 1e4          # tail slots of request 0 hold garbage
