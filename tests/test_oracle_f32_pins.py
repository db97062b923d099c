"""Pins of the fp32 build of the CPU oracle (the plain fp32 two-pass
reference that GPU results are held to).

The pins of tests/test_oracle_pins.py run here on the fp32 build.  Pins
whose expected value is exact (address translation, invariances that must
be bit-identical, a single key returning its value, zero rows) keep their
exact comparison; pins against a dense softmax computed in fp64 by numpy get
a tolerance of fp32 rounding, derived below.  A last pin holds the fp32
build within a rounding bound of the fp64 build, computed per row from the
data.

Tolerance: with unit roundoff u = 2^-24, a dot product over D terms is off
by at most about D u sum|q_d k_d|, exp and the normalisation add a few u per
weight, and a sum of n weighted values adds about n u max|v|.  The pins use
D <= 16 and at most 40 keys per row with |values| < 6, so every output lies
within (D + n + 8) u * 6 * (1 + |scale| sum|q k|) < 2e-5 of the exact
result; atol 2e-5 is used, a dropped or misplaced term moves a result by
0.01 or more.
"""
import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins
from workloads import make_c1, make_random

LIB32 = oracle.lib_for("f32")
TOL = 2e-5


def test_f32_build_is_a_distinct_single_precision_library():
    # the fp32 build really computes in single precision: a row whose exact
    # result needs more than 24 bits differs from the fp64 build
    x = make_random(7, B=1, H_q=1, H_kv=1, L=1, D=16, page_size=4, ctx=[30], dtype="f32",
                    causal=True)
    a = oracle.attention_of(x, precision="f32")
    b = oracle.attention_of(x, precision="f64")
    assert not np.array_equal(a, b)
    assert np.abs(a - b).max() < 1e-5
    assert np.array_equal(a, a.astype(np.float32).astype(np.float64))


def test_f32_p1_translation(golden_dir):
    pins.test_p1_translate_tinyllm_block_table_example(golden_dir, lib_path=LIB32)
    pins.test_p1_translate_page_analogy(golden_dir, lib_path=LIB32)
    pins.test_p1_translate_worked_example_placement(golden_dir, lib_path=LIB32)
    pins.test_translate_rejects_bad_ids_but_ignores_padding(lib_path=LIB32)


def test_f32_p3_worked_example(golden_dir):
    pins.test_p3_worked_example_matches_printed_output(golden_dir, lib_path=LIB32)
    pins.test_p3_worked_example_paged_equals_dense(golden_dir, lib_path=LIB32, atol=1e-6)


@pytest.mark.parametrize("seed,ps,H_q,H_kv,L,causal", [
    (10, 1, 2, 1, 1, True), (11, 3, 4, 2, 1, True), (12, 4, 6, 2, 3, True),
    (13, 5, 3, 3, 4, False), (14, 8, 8, 2, 5, True), (15, 2, 1, 1, 2, True)])
def test_f32_p4_brute_force(seed, ps, H_q, H_kv, L, causal):
    pins.test_p4_brute_force_vs_dense_library_softmax(seed, ps, H_q, H_kv, L, causal,
                                                      lib_path=LIB32, atol=TOL)


def test_f32_p4_bf16_widening():
    pins.test_p4_bf16_widening_is_exact(lib_path=LIB32, atol=TOL)


def test_f32_p5_p6_invariances_bit_identical():
    pins.test_p5_physical_relabel_is_bit_identical(lib_path=LIB32)
    for garbage in (1e4, -1e4, 0.0, "random", "nan"):
        pins.test_p6_stale_data_is_ignored_bit_identically(garbage, lib_path=LIB32)


def test_f32_p7_logical_reorder():
    pins.test_p7_logical_reorder(lib_path=LIB32, atol=TOL)


def test_f32_p8_closed_forms():
    pins.test_p8_single_key_returns_its_value(lib_path=LIB32)            # exact
    pins.test_p8_equal_keys_or_zero_query_give_mean_of_values(lib_path=LIB32, atol=TOL)
    pins.test_p8_full_causal_is_lower_triangular_textbook(lib_path=LIB32, atol=TOL)
    pins.test_p8_chunk_rows_equal_last_rows_of_full_causal(lib_path=LIB32)  # bit-identical
    pins.test_p8_gqa_equals_mha_on_repeated_kv(lib_path=LIB32)              # bit-identical
    pins.test_p8_noncausal_rows_see_whole_context_and_qlen_padding_is_zero(lib_path=LIB32,
                                                                          atol=TOL)
    pins.test_p8_empty_context_gives_zeros(lib_path=LIB32)


def test_f32_p9_online_walk():
    pins.test_p9_online_page_walk_equals_two_pass(lib_path=LIB32, rtol=0, atol=TOL)


@pytest.mark.parametrize("P_tok", [4, 8, 12, 64])
def test_f32_p10_split_merge(P_tok):
    pins.test_p10_split_merge_equals_unsplit(P_tok, lib_path=LIB32, atol=TOL)


def test_f32_p10_identity_and_closed_form():
    pins.test_p10_single_partition_is_identity(lib_path=LIB32)
    pins.test_p10_merge_closed_form_two_halves(lib_path=LIB32, atol=1e-7)


def test_f32_contract_checks():
    pins.test_oracle_validates_contract(lib_path=LIB32)
    pins.test_oracle_c1_request0_uses_worked_pages(lib_path=LIB32)


def _row_bound(x):
    """Per-output bound on |fp32 result - exact result|: (D + n + 8) u
    max|v| (1 + scale sum_d |q_d k_d| over the row's keys, at its largest),
    with u = 2^-24 (see the module docstring)."""
    u = 2.0 ** -24
    from workloads import bf16_bits_to_f32
    f = (lambda a: bf16_bits_to_f32(a).astype(np.float64)) if x.dtype == "bf16" else \
        (lambda a: np.asarray(a, np.float64))
    q, kp, vp = f(x.query), f(x.key_pages), f(x.value_pages)
    G = x.H_q // x.H_kv
    bound = np.zeros(x.query.shape)
    for b in range(x.B):
        n = int(x.context_lens[b])
        pages = x.block_table[b]
        K = np.stack([kp[pages[j // x.page_size], :, j % x.page_size] for j in range(n)], 1)
        V = np.stack([vp[pages[j // x.page_size], :, j % x.page_size] for j in range(n)], 1)
        for h in range(x.H_q):
            g = h // G
            dots = x.scale * np.abs(q[b, h]) @ np.abs(K[g]).T      # [L, n]
            bound[b, h] = ((x.D + n + 8) * u * np.abs(V[g]).max()
                           * (1 + dots.max(axis=1)))[:, None]
    return bound


@pytest.mark.parametrize("seed,dtype,L,ctx", [(1, "f32", 1, [10, 7]), (2, "bf16", 3, [40, 97]),
                                              (3, "f32", 2, [300, 5])])
def test_f32_build_within_rounding_bound_of_f64_build(seed, dtype, L, ctx):
    if seed == 1:
        x = make_c1()
    else:
        x = make_random(seed, B=len(ctx), H_q=8, H_kv=2, L=L, D=64, page_size=8, ctx=ctx,
                        dtype=dtype, causal=True)
    a = oracle.attention_of(x, precision="f32")
    b = oracle.attention_of(x, precision="f64")
    assert (np.abs(a - b) <= _row_bound(x)).all()
