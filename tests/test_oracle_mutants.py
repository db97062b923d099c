"""Planted mistakes: each mutant is a plausible bug written into a copy of the
oracle's C source, built on the CPU; the pins must reject every one of them.
This shows the pins constrain every step of the oracle (translation, gather,
scores, softmax, GQA mapping, causal alignment, partitions, merge, widening).
"""
import os

import pytest

import oracle
from tests import test_oracle_fp8 as fp8
from tests import test_oracle_pins as pins

MUTANTS = {
    "slot_off_by_one": ("*slot = j - lp * a->page_size;",
                        "*slot = (j + 1) % a->page_size;"),
    "wrong_logical_page": ("*page = a->bt[(size_t)b * a->max_pages + lp];",
                           "*page = a->bt[(size_t)b * a->max_pages + (lp > 0 ? lp - 1 : 0)];"),
    "kv_head_ignored": ("size_t base = (((size_t)page * a->Hkv + g) * a->page_size + slot) * (size_t)D;",
                        "size_t base = (((size_t)page * a->Hkv + 0) * a->page_size + slot) * (size_t)D;"),
    "value_read_from_keys": ("Vd[(size_t)j * D + d] = page_value(a, a->vp, base + d, a->v_scale);",
                             "Vd[(size_t)j * D + d] = page_value(a, a->kp, base + d, a->v_scale);"),
    "fp8_bias_off_by_one": ("(real)ldexp((double)(8 + m), e - 10)",
                            "(real)ldexp((double)(8 + m), e - 9)"),
    "fp8_subnormal_as_normal": ("e == 0 ? (real)ldexp((double)m, -9)",
                                "e == 0 ? (real)ldexp((double)(8 + m), -10)"),
    "fp8_nan_as_number": ("if (e == 15 && m == 7) return (real)NAN;", ""),
    "fp8_value_scale_swapped": ("Vd[(size_t)j * D + d] = page_value(a, a->vp, base + d, a->v_scale);",
                                "Vd[(size_t)j * D + d] = page_value(a, a->vp, base + d, a->k_scale);"),
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "dot_misaligned": ("acc += q[d] * Kd[(size_t)j * D + d];",
                       "acc += q[(d + 1) % D] * Kd[(size_t)j * D + d];"),
    "exp_sign_flipped": ("real w = R_EXP(s[j] - m);", "real w = R_EXP(m - s[j]);"),
    "not_normalised": ("for (int d = 0; d < D; ++d) o[d] /= Z;",
                       "for (int d = 0; d < D; ++d) o[d] /= 1.0;"),
    "gqa_strided_groups": ("const int h = g * G + hh;", "const int h = hh * a->Hkv + g;"),
    "causal_top_left": ("return ctx - qlen_of(a, b) + i + 1;", "return i + 1;"),
    "causal_off_by_one": ("return ctx - qlen_of(a, b) + i + 1;",
                          "return ctx - qlen_of(a, b) + i;"),
    "query_lens_ignored": ("static int qlen_of(const or_args *a, int b) { return a->ql ? a->ql[b] : a->L; }",
                           "static int qlen_of(const or_args *a, int b) { return a->L; }"),
    "partitions_overlap": ("int lo = sp * P, e = lo + P;", "int lo = sp * P, e = lo + P + 1;"),
    "lse_missing_log_sum": ("return m + R_LOG(Z);", "return m;"),
    "merge_unweighted": ("Z += R_EXP((real)part_lse[r * S + s] - M);", "Z += 1;"),
    "bf16_widen_shift": ("<< 16;", "<< 15;"),
    "trace_past_context": ("if ((int)j < cl[b]) {", "if ((int)j <= cl[b]) {"),
}

BATTERY = [
    ("p1_tinyllm", lambda lib, gd: pins.test_p1_translate_tinyllm_block_table_example(gd, lib_path=lib)),
    ("p1_placement", lambda lib, gd: pins.test_p1_translate_worked_example_placement(gd, lib_path=lib)),
    ("p3_printed", lambda lib, gd: pins.test_p3_worked_example_matches_printed_output(gd, lib_path=lib)),
    ("p4_brute", lambda lib, gd: pins.test_p4_brute_force_vs_dense_library_softmax(12, 4, 6, 2, 3, True, lib_path=lib)),
    ("p4_brute_noncausal", lambda lib, gd: pins.test_p4_brute_force_vs_dense_library_softmax(13, 5, 3, 3, 4, False, lib_path=lib)),
    ("p4_bf16", lambda lib, gd: pins.test_p4_bf16_widening_is_exact(lib_path=lib)),
    ("p8_lower_tri", lambda lib, gd: pins.test_p8_full_causal_is_lower_triangular_textbook(lib_path=lib)),
    ("p8_qlen", lambda lib, gd: pins.test_p8_noncausal_rows_see_whole_context_and_qlen_padding_is_zero(lib_path=lib)),
    ("p10_split", lambda lib, gd: pins.test_p10_split_merge_equals_unsplit(12, lib_path=lib)),
    ("fp8_codes", lambda lib, gd: fp8.test_fp8_decoder_hand_derived_codes(lib_path=lib)),
    ("fp8_dense", lambda lib, gd: fp8.test_fp8_pages_brute_force_vs_dense(3, lib_path=lib)),
]


def _build_mutant(tmp_path, old, new):
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return oracle.compile_library(src=path, out=os.path.join(tmp_path, "libmutant.so"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path, golden_dir):
    old, new = MUTANTS[name]
    lib = _build_mutant(str(tmp_path), old, new)
    caught = []
    for pin, run in BATTERY:
        try:
            run(lib, golden_dir)
        except Exception:                      # assertion or oracle error: pin fired
            caught.append(pin)
    assert caught, f"no pin rejects mutant {name}"
