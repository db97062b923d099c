"""Pins of the fp8 (E4M3) page handling of the oracles: the C oracle's code
decoder and its attention over fp8 pages, and the write side's encoder
(oracle/fp8.py).  Expected codes and values are derived by hand from the
format's definition (sign, 4 exponent bits with bias 7, 3 mantissa bits;
exponent 0 subnormal; s.1111.111 NaN; no infinity), or come from closed
forms and from dense attention on the decoded values computed in numpy."""
import math

import numpy as np
import pytest

import oracle
from oracle import fp8
from tests._dense import dense_attention_rows
from workloads import make_random

LIB = oracle._LIB

# (code, value) derived by hand from the definition
HAND = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x02, 2.0 ** -8), (0x03, 3 * 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x09, 1.125 * 2.0 ** -6),
    (0x0F, 1.875 * 2.0 ** -6), (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3C, 1.5),
    (0x3F, 1.875), (0x40, 2.0), (0x47, 3.75), (0x78, 256.0), (0x7E, 448.0),
    (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xC0, -2.0), (0xFE, -448.0),
]


def test_fp8_decoder_hand_derived_codes(lib_path=LIB):
    codes = np.array([c for c, _ in HAND], np.uint8)
    want = np.array([v for _, v in HAND])
    for got in (oracle.e4m3_values(codes, lib_path=lib_path), fp8.decode(codes)):
        assert np.array_equal(got, want)
    nan = oracle.e4m3_values(np.array([0x7F, 0xFF], np.uint8), lib_path=lib_path)
    assert np.isnan(nan).all()
    z = oracle.e4m3_values(np.array([0x80], np.uint8), lib_path=lib_path)
    assert z[0] == 0.0 and math.copysign(1.0, z[0]) == -1.0


def test_fp8_every_finite_code_increasing_and_symmetric(lib_path=LIB):
    pos = oracle.e4m3_values(np.arange(0x7F, dtype=np.uint8), lib_path=lib_path)
    neg = oracle.e4m3_values(np.arange(0x80, 0xFF, dtype=np.uint8), lib_path=lib_path)
    assert (np.diff(pos) > 0).all() and pos[-1] == 448.0
    assert np.array_equal(neg, -pos)
    # spacing doubles with each exponent: 2^-9 below 2^-5, 2^(e-10) in binade e
    assert np.allclose(np.diff(pos[:16]), 2.0 ** -9)


def test_fp8_encoder_hand_derived_roundings():
    cases = [
        (1.0, 0x38), (1.0625, 0x38),          # halfway 1 / 1.125: even mantissa 0
        (1.1875, 0x3A),                       # halfway 1.125 / 1.25: even mantissa 2
        (1.06, 0x38), (1.07, 0x39),
        (2.0 ** -10, 0x00),                   # halfway 0 / 2^-9: even code 0
        (3 * 2.0 ** -10, 0x02),               # halfway 2^-9 / 2^-8: even code 2
        (5 * 2.0 ** -10, 0x02),               # halfway 2^-8 / 3*2^-9: even code 2
        (2.0 ** -6, 0x08), (15 * 2.0 ** -10, 0x08),   # 7.5 * 2^-9: up to 2^-6
        (448.0, 0x7E), (460.0, 0x7E), (1e4, 0x7E), (np.inf, 0x7E),   # saturation
        (-1e4, 0xFE), (-np.inf, 0xFE), (-0.0, 0x80), (-1e-30, 0x80), (0.0, 0x00),
        (np.nan, 0x7F), (-3.75, 0xC7),
    ]
    got = fp8.encode(np.array([v for v, _ in cases], np.float32))
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_fp8_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes).astype(np.float32)), codes)


def test_fp8_quantize_rows_divides_in_fp32():
    # 0.3 / 0.1 in fp32 is 3.0000002 (not 3): the code of that, not of 3
    x = np.array([0.3], np.float32)
    q = np.float32(0.3) / np.float32(0.1)
    assert fp8.quantize_rows(x, 0.1)[0] == fp8.encode(np.array([q], np.float32))[0]
    # error bound: half a spacing, i.e. <= 2^-4 relative in the normal range
    r = np.random.default_rng(5).standard_normal(4096).astype(np.float32)
    back = fp8.decode(fp8.quantize_rows(r, 0.25)) * 0.25
    big = np.abs(r / 0.25) >= 2.0 ** -6
    assert (np.abs(back - r)[big] <= 2.0 ** -4 * np.abs(r)[big] + 1e-12).all()


def _fp8_inputs(seed, **kw):
    return make_random(seed, kv_dtype="fp8_e4m3", **kw)


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.5, 0.25)])
def test_fp8_pages_equal_bf16_pages_holding_the_values(scales, lib_path=LIB):
    """With power-of-two scales every dequantised element is a bf16 value,
    so fp8 pages must give the bits that bf16 pages holding those values give."""
    from workloads import f32_to_bf16_bits
    x = _fp8_inputs(41, B=3, H_q=8, H_kv=2, L=2, D=16, page_size=4, ctx=[5, 13, 30],
                    dtype="bf16", causal=True, kv_scales=scales, extra_free_pages=3)
    a = oracle.attention_of(x, lib_path=lib_path)
    kv = [f32_to_bf16_bits((fp8.decode(p) * s).astype(np.float32))
          for p, s in ((x.key_pages, scales[0]), (x.value_pages, scales[1]))]
    b = oracle.attention(x.query, kv[0], kv[1], x.block_table, x.context_lens, x.page_size,
                         dtype="bf16", causal=True, scale=x.scale, lib_path=lib_path)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", [3, 4])
def test_fp8_pages_brute_force_vs_dense(seed, lib_path=LIB):
    """Random codes and non-power-of-two scales against dense softmax
    attention on the dequantised rows, computed in numpy in fp64."""
    from workloads import bf16_bits_to_f32
    x = _fp8_inputs(seed, B=2, H_q=4, H_kv=2, L=1, D=16, page_size=8, ctx=[9, 37],
                    dtype="bf16", causal=True, kv_scales=(0.37, 1.7), extra_free_pages=2)
    out = oracle.attention_of(x, lib_path=lib_path)
    q = bf16_bits_to_f32(x.query).astype(np.float64)
    kd = fp8.decode(x.key_pages) * x.k_scale
    vd = fp8.decode(x.value_pages) * x.v_scale
    for b in range(2):
        n = int(x.context_lens[b])
        K = np.stack([kd[x.block_table[b, j // 8], :, j % 8] for j in range(n)], 1)
        V = np.stack([vd[x.block_table[b, j // 8], :, j % 8] for j in range(n)], 1)
        for h in range(4):
            ref = dense_attention_rows(q[b, h], K[h // 2], V[h // 2], x.scale, [n])
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("garbage", ["nan", "random", -1e4])
def test_fp8_stale_codes_are_ignored_bit_identically(garbage, lib_path=LIB):
    kw = dict(B=3, H_q=4, H_kv=2, L=2, D=16, page_size=4, ctx=[5, 8, 11], dtype="bf16",
              causal=True, extra_free_pages=4)
    a = oracle.attention_of(_fp8_inputs(42, **kw), lib_path=lib_path)
    b = oracle.attention_of(_fp8_inputs(42, garbage=garbage, **kw), lib_path=lib_path)
    assert np.array_equal(a, b) and np.isfinite(b).all()


def test_fp8_pins_hold_on_the_fp32_build():
    lib32 = oracle.lib_for("f32")
    test_fp8_decoder_hand_derived_codes(lib_path=lib32)
    test_fp8_every_finite_code_increasing_and_symmetric(lib_path=lib32)
    for s in ((1.0, 1.0), (0.5, 0.25)):
        test_fp8_pages_equal_bf16_pages_holding_the_values(s, lib_path=lib32)
    test_fp8_stale_codes_are_ignored_bit_identically("nan", lib_path=lib32)


def test_fp8_scatter_writes_hand_derived_codes_and_nothing_else():
    """The write side with an fp8 pool: planted rows whose quotients by the
    scale are exact values, ties, overflows and NaN land as the hand-derived
    codes; every other byte of the pool is untouched; a negative slot skips
    its token."""
    from oracle.scatter import scatter_tokens_fp8
    from workloads import f32_to_bf16_bits
    P, H, ps, D = 3, 2, 4, 4
    kp = np.full((P, H, ps, D), 0xAB, np.uint8)
    vp = np.full((P, H, ps, D), 0xCD, np.uint8)
    ks, vs = 0.5, 2.0
    # key / ks and value / vs per element (all exact in bf16 and in fp32)
    kq = np.array([[[1.0, 1.0625, 1.1875, -3.75], [2.0 ** -10, 3 * 2.0 ** -10, 448.0, 1e4]],
                   [[0.0, -0.0, 0.5, 256.0], [-1e4, 15 * 2.0 ** -10, 1.125, -1.0]]], np.float32)
    kcodes = [[[0x38, 0x38, 0x3A, 0xC7], [0x00, 0x02, 0x7E, 0x7E]],
              [[0x00, 0x80, 0x30, 0x78], [0xFE, 0x08, 0x39, 0xB8]]]
    key = f32_to_bf16_bits(kq * np.float32(ks))
    value = f32_to_bf16_bits(np.full((2, H, D), 3.0, np.float32) * np.float32(vs))
    value[1, 0, 2] = 0x7FC0                      # a bf16 NaN -> NaN code
    slots = [1 * ps + 2, 2 * ps + 0]             # page 1 slot 2, page 2 slot 0
    k2, v2 = scatter_tokens_fp8(kp, vp, key, value, slots, ks, vs)
    assert k2[1, :, 2].tolist() == kcodes[0] and k2[2, :, 0].tolist() == kcodes[1]
    assert (v2[1, :, 2] == 0x44).all()           # 3.0 = 1.5 * 2^1: e 8, m 4
    assert v2[2, 0, 0].tolist() == [0x44, 0x44, 0x7F, 0x44] and (v2[2, 1, 0] == 0x44).all()
    touched = np.zeros((P, H, ps, D), bool)
    touched[1, :, 2] = touched[2, :, 0] = True
    assert (k2[~touched] == 0xAB).all() and (v2[~touched] == 0xCD).all()
    k3, _ = scatter_tokens_fp8(kp, vp, key, value, [-1, 2 * ps + 0], ks, vs)
    assert (k3[1] == 0xAB).all() and k3[2, :, 0].tolist() == kcodes[1]
