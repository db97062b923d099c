"""8-bit float codes of fp8 K/V pages -- TEST INFRASTRUCTURE ONLY.

"Reading vLLM's PagedAttention Kernel", section 3.2: the cache write takes a
kv-cache dtype and per-tensor k/v scales, so an fp8 cache stores each element
as an 8-bit code together with one scale per pool.  The reading taken for
the fp8 variant is the OCP 8-bit floating-point format with 4 exponent and 3
mantissa bits (E4M3), the fp8 format of MI355X's matrix cores:

  bit 7 sign s, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m;
  e >= 1:  (-1)^s (1 + m/8) 2^(e-7)      (normal)
  e == 0:  (-1)^s (m/8) 2^-6              (subnormal, zero when m = 0)
  s.1111.111 is NaN; there is no infinity; the largest magnitude is 448.

Storing: a value x of a token row becomes the code nearest to x / scale
(the division done in fp32), ties going to the code whose mantissa is even;
magnitudes beyond 448 saturate to 448, and NaN stays NaN.  Reading: the
code's value times the scale.  Both directions are written here from that
definition (a table of the 127 non-negative finite values and a nearest
search), not from any conversion routine.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def _nonneg_table() -> np.ndarray:
    """Values of codes 0x00 .. 0x7E (all non-negative finite codes), which
    increase with the code."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


TABLE = _nonneg_table()


def decode(codes) -> np.ndarray:
    """Values (float64) of uint8 codes."""
    c = np.asarray(codes, dtype=np.uint8)
    mag_code = c & np.uint8(0x7F)
    out = TABLE[np.minimum(mag_code, 0x7E)].copy()
    out[mag_code == NAN_CODE] = np.nan
    neg = (c & np.uint8(0x80)) != 0
    out[neg] = -out[neg]
    return out


def encode(x) -> np.ndarray:
    """Codes (uint8) of float32 values: nearest code value, ties to the even
    code, saturating at 448, NaN to the NaN code (sign kept throughout)."""
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(v), MAX_FINITE)
    a = np.where(np.isnan(v), 0.0, a)
    hi = np.clip(np.searchsorted(TABLE, a, side="left"), 0, len(TABLE) - 1)
    lo = np.clip(hi - 1, 0, len(TABLE) - 1)
    d_lo = a - TABLE[lo]
    d_hi = TABLE[hi] - a
    pick = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(d_hi == 0, hi, pick)
    code = pick.astype(np.uint8)
    code = np.where(np.isnan(v), np.uint8(NAN_CODE), code)
    sign = np.signbit(v)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(rows_f32: np.ndarray, scale: float) -> np.ndarray:
    """Codes of float32 rows stored under `scale`: encode(rows / scale) with
    the division in fp32."""
    r = np.asarray(rows_f32, dtype=np.float32)
    return encode(r / np.float32(scale))
