"""CPU oracle for the FP8 (E4M3) KV cache: the code table, the quantizer, and dequantized pools.

TEST INFRASTRUCTURE ONLY (like oracle/paged_attention.py): only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the HIP library never does, and the two share no code.

The lfm25-inference page lists FP8 KV storage as the next step after its BF16 KV cache ("Current
Scope and Limitations": KV cache remains BF16; FP8 decode is already used for selected GEMMs,
"Selective E4M3 decode").  The format here is the 8-bit E4M3 floating-point format of the open FP8
specification, as MI355X handles it natively:
  bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m
  e = 0      subnormal   (m / 8) * 2^-6
  e = 1..15  normal      (1 + m / 8) * 2^(e - 7), except e = 15, m = 7, which is NaN
  no infinities; the largest finite magnitude is (1 + 6/8) * 2^8 = 448.
A cache element is a code c; the value it stands for is decode(c) * scale, with one scale for the
K pool and one for the V pool.

Quantization (the write path): x / scale rounded to float32, then the nearest code, ties to the even
code (the code whose mantissa is even: E4M3 codes of one sign are ordered like their magnitudes, so
that is the even integer); magnitudes beyond 448 saturate to 448; NaN goes to the NaN code of its
sign.  The saturating, ties-to-even rule is a reading: the pages fix no rounding.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# magnitudes of the 127 finite non-negative codes 0x00..0x7E, increasing with the code
_MAGS = decode(np.arange(0x7F, dtype=np.uint8))


def encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (float array), ties to even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))
    hi = np.searchsorted(_MAGS, a, side="left")          # first code with magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _MAGS[hi] - a
    d_lo = a - _MAGS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo & (lo < hi), lo, hi).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def dequantize(codes, scale: float) -> np.ndarray:
    """The values a pool of codes stands for: decode(c) * scale, float64."""
    return decode(codes) * float(scale)


def quantize(x, scale: float) -> np.ndarray:
    """Codes for values x (float32, or bf16 widened to float32) under `scale`: encode(x / scale), the
    division rounded to float32 as the kernel does it (the code is an integer decided by floating
    point, so both sides decide it in the same precision)."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return encode(q.astype(np.float64))
