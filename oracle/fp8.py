"""The 8-bit E4M3 floating-point format of an FP8 KV cache, in float64.

TEST INFRASTRUCTURE (see the package docstring).

The pages give FP8 only as a 1-byte element ([Optimizing] §The Math of the
KV Cache Bottleneck: bytes per element are 1 for FP8) and name FP8 among the
quantization formats becoming standard (§Conclusion).  The format read here
is E4M3 as the 8-bit floating-point standard of the OCP defines it: one
sign bit, a 4-bit exponent with bias 7 and a 3-bit mantissa; exponent field
0 holds the subnormals m/8 * 2^-6; there are no infinities; S.1111.111 is
NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.

A stored K (V) code c stands for decode(c) * k_scale (v_scale), one scale
per layer; a value x is stored as encode(x * (1 / scale)) with the product
and the reciprocal taken in float32, rounding to the nearest code (ties to
the even mantissa) and saturating at +-448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even mantissa),
    saturating at +-448; NaN gives the NaN code 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    a = np.abs(x)
    finite = np.isfinite(a)
    a = np.where(finite, a, 0.0)
    # binade of a (floor(log2 a) exactly, via frexp), never below the subnormal range
    _, E = np.frexp(a)
    e = np.maximum(E - 1, -6)
    e = np.where(a == 0, -6, e)
    quantum = np.ldexp(1.0, e - 3)          # spacing of codes in that binade
    m = np.rint(a / quantum)                 # quanta, ties to even
    carry = m >= 16                          # rounded up into the next binade
    e = np.where(carry, e + 1, e)
    m = np.where(carry, m / 2, m)
    value = m * np.ldexp(1.0, e - 3)
    normal = m >= 8
    code = np.where(normal, ((e + 7) << 3) | (m.astype(np.int64) - 8), m.astype(np.int64))
    code = np.where((value > E4M3_MAX) | np.isinf(x), 0x7E, code)
    code = np.where(np.isnan(x), E4M3_NAN, code | sign)
    return code.astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Codes of the values x (float32, or bf16 bit patterns as uint16) stored
    with scale: encode(x * (1 / scale)), reciprocal and product in float32."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):  # past float32's range: inf, saturates; NaN stays NaN
        y = (x.astype(np.float32) * inv).astype(np.float32)
    return e4m3_encode(y)
