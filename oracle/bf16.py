"""bfloat16 decoding and encoding (oracle; test infrastructure only).

The pages let the index cache follow the KV cache's dtype: fp8 when the KV
cache is fp8, the model's own dtype otherwise ([ATOM-1473] "Pull request
overview": the index cache dtype; commit "convert auto for bf16 type"). The
non-fp8 case read here is bfloat16, stored as its 16-bit patterns:

* bit layout ``s eeeeeeee fffffff``: the upper half of an IEEE binary32;
* exponent bias 127; exponent field 0 encodes subnormals
  ``(-1)^s * (f / 128) * 2^-126``;
* otherwise the value is ``(-1)^s * (1 + f / 128) * 2^(e - 127)``;
* exponent field 255 holds infinities (f = 0) and NaNs (f != 0).
"""
from __future__ import annotations

import math

import numpy as np


def bf16_value(bits: int) -> float:
    """Closed-form value of one bf16 bit pattern."""
    bits = int(bits) & 0xFFFF
    sign = -1.0 if (bits >> 15) & 1 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * (frac / 128.0) * 2.0 ** -126
    return sign * (1.0 + frac / 128.0) * 2.0 ** (exp - 127)


# all 65536 patterns, decoded once from the closed form
BF16_TABLE = np.array([bf16_value(b) for b in range(1 << 16)], dtype=np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """float64 values of an array of bf16 bit patterns (exact)."""
    return BF16_TABLE[np.asarray(bits, dtype=np.uint16).astype(np.int64)]


def encode_bf16(x) -> np.ndarray:
    """bf16 patterns nearest to the float64 values x, ties to the even
    fraction (IEEE round to nearest even).

    Plain search: the candidates are the two finite bf16 values that bracket
    |x| (found by bisection in the table of non-negative finite patterns,
    which the closed form makes increasing); the nearer one wins, an exact
    tie goes to the one whose fraction is even. Magnitudes at or beyond the
    midpoint between the largest finite value and 2^128 round to infinity,
    as IEEE rounding does. NaN is outside the domain and raises.
    """
    v = np.asarray(x, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no bf16 encoding here")
    pos = BF16_TABLE[:0x7F81]  # +0 .. +inf, increasing
    mag = np.abs(v).reshape(-1)
    hi = np.searchsorted(pos, mag, side="left")  # first pattern >= |x|
    out = np.empty(mag.shape, dtype=np.int64)
    for i, (m, h) in enumerate(zip(mag, hi)):
        if h < len(pos) and pos[h] == m:
            out[i] = h
            continue
        lo = h - 1
        if h >= 0x7F80:  # beyond the largest finite value (0x7F7F)
            top = pos[0x7F7F]
            mid = top + (2.0 ** 128 - top) / 2
            out[i] = 0x7F80 if m >= mid else 0x7F7F
            continue
        dl, dh = m - pos[lo], pos[h] - m
        if dl < dh:
            out[i] = lo
        elif dh < dl:
            out[i] = h
        else:
            out[i] = lo if lo % 2 == 0 else h
    sign = (np.signbit(v.reshape(-1))).astype(np.int64) << 15
    return (out | sign).astype(np.uint16).reshape(v.shape)
