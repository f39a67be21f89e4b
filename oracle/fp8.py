"""OCP e4m3fn decoding (oracle; test infrastructure only).

The pages name the index-cache format only as an fp8 e4m3 dtype
([SGL-37889] "Reproduce": ``--kv-cache-dtype fp8_e4m3``; [ATOM-1473] "Pull
request overview": the index cache is allocated in FP8 when the KV cache is
FP8). The reading used here is the OCP 8-bit floating-point E4M3 encoding,
which is gfx950's native fp8:

* bit layout ``s eeee mmm``, exponent bias 7;
* exponent field 0 encodes subnormals ``(-1)^s * m * 2^-9``;
* otherwise the value is ``(-1)^s * (1 + m/8) * 2^(e-7)``;
* ``S.1111.111`` (0x7F, 0xFF) is NaN;
* there are no infinities; the largest finite magnitude is 448 (0x7E).
"""
from __future__ import annotations

import math

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Closed-form value of one e4m3fn byte (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = (code >> 7) & 1
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = man * 2.0 ** -9
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return -mag if sign else mag


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode an array of e4m3fn bytes to float64, refusing NaN codes.

    The inputs of this path never hold NaN, so a NaN code means the caller
    read memory that it should not have read.
    """
    c = np.asarray(codes, dtype=np.uint8)
    v = E4M3FN_TABLE[c]
    if np.isnan(v).any():
        raise ValueError("e4m3fn NaN code in indexer input")
    return v


# Non-negative finite codes 0x00..0x7E in ascending value order (0x7F is NaN).
_NONNEG = E4M3FN_TABLE[:0x7F]


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest e4m3fn code of each value, ties to the even code, magnitudes
    above 448 saturating to 448, the sign kept (so -0.0 gives 0x80).

    READING: the pages store index keys in an fp8 e4m3 cache ([ATOM-1473],
    Pull request overview) without saying how keys are rounded into it. This
    uses round-to-nearest-even, the IEEE default, and saturation, since the
    format has no infinity. It is written as a search over the value table:
    among adjacent codes exactly one is even, and an even code has a zero
    mantissa LSB, which is what ties-to-even means.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("cannot encode NaN")
    a = np.minimum(np.abs(x), 448.0)
    lo = np.clip(np.searchsorted(_NONNEG, a, side="right") - 1, 0, 0x7E)  # _NONNEG[lo] <= a
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - _NONNEG[lo]
    dhi = _NONNEG[hi] - a
    up = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    code = np.where(up, hi, lo).astype(np.uint8)
    return (code | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)
