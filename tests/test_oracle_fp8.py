"""Pins for the oracle's e4m3fn decoding (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle.fp8 import E4M3FN_TABLE, decode_e4m3fn


# Spot values fixed by the OCP 8-bit floating point specification (E4M3 table:
# max normal S.1111.110 = 448, min normal S.0001.000 = 2^-6, max subnormal
# S.0000.111 = 0.875 * 2^-6, min subnormal S.0000.001 = 2^-9, NaN S.1111.111).
SPOT = {
    0x00: 0.0,
    0x01: 2.0 ** -9,
    0x07: 0.875 * 2.0 ** -6,
    0x08: 2.0 ** -6,
    0x38: 1.0,
    0x39: 1.125,
    0x40: 2.0,
    0x7E: 448.0,
    0xB8: -1.0,
    0xFE: -448.0,
    0x81: -(2.0 ** -9),
}


@pytest.mark.parametrize("code,val", sorted(SPOT.items()))
def test_spot_values(code, val):
    assert E4M3FN_TABLE[code] == val


def test_nan_codes_and_signed_zero():
    assert math.isnan(E4M3FN_TABLE[0x7F]) and math.isnan(E4M3FN_TABLE[0xFF])
    assert E4M3FN_TABLE[0x80] == 0.0 and math.copysign(1.0, E4M3FN_TABLE[0x80]) == -1.0
    assert np.isnan(E4M3FN_TABLE).sum() == 2


def test_matches_torch_float8_e4m3fn_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = E4M3FN_TABLE
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~both_nan], ours[~both_nan])
    # signs of zero agree too
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


def test_monotone_and_symmetric():
    pos = E4M3FN_TABLE[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(E4M3FN_TABLE[0x80:0xFF], -pos)


def test_decode_refuses_nan():
    with pytest.raises(ValueError):
        decode_e4m3fn(np.array([0x38, 0x7F], np.uint8))
    assert decode_e4m3fn(np.array([0x38, 0x40], np.uint8)).tolist() == [1.0, 2.0]
