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


# ---------------------------------------------------------------------------
# Encoding (the key-cache writer's rounding)
# ---------------------------------------------------------------------------

from oracle.fp8 import encode_e4m3fn  # noqa: E402
from oracle.indexer import cache_write, quantize_key  # noqa: E402

FINITE = [c for c in range(256) if not np.isnan(E4M3FN_TABLE[c])]


def test_encode_round_trips_every_finite_code():
    vals = E4M3FN_TABLE[FINITE]
    assert np.array_equal(encode_e4m3fn(vals), np.array(FINITE, np.uint8))


def test_encode_is_nearest_by_brute_force():
    """Against an exhaustive search over all finite codes: the chosen value is
    never farther from x than any other code's value, and on exact ties the
    code with the even mantissa is chosen."""
    g = np.random.default_rng(5)
    x = np.concatenate([g.uniform(-460, 460, 3000), g.standard_normal(3000) * 2.0 ** g.integers(-12, 8, 3000)])
    vals = E4M3FN_TABLE[FINITE]
    codes = encode_e4m3fn(x)
    for xi, c in zip(x, codes):
        a = min(abs(xi), 448.0)
        d = np.abs(np.abs(vals) - a)
        got = abs(E4M3FN_TABLE[c])
        assert abs(got - a) <= d.min()
        assert (c >> 7) == int(np.signbit(xi))


def test_encode_ties_go_to_even_mantissa():
    pos = E4M3FN_TABLE[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2.0
    codes = encode_e4m3fn(mid)
    lo = np.arange(0x7E)
    assert np.array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))


def test_encode_saturates_and_keeps_sign():
    assert list(encode_e4m3fn([448.0, 449.0, 463.9, 464.0, 1e30, np.inf])) == [0x7E] * 6
    assert list(encode_e4m3fn([-449.0, -np.inf])) == [0xFE] * 2
    assert list(encode_e4m3fn([0.0, -0.0])) == [0x00, 0x80]


def test_encode_matches_torch_cast_in_range():
    """Library special case: torch's float32 -> float8_e4m3fn cast (round to
    nearest even) on random values and on every midpoint between codes."""
    g = np.random.default_rng(6)
    pos = E4M3FN_TABLE[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2.0
    x = np.concatenate([g.uniform(-448, 448, 20000), g.standard_normal(20000) * 0.01, mid, -mid]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3fn(x), ref)


def test_quantize_key_properties():
    g = np.random.default_rng(7)
    k = g.standard_normal(128).astype(np.float32)
    codes, scale = quantize_key(k)
    j = int(np.argmax(np.abs(k)))
    assert codes[j] & 0x7F == 0x7E                 # the largest magnitude maps to 448
    assert scale == np.float32(np.float32(np.abs(k).max()) / np.float32(448.0))
    for p in (-20, -3, 5):                          # exact power-of-two rescaling
        c2, s2 = quantize_key((k * np.float32(2.0 ** p)).astype(np.float32))
        assert np.array_equal(c2, codes) and s2 == np.float32(scale * np.float32(2.0 ** p))
    c0, s0 = quantize_key(np.zeros(128, np.float32))
    assert s0 == 1.0 and not c0.any()
    # decoding reproduces the key to e4m3 precision
    back = E4M3FN_TABLE[codes] * float(scale)
    assert np.all(np.abs(back - k) <= np.abs(k) * 2.0 ** -4 + float(scale) * 2.0 ** -10)


def test_quantize_key_reproduces_the_generated_cache():
    """The input generator builds its cache with torch's cast (after a clamp);
    the oracle's writer, from its own encoder, gives the same bytes and
    scales for the same fp32 keys."""
    import workloads
    from workloads.synth import STREAM_KEY, rng

    case = workloads.indexer_case(41, batch=3, n_lo=1, n_hi=300, page_size=16, k=8, heads=16)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        kf = rng(41, STREAM_KEY, b).standard_normal((n, case.dim), dtype=np.float32)
        pages = case.block_table[b]
        for j in range(n):
            slot = int(pages[j // 16]) * 16 + j % 16
            codes, scale = quantize_key(kf[j])
            assert np.array_equal(codes, case.kcache[slot]) and scale == case.k_scale[slot]


def test_cache_write_scatters_and_skips_negative_slots():
    g = np.random.default_rng(8)
    keys = g.standard_normal((5, 128)).astype(np.float32)
    kc = np.full((10, 128), 0xAA, np.uint8)
    ks = np.full(10, -1.0, np.float32)
    cache_write(keys, np.array([3, -1, 7, 0, -5], np.int32), kc, ks)
    for t, s in ((0, 3), (2, 7), (3, 0)):
        codes, scale = quantize_key(keys[t])
        assert np.array_equal(kc[s], codes) and ks[s] == scale
    untouched = [i for i in range(10) if i not in (0, 3, 7)]
    assert (kc[untouched] == 0xAA).all() and (ks[untouched] == -1.0).all()
