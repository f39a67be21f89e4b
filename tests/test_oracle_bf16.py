"""Pins for the oracle's bf16 format and bf16-cache scoring (CPU only)."""
import numpy as np
import pytest

import workloads
from oracle.bf16 import BF16_TABLE, bf16_value, decode_bf16, encode_bf16
from oracle.indexer import cache_write_bf16, index_scores, index_scores_bf16


def _torch():
    return pytest.importorskip("torch")


def test_closed_forms():
    assert bf16_value(0x3F80) == 1.0
    assert bf16_value(0xC000) == -2.0
    assert bf16_value(0x3F00) == 0.5
    assert bf16_value(0x0000) == 0.0 and np.signbit(bf16_value(0x8000))
    assert bf16_value(0x0001) == 2.0 ** -133          # smallest subnormal
    assert bf16_value(0x0080) == 2.0 ** -126          # smallest normal
    assert bf16_value(0x7F7F) == (2 - 2.0 ** -7) * 2.0 ** 127
    assert bf16_value(0x7F80) == np.inf and bf16_value(0xFF80) == -np.inf
    assert np.isnan(bf16_value(0x7FC0))


def test_decode_matches_library_cast():
    """Library special case: torch reinterprets the 16-bit patterns as
    bfloat16 and widens them; every non-NaN pattern decodes the same."""
    torch = _torch()
    bits = np.arange(1 << 16, dtype=np.int64)
    lib = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = decode_bf16(bits)
    keep = ~np.isnan(lib)
    assert np.array_equal(np.isnan(ours), ~keep)
    assert np.array_equal(ours[keep], lib[keep])


def test_encode_matches_library_rounding():
    """torch's float32 -> bfloat16 conversion rounds to nearest even; on
    random float32 values, exact ties and values past the largest finite
    one, the oracle's search picks the same patterns."""
    torch = _torch()
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (g.standard_normal(2000) * 1e-38).astype(np.float32),          # subnormal range
        # exact ties: a bf16 value plus half its last place
        (decode_bf16(g.integers(0x0080, 0x7F00, 2000)) * (1 + 2.0 ** -8)).astype(np.float32),
        np.array([3.4e38, -3.4e38, 3.3895e38, 0.0, -0.0], np.float32),
    ])
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(encode_bf16(x.astype(np.float64)), lib)


def test_encode_decode_round_trip():
    """Every finite pattern encodes back to itself (the table is increasing
    on the non-negative patterns, which the search relies on)."""
    pos = BF16_TABLE[:0x7F81]
    assert np.all(np.diff(pos) > 0)
    bits = np.array([b for b in range(1 << 16) if np.isfinite(BF16_TABLE[b])], dtype=np.int64)
    assert np.array_equal(encode_bf16(decode_bf16(bits)).astype(np.int64), bits)


def test_encode_refuses_nan():
    with pytest.raises(ValueError):
        encode_bf16([1.0, np.nan])


# values exact in both formats: 0, +-0.5, +-1, +-2
_E4M3 = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)
_BF16 = np.array([0x0000, 0x3F00, 0x3F80, 0x4000, 0xBF00, 0xBF80, 0xC000], np.uint16)


@pytest.mark.parametrize("seed", range(6))
def test_scores_equal_fp8_scores_on_shared_values(seed):
    """Cross-pin: on inputs exact in both e4m3 and bf16 with unit scales,
    the bf16 scorer equals the fp8 one (pinned on its own), key by key."""
    g = np.random.default_rng(seed)
    H, D, P, n = 16, 128, 16, int(g.integers(1, 100))
    qi = g.integers(0, 7, size=(H, D))
    ki = g.integers(0, 7, size=(128, D))
    w = g.choice(np.array([0.5, 1.0, -1.0, 2.0], np.float32), size=H)
    bt = g.permutation(8).astype(np.int32)
    s8 = index_scores(_E4M3[qi], 1.0, w, _E4M3[ki], np.ones(128, np.float32), bt, P, n)
    s16 = index_scores_bf16(_BF16[qi], w, _BF16[ki], bt, P, n)
    assert np.array_equal(s8, s16)


def test_score_closed_form():
    """One head, weight 1, each key a multiple c_j of the query: S_j =
    max(0, c_j) * |q|^2."""
    g = np.random.default_rng(3)
    q = g.integers(-3, 4, size=128).astype(np.float64) / 4
    c = np.array([1.0, -1.0, 0.5, 0.0, 2.0])
    keys = c[:, None] * q[None, :]
    S = index_scores_bf16(encode_bf16(q)[None, :], np.ones(1, np.float32), encode_bf16(keys),
                          np.arange(5, dtype=np.int32), 1, 5)
    assert np.array_equal(S, np.maximum(c, 0.0) * float(q @ q))


def test_case_generator_bf16_values():
    """Generated bf16 cases: keys are the upper halves of the float32 draws,
    unused slots hold the sentinel, and the scorer reads them."""
    c = workloads.indexer_case(9, batch=2, n_lo=5, n_hi=40, page_size=16, k=8, heads=16, cache_dtype="bf16")
    assert c.q.dtype == np.uint16 and c.kcache.dtype == np.uint16
    assert (c.kcache[-1] == workloads.SENTINEL_KEY_BF16).all()
    assert decode_bf16(workloads.SENTINEL_KEY_BF16) == 2.0 ** 23


def test_cache_write_bf16_matches_library():
    torch = _torch()
    g = np.random.default_rng(11)
    keys = g.standard_normal((6, 128)).astype(np.float32)
    slots = np.array([3, -1, 0, 7, 5, -1], np.int64)
    kc = np.full((8, 128), 0x1234, np.uint16)
    cache_write_bf16(keys, slots, kc)
    lib = torch.from_numpy(keys).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(kc[s], lib[t])
    assert (kc[[1, 2, 4, 6]] == 0x1234).all()
