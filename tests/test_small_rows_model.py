"""A CPU model of topk_rows' small-row path (`topk_small_rows_kernel`).

Not the oracle and not the kernel: a plain restatement of the kernel's
steps for one row of at most 4096 keys, 1024 threads of 4 consecutive keys
each:

* up to four radix rounds over the 32-bit value keys, 8 bits per round
  from the top; in each round one wave of 64 lanes (4 digits per lane)
  finds the digit where the count from the top reaches the remaining rank,
  and the rounds stop early when the keys matching the bits found so far
  (the prefix) number exactly the remaining rank;
* one scan of the packed counts (keys above the prefix) << 16 | (keys
  matching it) in thread order, which gives each thread its output offset
  and its ties' ranks; the matching keys with the lowest positions are
  kept.

Checked here: every round has exactly one lane that holds the digit, the
packed counts never carry between their halves, exactly k distinct outputs
are written, and the selected set equals the oracle's (`oracle.topk_order`)
for random rows, heavy ties, signed zeros, denormals and infinities.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

SM_WG, SM_PER, WAVE = 1024, 4, 64


def float_key(x):
    """The kernel's order-preserving key: 2^31 + |x| for x >= +0, 2^31 - |x|
    for negative x (bit patterns), so -0 and +0 share one key."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.int64)
    mag = u & 0x7FFFFFFF
    return np.where(u >> 31 == 1, 0x80000000 - mag, 0x80000000 + mag)


def small_row(vals: np.ndarray, k: int) -> list:
    """Row-local positions the small-row path emits (any order)."""
    n = vals.shape[0]
    assert n <= SM_WG * SM_PER
    if n <= k:
        return list(range(n))
    vk = np.zeros(SM_WG * SM_PER, np.int64)
    ok = np.zeros(SM_WG * SM_PER, bool)
    vk[:n] = float_key(vals)
    ok[:n] = True
    prefix, pmask, kk = 0, 0, k
    for d in range(4):
        shift = 24 - 8 * d
        match = ok & ((vk & pmask) == prefix)
        hist = np.bincount(((vk[match] >> shift) & 255).astype(np.int64), minlength=256)
        holders = []
        for lane in range(WAVE):
            c = hist[4 * lane:4 * lane + 4]
            above = int(hist[4 * lane + 4:].sum())  # keys in the digits of higher lanes
            if above < kk <= above + int(c.sum()):
                i = 3
                while i > 0 and above + int(c[i]) < kk:
                    above += int(c[i])
                    i -= 1
                holders.append((4 * lane + i, above, int(c[i])))
        assert len(holders) == 1
        digit, above, count = holders[0]
        kk -= above
        prefix |= digit << shift
        pmask |= 255 << shift
        if count == kk:
            break
    t_keys = vk.reshape(SM_WG, SM_PER) & pmask
    t_ok = ok.reshape(SM_WG, SM_PER)
    gt = (t_ok & (t_keys > prefix)).sum(axis=1)
    eq = (t_ok & (t_keys == prefix)).sum(axis=1)
    assert gt.sum() < 1 << 16 and eq.sum() < 1 << 16
    packed = (gt << 16) | eq
    before = np.concatenate([[0], np.cumsum(packed)[:-1]])
    out = [None] * k
    for t in range(SM_WG):
        eq_before = int(before[t]) & 0xFFFF
        at = (int(before[t]) >> 16) + min(eq_before, kk)
        tie = eq_before
        for e in range(SM_PER):
            p = SM_PER * t + e
            if not ok[p]:
                continue
            keep = False
            if vk[p] & pmask > prefix:
                keep = True
            elif vk[p] & pmask == prefix:
                keep = tie < kk
                tie += 1
            if keep:
                assert at < k and out[at] is None
                out[at] = p
                at += 1
    assert all(o is not None for o in out)
    return out


def _rows(g, n):
    yield g.standard_normal(n).astype(np.float32)
    yield g.integers(-3, 4, n).astype(np.float32)
    yield np.where(g.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    v = np.full(n, -1.0, np.float32)
    v[g.choice(n, min(n, 300), replace=False)] = (np.arange(1, min(n, 300) + 1) * 1.4e-45).astype(np.float32)
    yield v
    x = g.standard_normal(n).astype(np.float32)
    x[g.choice(n, min(n, 20), replace=False)] = np.inf
    x[g.choice(n, min(n, 20), replace=False)] = -np.inf
    yield x
    yield np.full(n, 2.5, np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_small_row_model_matches_oracle(seed):
    g = np.random.default_rng(300 + seed)
    for _ in range(3):
        n = int(g.integers(1, SM_WG * SM_PER + 1))
        k = int(g.integers(1, min(n + 2, 1500)))
        for vals in _rows(g, n):
            got = sorted(small_row(vals, k))
            exp = sorted(int(i) for i in oracle.topk_order(vals.astype(np.float64), k) if i >= 0)
            assert got == exp, (seed, n, k)


def test_small_row_model_edges():
    g = np.random.default_rng(7)
    for n, k in ((4096, 1), (4096, 4095), (4096, 4096), (2, 1), (1, 1), (4096, 2048)):
        for vals in _rows(g, n):
            got = sorted(small_row(vals, k))
            exp = sorted(int(i) for i in oracle.topk_order(vals.astype(np.float64), k) if i >= 0)
            assert got == exp, (n, k)
