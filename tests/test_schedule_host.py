"""Host-side checks of the balanced (quad, chunk) schedule of the row-group
call for few rows: the arithmetic its kernel relies on, restated and checked
over many length mixes (no GPU)."""
import math

import numpy as np
import pytest

PF_SAMPLE = 64  # groups per chunk at most (a chunk is then all sample)
GROUP = 16


def ceil_div_small(x: int, d: int) -> int:
    """The kernel's ceil(x / d) for x < 2^24: a float32 estimate of
    (x + d - 1) / d from the float32 reciprocal of d, corrected by one step
    each way."""
    y = x + d - 1
    q = int(np.float32(y) * np.float32(np.float32(1.0) / np.float32(d)))
    q -= 1 if q * d > y else 0
    q += 1 if (q + 1) * d <= y else 0
    return q


def test_ceil_div_small_exact():
    g = np.random.default_rng(5)
    xs = np.concatenate([np.arange(0, 4096), g.integers(0, 1 << 24, size=20000), [(1 << 24) - 1, (1 << 24) - 64]])
    for d in range(1, PF_SAMPLE + 1):
        for x in xs[:: max(1, d // 8)]:
            x = int(x)
            assert ceil_div_small(x, d) == -(-x // d), (x, d)


def schedule(lens, simds=1024, msl=None):
    """Grid waves as the host sizes them and the device's (quad, chunk)
    pairs: lane q holds quad q's longest row in groups, g groups per chunk."""
    lens = np.asarray(lens, np.int64)
    batch = len(lens)
    nq = (batch + 3) // 4
    msl = int(lens.max()) if msl is None else msl
    full = nq * ((max(msl, 1) + PF_SAMPLE * GROUP - 1) // (PF_SAMPLE * GROUP))
    waves = max(simds, full, 2 * nq)
    W = (waves + 3) // 4 * 4  # whole workgroups of four waves
    gq = [-(-int(lens[4 * q:4 * q + 4].max()) // GROUP) for q in range(nq)]
    G = sum(gq)
    g = -(-G // (W - nq)) if W > nq else 1
    g = min(max(g, 1), PF_SAMPLE)
    pairs = [(q, c) for q in range(nq) for c in range(ceil_div_small(gq[q], g) if gq[q] else 0)]
    return W, g, gq, pairs


@pytest.mark.parametrize("seed", range(40))
def test_balanced_pairs_fit_grid_and_cover_every_group(seed):
    g = np.random.default_rng(seed)
    nq = int(g.integers(1, 65))
    batch = 4 * nq - int(g.integers(0, 4))
    kind = seed % 4
    msl = int(g.choice([1024, 6000, 65536, 300000]))
    if kind == 0:
        lens = g.integers(0, msl + 1, size=batch)
    elif kind == 1:
        lens = np.full(batch, msl)
    elif kind == 2:
        lens = np.where(g.random(batch) < 0.5, 0, g.integers(1, msl + 1, size=batch))
    else:
        lens = g.integers(msl // 2, msl + 1, size=batch)
    W, gsz, gq, pairs = schedule(lens, simds=int(g.choice([256, 1024])), msl=msl)
    assert len(pairs) <= W
    assert 1 <= gsz <= PF_SAMPLE
    # every 16-token group of every quad lies in exactly one pair's chunk
    for q in range(len(gq)):
        chunks = [c for (qq, c) in pairs if qq == q]
        covered = sum(min(gsz, gq[q] - c * gsz) for c in chunks)
        assert covered == gq[q]
        assert chunks == list(range(len(chunks)))


def test_balanced_all_rows_empty():
    W, gsz, gq, pairs = schedule(np.zeros(8, np.int64), msl=4096)
    assert pairs == [] and gsz == 1
