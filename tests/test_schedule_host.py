"""Host-side checks of the chunk schedules (no GPU): the balanced (quad,
chunk) schedule of the row-group call for few rows, restated and checked
over many length mixes, and the workgroup -> (rows, chunk) maps of the
chunk-major indexer grids (one row, or two rows of a quad, per workgroup)."""
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


# ---------------------------------------------------------------------------
# Chunk-major grids of the indexer kernels (csrc/indexer.hip: chunk_of with
# quad_map, pair_chunk_of), restated: workgroup index -> (rows, chunk).
# ---------------------------------------------------------------------------


def quad_slot(i: int, batch: int):
    """chunk_of under quad_map: workgroup i -> (row, chunk)."""
    r = (i >> 3) & 3
    Q = ((i >> 5) << 3) | (i & 7)
    nq = batch >> 2
    c = Q // nq
    return 4 * ((Q + c) % nq) + r, c


def pair_slot(i: int, batch: int):
    """pair_chunk_of: workgroup i -> (first row of the pair, chunk)."""
    h = (i >> 3) & 1
    Q = ((i >> 4) << 3) | (i & 7)
    nq = batch >> 2
    c = Q // nq
    return 4 * ((Q + c) % nq) + 2 * h, c


@pytest.mark.parametrize("batch,nchunk", [(8, 1), (12, 5), (64, 33), (16, 40), (256, 3)])
def test_pair_grid_covers_every_pair_chunk_once(batch, nchunk):
    """Every (pair, chunk) with chunk < nchunk is taken by exactly one
    workgroup of the pair grid (whole groups of 16), padding workgroups get
    chunks >= nchunk, and the two pairs of a quad on one chunk sit on the same
    XCD (workgroups dealt to 8 XCDs round-robin by index)."""
    grid = -(-(nchunk * (batch // 2)) // 16) * 16
    seen = {}
    for i in range(grid):
        b0, c = pair_slot(i, batch)
        assert b0 % 2 == 0 and 0 <= b0 <= batch - 2
        if c >= nchunk:
            continue
        assert (b0, c) not in seen
        seen[(b0, c)] = i % 8
    assert len(seen) == nchunk * (batch // 2)
    for (b0, c), xcd in seen.items():
        if b0 % 4 == 0:
            assert seen[(b0 + 2, c)] == xcd


@pytest.mark.parametrize("batch,nchunk", [(8, 1), (12, 5), (64, 33)])
def test_quad_grid_matches_pair_grid_rows(batch, nchunk):
    """The per-row quad grid (chunk_of) and the pair grid cover the same
    (row, chunk) set, and both keep a quad's rows of one chunk on one XCD."""
    grid_q = -(-(nchunk * batch) // 32) * 32
    rows_q = {}
    for i in range(grid_q):
        b, c = quad_slot(i, batch)
        if c < nchunk:
            assert (b, c) not in rows_q
            rows_q[(b, c)] = i % 8
    grid_p = -(-(nchunk * (batch // 2)) // 16) * 16
    rows_p = set()
    for i in range(grid_p):
        b0, c = pair_slot(i, batch)
        if c < nchunk:
            rows_p.update({(b0, c), (b0 + 1, c)})
    assert set(rows_q) == rows_p == {(b, c) for b in range(batch) for c in range(nchunk)}
    for (b, c), xcd in rows_q.items():
        assert rows_q[(b - b % 4, c)] == xcd
