"""A CPU model of topk_rows' workgroup path at wave granularity.

Not the oracle and not the kernel: a plain restatement of the kernel's
streaming selection (sparse_attention_indexer_fp8_amd/csrc/topk_rows.hip,
`stream_row`, `append_tile`, `after_tile`, `keep_compact`, `wg_row`) on the
LDS candidate buffer, used to check three things the GPU cannot show
directly, over many rows and every buffer size the launch accepts:

* every candidate index the workgroup writes or reads lies inside the
  buffer, and every emitted position inside the row;
* between two barriers, no entry of the buffer is written by one wave and
  read or written by another (the model records, per entry, the phase and
  wave of its last write and the waves that read it in the current phase;
  waves take their atomic reservations in a random order each phase);
* the selected set equals the oracle's (`oracle.topk_order`) for rows with
  ties, +-0, one value repeated, and rows just above k.

The bounds the kernel takes from its own histograms (the first tile's
estimate, the proven first-histogram bound, the compaction's slack select)
are drawn here at random among the values those routines may return, so
the rest of the algorithm is exercised on all of them.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

TR_WG, TR_VEC = 256, 2
TR_TILE = TR_WG * TR_VEC * 4
TR_BATCH = 4
TR_EMIT = 8
WAVE = 64
NWAVES = TR_WG // WAVE
SEL_BINS = 1024


def float_key(x):
    """Order-preserving map of float32 values to uint32 (negative values
    flipped, positive values offset by 2^31)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    mag = u & 0x7FFFFFFF
    return np.where(u >> 31, 0x80000000 - mag, 0x80000000 + mag).astype(np.uint64)


def key_float(k):
    k = np.uint64(k)
    if k >= 0x80000000:
        return np.array([k - 0x80000000], dtype=np.uint64).astype(np.uint32).view(np.float32)[0]
    return np.array([(0x80000000 - k) | 0x80000000], dtype=np.uint64).astype(np.uint32).view(np.float32)[0]


def rank_keys(vals, pos):
    return (float_key(vals) << np.uint64(32)) | (~np.asarray(pos, dtype=np.uint64) & np.uint64(0xFFFFFFFF))


class Race(AssertionError):
    pass


class Lds:
    """The candidate buffer with per-entry access records."""

    def __init__(self, cap):
        self.cap = cap
        self.a = np.zeros(cap, dtype=np.uint64)
        self.w_phase = np.full(cap, -1, dtype=np.int64)
        self.w_wave = np.full(cap, -1, dtype=np.int64)
        self.r_phase = np.full(cap, -1, dtype=np.int64)
        self.r_waves = np.zeros(cap, dtype=np.uint8)  # bit per wave, for r_phase
        self.live = 0  # entries [0, live) hold keys of the current epoch
        self.phase = 0

    def barrier(self):
        self.phase += 1

    def write(self, wave, idx, vals):
        idx = np.asarray(idx, dtype=np.int64)
        if idx.size == 0:
            return
        if idx.min() < 0 or idx.max() >= self.cap:
            raise AssertionError(f"candidate write outside the buffer: {idx.max()} >= {self.cap}")
        same = self.w_phase[idx] == self.phase
        if (same & (self.w_wave[idx] != wave)).any():
            raise Race("two waves write one entry between barriers")
        rd = (self.r_phase[idx] == self.phase) & ((self.r_waves[idx] & ~np.uint8(1 << wave)) != 0)
        if rd.any():
            raise Race("an entry read by another wave is overwritten between barriers")
        self.a[idx] = vals
        self.w_phase[idx] = self.phase
        self.w_wave[idx] = wave

    def read(self, wave, idx):
        idx = np.asarray(idx, dtype=np.int64)
        if idx.size == 0:
            return np.zeros(0, dtype=np.uint64)
        if idx.min() < 0 or idx.max() >= self.cap:
            raise AssertionError(f"candidate read outside the buffer: {idx.max()} >= {self.cap}")
        if idx.max() >= self.live:
            raise AssertionError("read of an entry no thread of this epoch wrote")
        if ((self.w_phase[idx] == self.phase) & (self.w_wave[idx] != wave)).any():
            raise Race("an entry written by another wave is read between barriers")
        fresh = self.r_phase[idx] != self.phase
        self.r_waves[idx[fresh]] = 0
        self.r_phase[idx] = self.phase
        self.r_waves[idx] |= np.uint8(1 << wave)
        return self.a[idx]


def wave_of_thread(tid):
    return tid // WAVE


def first_hist_bound(keys, rank):
    """wg_select's first histogram over [min, max] of 64-bit keys: the lower
    edge of the bin where the count from the top reaches `rank` (at least
    rank keys are >= it)."""
    lo, hi = int(keys.min()), int(keys.max())
    span = hi - lo
    if span == 0:
        return lo
    shift = max(span.bit_length() - 10, 0)
    bins = (keys - np.uint64(lo)) >> np.uint64(shift)
    counts = np.bincount(bins.astype(np.int64), minlength=SEL_BINS)
    above = np.cumsum(counts[::-1])[::-1]  # keys in bins >= b
    b = int(np.nonzero(above >= rank)[0].max())
    return lo + (b << shift)


def slack_select(keys, k, slack, rng):
    """A bound T with k <= (keys >= T) <= k + slack, drawn at random."""
    desc = np.sort(keys)[::-1]
    hi = min(len(desc), k + slack)
    r = int(rng.integers(k, hi + 1))
    return int(desc[r - 1])


class Row:
    def __init__(self, vals, head):
        self.v = np.asarray(vals, dtype=np.float32)
        self.n = len(vals)
        self.head = min(head, self.n)
        self.nv = (self.n - self.head) // 4
        self.tail0 = self.head + 4 * self.nv
        self.ntail = self.n - self.tail0
        self.ntiles = (self.nv + TR_WG * TR_VEC - 1) // (TR_WG * TR_VEC)

    def tile(self, t):
        """Per wave: the positions of its valid elements of tile t in ballot
        order (vector v, component c, then lane), as the kernel appends them."""
        vi0 = t * TR_WG * TR_VEC
        out = []
        for w in range(NWAVES):
            tid = w * WAVE + np.arange(WAVE)
            ps = []
            for v in range(TR_VEC):
                vi = vi0 + v * TR_WG + tid
                ok = vi < self.nv
                for c in range(4):
                    ps.append((self.head + 4 * vi + c)[ok])
            out.append(np.concatenate(ps))
        return out

    def extras(self):
        return {tid: (tid if tid < self.head else self.tail0 + (tid - self.head))
                for tid in range(self.head + self.ntail)}


def append_tile(lds, cnt, row, per_wave, extra, lf, rng):
    """Each wave reserves its kept elements with one atomic add (waves in a
    random order) and writes them in ballot order."""
    for w in rng.permutation(NWAVES):
        pos = per_wave[w]
        pos = pos[row.v[pos] >= lf]
        ex = [extra[tid] for tid in range(w * WAVE, (w + 1) * WAVE) if tid in extra and row.v[extra[tid]] >= lf]
        pos = np.concatenate([pos, np.asarray(ex, dtype=np.int64)]).astype(np.int64)
        if pos.size == 0:
            continue
        base = cnt[0]
        cnt[0] += pos.size
        lds.live = max(lds.live, cnt[0])
        lds.write(w, np.arange(base, base + pos.size), rank_keys(row.v[pos], pos))


def strided_read(lds, c):
    """Every thread reads entries tid, tid + WG, ... below c (its wave's)."""
    i = np.arange(c)
    w = (i % TR_WG) // WAVE
    return np.concatenate([lds.read(x, i[w == x]) for x in range(NWAVES)])


def keep_compact(lds, cnt, c, T, rng):
    """In place, in batches of TR_BATCH * WG entries: a batch is read
    (barrier), then each wave reserves its kept count and writes them below
    the batch's end. Returns the smallest kept value key."""
    lds.barrier()  # tid 0 clears the counter, then a barrier
    kept_total = 0
    minkey = None
    B = TR_BATCH * TR_WG
    for b0 in range(0, c, B):
        batch = {}
        i = np.arange(b0, min(c, b0 + B))
        wv = ((i - b0) % TR_WG) // WAVE
        for w in range(NWAVES):
            idx = i[wv == w]
            batch[w] = (idx, lds.read(w, idx))
        lds.barrier()
        for w in rng.permutation(NWAVES):
            idx, keys = batch[w]
            keep = keys[keys >= np.uint64(T)]
            at = kept_total
            kept_total += len(keep)
            if len(keep):
                if at + len(keep) > b0 + B:
                    raise AssertionError("a compaction write lands above the batch being read")
                lds.write(w, np.arange(at, at + len(keep)), keep)
                mk = int((keep >> np.uint64(32)).min())
                minkey = mk if minkey is None else min(minkey, mk)
    lds.barrier()
    cnt[0] = kept_total
    lds.live = kept_total
    return minkey


def stream_row(row, k, cap, estimate, lds, cnt, rng):
    lf = -np.inf
    estimated = False
    empty = [np.zeros(0, dtype=np.int64) for _ in range(NWAVES)]
    t0 = row.tile(0) if row.ntiles > 0 else empty
    ex = row.extras()
    n0 = 4 * min(row.nv, TR_WG * TR_VEC) + row.head + row.ntail
    if row.ntiles > 1 and n0 > k:
        rank = k
        if estimate:
            want = (3 * k * n0 + 2 * row.n - 1) // (2 * row.n) + 8
            if want < k:
                rank, estimated = want, True
        pos = np.concatenate([np.concatenate(t0), np.asarray(sorted(ex.values()), dtype=np.int64)]).astype(np.int64)
        keys = rank_keys(row.v[pos], pos)
        vals = row.v[pos]
        vmin, vmax = float(vals.min()), float(vals.max())
        width = np.float32(vmax) - np.float32(vmin)
        if estimated and 0 < width < np.inf:
            scale = np.float32(SEL_BINS) / np.float32(width)
            f = np.clip((vals - np.float32(vmin)) * scale, 0, SEL_BINS - 1).astype(np.int64)
            counts = np.bincount(f, minlength=SEL_BINS)
            above = np.cumsum(counts[::-1])[::-1]
            b = int(np.nonzero(above >= rank)[0].max())
            lf = np.float32(vmin) + np.float32(b) / scale
        else:
            lf = key_float(first_hist_bound(keys, rank) >> 32)
    if row.ntiles > 0:
        append_tile(lds, cnt, row, t0, ex, lf, rng)
        lf = after_tile(row, 0, k, cap, lf, lds, cnt, rng)
    else:
        append_tile(lds, cnt, row, empty, ex, lf, rng)
        lds.barrier()
    for t in range(1, row.ntiles):
        append_tile(lds, cnt, row, row.tile(t), {}, lf, rng)
        lf = after_tile(row, t, k, cap, lf, lds, cnt, rng)
    return estimated


def after_tile(row, t, k, cap, lf, lds, cnt, rng):
    lds.barrier()
    c = cnt[0]
    lds.barrier()
    if c > cap:
        raise AssertionError(f"candidate buffer overrun: {c} > {cap}")
    if t + 1 == row.ntiles or c <= k or c + TR_TILE <= cap:
        return lf
    slack = ((cap - TR_TILE - k) & 0xFFFFFFFF) // 2
    if slack >= 1 << 30:
        raise AssertionError("the compaction slack wrapped")
    keys = strided_read(lds, c)
    lds.barrier()
    T = slack_select(keys, k, slack, rng)
    minkey = keep_compact(lds, cnt, c, T, rng)
    if cnt[0] + TR_TILE > cap:
        raise AssertionError("the next tile would not fit after a compaction")
    return key_float(minkey)


def model_row(vals, k, cap, head, rng):
    """The workgroup path for one row; returns the selected positions."""
    row = Row(vals, head)
    if row.n <= k:
        return np.arange(row.n)
    lds = Lds(cap)
    cnt = [0]
    estimated = stream_row(row, k, cap, True, lds, cnt, rng)
    c = cnt[0]
    if estimated and c < k:
        lds.barrier()
        cnt[0] = 0
        lds.live = 0
        lds.barrier()
        stream_row(row, k, cap, False, lds, cnt, rng)
        c = cnt[0]
    keys = strided_read(lds, c)
    T = np.sort(keys)[::-1][k - 1] if c > k else 0
    # emission: keys >= T, positions inside the row
    sel = keys[keys >= np.uint64(T)]
    pos = (~sel & np.uint64(0xFFFFFFFF)).astype(np.int64)
    assert (pos < row.n).all() and (pos >= 0).all(), "emitted position outside the row"
    assert len(pos) == min(k, row.n)
    return pos


def rows_cap(k):
    return max(k + TR_TILE + TR_TILE // 2, 2 * TR_TILE) + 8


def cap_ok(cap, k):
    return cap >= TR_TILE + 6 and cap - TR_TILE - k >= 2


def _row(kind, n, rng):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":
        return rng.integers(-20, 20, n).astype(np.float32)
    if kind == "zeros":
        v = rng.standard_normal(n).astype(np.float32)
        v[rng.random(n) < 0.3] = 0.0
        v[rng.random(n) < 0.3] = -0.0
        return v
    if kind == "const":
        return np.full(n, 1.5, np.float32)
    if kind == "rising":
        return np.arange(n, dtype=np.float32)
    if kind == "falling":  # the first tile holds the best: the estimated bound is too high, the row streams again
        return -np.arange(n, dtype=np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("k", [1, 7, 64, 512, 1000])
@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "const", "rising", "falling"])
def test_model_matches_oracle_at_every_accepted_cap(k, kind):
    """Buffer sizes from the smallest the launch guard accepts to the one
    launches use; row lengths from just above k to several tiles; heads of
    0..3 scalar elements (unaligned starts)."""
    rng = np.random.default_rng(hash((k, kind)) % (1 << 32))
    lo = TR_TILE + k + 2 if TR_TILE + k + 2 >= TR_TILE + 6 else TR_TILE + 6
    caps = sorted({lo, lo + 1, (lo + rows_cap(k)) // 2, rows_cap(k)})
    for cap in caps:
        assert cap_ok(cap, k)
        for n in (k + 1, TR_TILE + 3, 3 * TR_TILE + 17, 6 * TR_TILE + 1):
            if n <= k:
                continue
            for head in (0, 3):
                vals = _row(kind, n, rng)
                got = model_row(vals, k, cap, head, rng)
                exp = oracle.topk_order(vals.astype(np.float64), k)
                assert np.array_equal(np.sort(got), np.sort(exp)), (cap, n, head)


def test_model_detects_a_missing_barrier():
    """The race check itself: a compaction whose writes are not separated
    from its reads by a barrier is caught."""
    rng = np.random.default_rng(5)
    lds = Lds(64)
    lds.live = 64
    lds.write(0, np.arange(64), np.arange(64, dtype=np.uint64))
    lds.barrier()
    lds.read(1, np.arange(32))
    with pytest.raises(Race):
        lds.write(0, np.arange(16), np.zeros(16, dtype=np.uint64))
    with pytest.raises(AssertionError):
        Lds(8).write(0, np.array([8]), np.zeros(1, dtype=np.uint64))
    assert rng is not None


def test_model_rejects_a_buffer_below_the_guard():
    """A buffer one entry below the guard's minimum (cap - TILE - k = 1)
    makes the compaction slack zero; with 0 the uint32 slack would wrap. The
    model flags the wrapped form, which the launch guard excludes."""
    k = 64
    with pytest.raises(AssertionError):
        rng = np.random.default_rng(1)
        vals = rng.standard_normal(6 * TR_TILE).astype(np.float32)
        model_row(vals, k, TR_TILE + k - 1, 0, rng)
