"""GPU parity of topk_rows / topk_page_transform against the oracle (bit-exact sets)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests._helpers import dev, log, sorted_rows

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ops():
    import torch
    from sparse_attention_indexer_fp8_amd import ops as _ops

    torch.cuda.set_device(0)
    return _ops


def _run_rows(ops, scores, seq_lens, k, row_starts=None, row_to_batch=None, page_table=None, page_size=1):
    import torch

    out = ops.topk_rows(dev(scores), dev(seq_lens), k,
                        None if row_starts is None else dev(row_starts),
                        None if row_to_batch is None else dev(row_to_batch),
                        None if page_table is None else dev(page_table), page_size)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _hand_cases():
    with open(os.path.join(GOLDEN, "topk_hand_cases.json")) as f:
        return json.load(f)["cases"]


def test_hand_built_cases(ops):
    for c in _hand_cases():
        vals = np.array([float(v) for v in c["values"]], dtype=np.float32)
        n = vals.shape[0]
        buf = np.full((1, max(n, 1) + 3), np.inf, np.float32)
        buf[0, :n] = vals
        got = _run_rows(ops, buf, np.array([n], np.int32), c["k"])
        assert sorted(got[0].tolist()) == sorted(c["expected"]), c["name"]


def test_decode_c1_full(ops):
    case = workloads.c1_decode_topk()
    log(f"case {case.name}")
    got = _run_rows(ops, case.scores, case.seq_lens, case.k, page_table=case.page_table)
    ref = oracle.topk_rows(case.scores, case.seq_lens, case.k, page_table=case.page_table)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))
    # row-local positions too (no page table)
    got = _run_rows(ops, case.scores, case.seq_lens, case.k)
    ref = oracle.topk_rows(case.scores, case.seq_lens, case.k)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


@pytest.mark.parametrize("k", [1, 7, 64, 512, 2048])
def test_decode_rows_many_tiles(ops, k):
    """Rows spanning several 4096-float tiles, ragged tails, n around k."""
    case = workloads.decode_rows_case(seed=31 + k, rows=24, stride=20011, n_lo=max(1, k - 3), n_hi=20011,
                                      k=k, tie_frac=0.05, pt_width=20011)
    case.seq_lens[:4] = [k - 1 if k > 1 else 1, k, k + 1, 20011]
    log(f"decode rows k={k}")
    got = _run_rows(ops, case.scores, case.seq_lens, k, page_table=case.page_table)
    ref = oracle.topk_rows(case.scores, case.seq_lens, k, page_table=case.page_table)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


def test_packed_prefill_reduced(ops):
    """Packed extend layout with an odd stride and both indirections."""
    case = workloads.packed_prefill_case(seed=41, prefix0=9000, new_tokens=256, k=512)
    log(f"packed reduced stride={case.stride}")
    got = _run_rows(ops, case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch,
                    case.page_table, 1)
    ref = oracle.topk_rows(case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch,
                           case.page_table, 1)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


def test_packed_equals_row_local_on_gpu(ops):
    case = workloads.packed_prefill_case(seed=42, prefix0=5000, new_tokens=128, k=256)
    packed = _run_rows(ops, case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch,
                       case.page_table, 1)
    n_max = int(case.seq_lens.max())
    local = np.full((case.rows, n_max), np.inf, np.float32)
    pt_local = np.empty((case.rows, case.page_table.shape[1]), np.int32)
    for i in range(case.rows):
        rs, n = int(case.row_starts[i]), int(case.seq_lens[i])
        local[i, :n] = case.scores[i, rs:rs + n]
        pt_local[i] = case.page_table[case.row_to_batch[i]]
    row_local = _run_rows(ops, local, case.seq_lens, case.k, page_table=pt_local)
    assert np.array_equal(sorted_rows(packed), sorted_rows(row_local))


def _adversarial_rows(n=30000):
    rows = {}
    g = np.random.default_rng(5)
    rows["ascending"] = np.arange(n, dtype=np.float32)  # every tile beats the last: many compactions
    rows["descending"] = np.arange(n, 0, -1, dtype=np.float32)
    rows["all_equal"] = np.full(n, 3.25, np.float32)
    v = np.full(n, -1.0, np.float32)
    v[g.choice(n, 700, replace=False)] = (np.arange(1, 701) * 1.401298464324817e-45).astype(np.float32)
    z = g.choice(n, 4000, replace=False)
    v[z[:2000]] = 0.0
    v[z[2000:]] = -0.0
    rows["denormal_threshold"] = v
    w = np.where(g.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    rows["signed_zeros_only"] = w
    x = g.standard_normal(n).astype(np.float32)
    x[g.choice(n, 50, replace=False)] = np.inf
    x[g.choice(n, 50, replace=False)] = -np.inf
    rows["with_infinities"] = x
    y = np.round(g.standard_normal(n) * 2).astype(np.float32)  # few distinct values, heavy ties
    rows["coarse_ties"] = y
    return rows


@pytest.mark.parametrize("k", [512, 2048])
def test_adversarial_rows(ops, k):
    rows = _adversarial_rows()
    names = list(rows)
    n = 30000
    buf = np.stack([rows[nm] for nm in names])
    lens = np.full(len(names), n, np.int32)
    got = _run_rows(ops, buf, lens, k)
    ref = oracle.topk_rows(buf, lens, k)
    for i, nm in enumerate(names):
        assert np.array_equal(np.sort(got[i]), np.sort(ref[i])), nm


@pytest.mark.parametrize("k", [1, 512, 2048, 4095])
def test_small_rows_adversarial(ops, k):
    """Launches of few rows whose windows hold at most 4096 keys take one
    1024-thread workgroup per row (radix select on the value keys, ties to the
    lowest positions). The adversarial rows at 4096 keys and at shorter and
    odd lengths, exact sets against the oracle."""
    rows = _adversarial_rows(n=4096)
    names = list(rows)
    buf = np.stack([rows[nm] for nm in names])
    for lens in (np.full(len(names), 4096, np.int32),
                 np.array([4095, 3001, 2049, 1025, min(k + 1, 4096), 7, 4096], np.int32)):
        got = _run_rows(ops, buf, lens, k)
        ref = oracle.topk_rows(buf, lens, k)
        for i, nm in enumerate(names):
            assert np.array_equal(np.sort(got[i]), np.sort(ref[i])), (nm, int(lens[i]))


def test_small_rows_packed_paged(ops):
    """The one-workgroup small-row path with packed windows at unaligned
    starts, row_to_batch, a page size of 3 and heavily tied values."""
    g = np.random.default_rng(12)
    rows, stride, k, P, reqs = 40, 4093, 300, 3, 5
    lens = g.integers(1, 2000, size=rows).astype(np.int32)
    starts = g.integers(0, stride - lens + 1).astype(np.int32)
    buf = np.round(g.standard_normal((rows, stride)) * 3).astype(np.float32)
    r2b = g.integers(0, reqs, size=rows).astype(np.int32)
    npg = -(-2000 // P) + 1
    pt = np.stack([g.permutation(npg * 4)[:npg] for _ in range(reqs)]).astype(np.int32)
    got = _run_rows(ops, buf, lens, k, starts, r2b, pt, P)
    ref = oracle.topk_rows(buf, lens, k, starts, r2b, pt, P)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


@pytest.mark.parametrize("k,page_size,with_offset", [(512, 1, False), (64, 16, True), (300, 1, True)])
def test_short_rows_one_wave(ops, k, page_size, with_offset):
    """Launches of 2048 rows or more take rows of at most 8192 keys one wave
    per row. Every row against the oracle: lengths 1..8192 at odd window
    starts (so heads and tails are scalar, and some rows have no whole
    vector), 5% ties, and rows that defeat the wave's estimated bound and go
    to the workgroup path (ascending, descending, all equal, +-inf, a run of
    -0.0 / +0.0), with page tables and per-row KV offsets."""
    import torch

    rows, stride = 2304, 8200
    g = np.random.default_rng(500 + k)
    lens = g.integers(1, 8193, size=rows).astype(np.int32)
    lens[:8] = [1, 2, 3, 5, 6, 7, k, k + 1]
    starts = g.integers(0, stride - lens + 1).astype(np.int32)
    buf = np.full((rows, stride), np.inf, np.float32)
    for i in range(rows):
        n = int(lens[i])
        kind = i % 16
        if kind == 1:
            v = np.arange(n, dtype=np.float32)
        elif kind == 2:
            v = np.arange(n, 0, -1, dtype=np.float32)
        elif kind == 3:
            v = np.full(n, 0.25, np.float32)
        elif kind == 4:
            v = g.standard_normal(n).astype(np.float32)
            v[g.random(n) < 0.01] = np.inf
            v[g.random(n) < 0.01] = -np.inf
        elif kind == 5:
            v = np.where(g.random(n) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        else:
            v = g.standard_normal(n).astype(np.float32)
            m = g.random(n) < 0.05
            v[m] = np.round(v[m] * 16) / 16
        buf[i, starts[i]:starts[i] + n] = v
    off = g.integers(0, 1000, size=rows).astype(np.int32) if with_offset else None
    width = -(-(stride + 1000) // page_size)
    pt = np.stack([g.permutation(width * 2)[:width] for _ in range(4)]).astype(np.int32)
    r2b = g.integers(0, 4, size=rows).astype(np.int32)
    log(f"short rows: rows={rows} k={k} page_size={page_size} offset={with_offset}")
    out = ops.topk_rows(dev(buf), dev(lens), k, dev(starts), dev(r2b), dev(pt), page_size,
                        kv_offset=None if off is None else dev(off))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.topk_rows(buf, lens, k, starts, r2b, pt, page_size, kv_offset=off)
    bad = [i for i in range(rows) if not np.array_equal(np.sort(got[i]), np.sort(ref[i]))]
    assert not bad, f"rows differ from the oracle: {bad[:10]}"


def test_restream_inside_persistent_loop(ops):
    """More rows than resident workgroups, so each workgroup takes several rows
    in turn: descending rows defeat the estimated first-tile bound and are
    streamed again, ascending rows force compactions, and trivial rows
    (n <= k) sit in between, all next to ordinary random rows."""
    k, rows, stride = 512, 3000, 6007
    g = np.random.default_rng(11)
    lens = g.integers(300, stride + 1, size=rows).astype(np.int32)
    buf = np.full((rows, stride), np.inf, np.float32)
    for i in range(rows):
        n = int(lens[i])
        kind = i % 4
        if kind == 0:
            buf[i, :n] = np.arange(n, 0, -1, dtype=np.float32) * 0.5
        elif kind == 1:
            buf[i, :n] = np.arange(n, dtype=np.float32)
        else:
            buf[i, :n] = g.standard_normal(n).astype(np.float32)
    log(f"restream rows={rows} k={k}")
    got = _run_rows(ops, buf, lens, k)
    ref = oracle.topk_rows(buf, lens, k)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


def test_max_k(ops):
    case = workloads.decode_rows_case(seed=77, rows=6, stride=40000, n_lo=8000, n_hi=40000, k=8192,
                                      pt_width=40000)
    got = _run_rows(ops, case.scores, case.seq_lens, 8192, page_table=case.page_table)
    ref = oracle.topk_rows(case.scores, case.seq_lens, 8192, page_table=case.page_table)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


def test_empty_and_tiny_rows(ops):
    buf = np.full((5, 16), np.inf, np.float32)
    buf[1, :1] = 5.0
    buf[2, :3] = [1.0, -2.0, 3.0]
    buf[3, :16] = np.arange(16)
    buf[4, :5] = [2.0, 2.0, 2.0, 2.0, 2.0]
    lens = np.array([0, 1, 3, 16, 5], np.int32)
    got = _run_rows(ops, buf, lens, 4)
    ref = oracle.topk_rows(buf, lens, 4)
    assert np.array_equal(sorted_rows(got), sorted_rows(ref))


def test_page_sizes_and_transform(ops):
    """General page sizes (including non powers of two) in the fused epilogue
    and in the standalone transform."""
    import torch

    g = np.random.default_rng(9)
    for P in (1, 3, 16, 48, 64, 100):
        rows, k, n_hi = 6, 300, 9000
        case = workloads.decode_rows_case(seed=90 + P, rows=rows, stride=n_hi, n_lo=100, n_hi=n_hi, k=k,
                                          pt_width=4)
        npg = -(-n_hi // P)
        pt = np.stack([g.permutation(npg * 3)[:npg] for _ in range(rows)]).astype(np.int32)
        got = _run_rows(ops, case.scores, case.seq_lens, k, page_table=pt, page_size=P)
        ref = oracle.topk_rows(case.scores, case.seq_lens, k, page_table=pt, page_size=P)
        assert np.array_equal(sorted_rows(got), sorted_rows(ref)), P
        # standalone transform of the oracle's row-local positions
        pos = oracle.topk_rows(case.scores, case.seq_lens, k).astype(np.int32)
        r2b = g.integers(0, rows, size=rows).astype(np.int32)
        out = ops.topk_page_transform(dev(pos), dev(pt), P, dev(r2b))
        torch.cuda.synchronize()
        exp = np.stack([oracle.page_transform(pos[i], pt[r2b[i]], P) for i in range(rows)])
        assert np.array_equal(out.cpu().numpy(), exp), P


def test_deterministic_sets(ops):
    case = workloads.packed_prefill_case(seed=43, prefix0=3000, new_tokens=64, k=128)
    a = _run_rows(ops, case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch)
    b = _run_rows(ops, case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch)
    assert np.array_equal(sorted_rows(a), sorted_rows(b))


def test_packed_prefill_full_size(ops):
    """The full 16384 x 70001 packed buffer, in the launch configuration the
    benchmark times, plain and sorted output: every row against the oracle
    (set equality, and for the sorted call the oracle's exact sequence), in
    the oracle pool."""
    import torch

    from tests import _fullsize

    log("generating packed-prefill 16384x70001")
    case = workloads.c3_packed_prefill()
    sc = dev(case.scores)
    args = (dev(case.seq_lens), case.k, dev(case.row_starts), dev(case.row_to_batch), dev(case.page_table), 1)
    out = ops.topk_rows(sc, *args)
    srt = ops.topk_rows(sc, *args, sorted=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64)
    srt = srt.cpu().numpy().astype(np.int64)
    del sc, out
    case.scores = None  # the workers draw the rows again
    log("checking every row against the oracle")
    n = _fullsize.run(_fullsize.packed_rows_task, _fullsize.packed_tasks(case, got, srt), "packed prefill")
    assert n == case.seq_lens.shape[0]


@pytest.mark.parametrize("k", [1, 300, 512, 1000, 2048, 4000, 8192])
def test_topk_rows_sorted_order(ops, k):
    import torch

    case = workloads.c1_decode_topk()
    lens = case.seq_lens.copy()
    lens[0] = min(k - 1, lens[0])  # a padded row (empty for k = 1)
    out = ops.topk_rows(dev(case.scores), dev(lens), k, page_table=dev(case.page_table),
                        page_size=case.page_size, sorted=True)
    torch.cuda.synchronize()
    ref = oracle.topk_rows(case.scores, lens, k, page_table=case.page_table, page_size=case.page_size)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_topk_rows_sorted_ties_and_packed(ops):
    """Scores on a quarter grid (many ties) in the packed layout with
    row_starts and row_to_batch: ties come out by ascending position."""
    import torch

    case = workloads.packed_prefill_case(seed=661, prefix0=3000, new_tokens=128, k=256)
    buf = (np.round(case.scores * 4) / 4).astype(np.float32)
    out = ops.topk_rows(dev(buf), dev(case.seq_lens), case.k, row_starts=dev(case.row_starts),
                        row_to_batch=dev(case.row_to_batch), page_table=dev(case.page_table),
                        page_size=case.page_size, sorted=True)
    torch.cuda.synchronize()
    ref = oracle.topk_rows(buf, case.seq_lens, case.k, case.row_starts, case.row_to_batch, case.page_table,
                           case.page_size)
    assert np.array_equal(out.cpu().numpy(), ref)


# Chunked-prefix-cache extend: the call sees one chunk [c0, c1) of each
# request's KV, so row i's window is the slice of its full window that falls
# in the chunk, starting c0 columns later, and kv_offset = c0 puts the kept
# positions back in the request's KV before the page transform.
def _chunk_call(case, c0, c1):
    n = case.seq_lens.astype(np.int64)
    lens = np.clip(np.minimum(n, c1) - c0, 0, None).astype(np.int32)
    starts = (case.row_starts.astype(np.int64) + c0).astype(np.int32)
    off = np.full(case.rows, c0, np.int32)
    return lens, starts, off


@pytest.mark.parametrize("c0,c1,sorted_", [(0, 1 << 30, False), (1000, 5000, False), (4096, 9000, True),
                                           (8000, 1 << 30, True)])
def test_topk_rows_kv_offset_chunk(ops, c0, c1, sorted_):
    import torch

    case = workloads.packed_prefill_case(seed=43, prefix0=7000, new_tokens=256, k=512)
    lens, starts, off = _chunk_call(case, c0, c1)
    out = ops.topk_rows(dev(case.scores), dev(lens), case.k, row_starts=dev(starts),
                        row_to_batch=dev(case.row_to_batch), page_table=dev(case.page_table), page_size=1,
                        sorted=sorted_, kv_offset=dev(off))
    torch.cuda.synchronize()
    ref = oracle.topk_rows(case.scores, lens, case.k, starts, case.row_to_batch, case.page_table, 1,
                           kv_offset=off)
    got = out.cpu().numpy()
    if sorted_:
        assert np.array_equal(got, ref)
    else:
        assert np.array_equal(sorted_rows(got), sorted_rows(ref))
    if c0 == 0:
        full = _run_rows(ops, case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch,
                         case.page_table, 1)
        assert np.array_equal(sorted_rows(got), sorted_rows(full))


def test_topk_rows_kv_offset_paged_unaligned(ops):
    """Per-row offsets that do not fall on page boundaries (page size 16),
    and the unpaged output (positions in the request's KV)."""
    import torch

    case = workloads.c1_decode_topk()
    g = np.random.default_rng(44)
    rows = case.scores.shape[0]
    off = g.integers(0, 3000, size=rows).astype(np.int32)
    P = 16
    width = (4096 + 3000) // P + 2
    pt = np.stack([g.permutation(rows * width)[:width] for _ in range(rows)]).astype(np.int32)
    for page_table in (pt, None):
        out = ops.topk_rows(dev(case.scores), dev(case.seq_lens), case.k,
                            page_table=None if page_table is None else dev(page_table), page_size=P,
                            kv_offset=dev(off))
        torch.cuda.synchronize()
        ref = oracle.topk_rows(case.scores, case.seq_lens, case.k, page_table=page_table, page_size=P, kv_offset=off)
        assert np.array_equal(sorted_rows(out.cpu().numpy()), sorted_rows(ref))
