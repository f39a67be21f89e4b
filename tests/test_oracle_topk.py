"""Pins for the oracle's selection, addressing and page transform (CPU only)."""
import heapq
import itertools
import json
import os

import numpy as np
import pytest

import workloads
from oracle.indexer import page_transform, topk_order, topk_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_cases():
    with open(os.path.join(GOLDEN, "topk_hand_cases.json")) as f:
        d = json.load(f)
    out = []
    for c in d["cases"]:
        vals = np.array([float(v) for v in c["values"]], dtype=np.float32)
        out.append(pytest.param(vals, c["k"], c["expected"], id=c["name"]))
    return out


@pytest.mark.parametrize("values,k,expected", _hand_cases())
def test_hand_built_cases(values, k, expected):
    assert topk_order(values.astype(np.float64), k).tolist() == expected


def _dominates(v, s, u):
    return v[s] > v[u] or (v[s] == v[u] and s < u)


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_unique_dominant_subset(seed):
    """On tiny rows, the selected set is the only subset of size min(k, n) whose
    every member beats every non-member (by value, ties to lower position)."""
    g = np.random.default_rng(seed)
    n = int(g.integers(0, 9))
    k = int(g.integers(1, 7))
    pool = np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 2.0, np.inf, -np.inf, 1e-45])
    v = g.choice(pool, size=n)
    got = topk_order(v, k)
    m = min(k, n)
    assert (got[m:] == -1).all() and (got[:m] >= 0).all()
    sel = set(got[:m].tolist())
    winners = []
    for sub in itertools.combinations(range(n), m):
        s = set(sub)
        if all(_dominates(v, a, b) for a in s for b in range(n) if b not in s):
            winners.append(s)
    assert winners == [sel]
    # and in order: each output beats the next one
    assert all(_dominates(v, int(got[i]), int(got[i + 1])) for i in range(m - 1))


@pytest.mark.parametrize("seed", range(20))
def test_matches_heapq_nlargest(seed):
    """Library special case: heapq.nlargest keyed on (value, -position) gives the
    same positions in the same order (documented equal to sorted(...)[:k])."""
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(1, 300))
    k = int(g.integers(1, 64))
    v = np.round(g.standard_normal(n) * 4) / 4  # many ties
    ref = heapq.nlargest(k, range(n), key=lambda i: (v[i], -i))
    got = topk_order(v, k)
    assert got[:len(ref)].tolist() == ref
    assert (got[len(ref):] == -1).all()


def test_nan_refused():
    with pytest.raises(ValueError):
        topk_order(np.array([1.0, np.nan]), 1)


def _check_invariants(vals, sel, k):
    n = vals.shape[0]
    m = min(k, n)
    assert sel.shape == (k,)
    assert (sel[:m] >= 0).all() and (sel[:m] < n).all() and (sel[m:] == -1).all()
    assert len(set(sel[:m].tolist())) == m
    if m < n:
        mask = np.zeros(n, bool)
        mask[sel[:m]] = True
        assert vals[mask].min() >= vals[~mask].max()


def test_invariants_on_decode_rows():
    case = workloads.decode_rows_case(seed=7, rows=8, stride=1024, n_lo=1, n_hi=1024, k=256)
    out = topk_rows(case.scores, case.seq_lens, case.k)
    for i in range(case.rows):
        vals = case.scores[i, :case.seq_lens[i]].astype(np.float64)
        _check_invariants(vals, out[i], case.k)


def test_packed_equals_row_local():
    """The packed extend layout gives exactly the result of the row-local layout
    (each window copied to column 0 of its own row, page-table row repeated)."""
    case = workloads.packed_prefill_case(seed=11, prefix0=300, new_tokens=40, k=64)
    packed = topk_rows(case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch,
                       case.page_table, 1)
    n_max = int(case.seq_lens.max())
    local = np.full((case.rows, n_max), np.inf, np.float32)
    pt_local = np.empty((case.rows, case.page_table.shape[1]), np.int32)
    for i in range(case.rows):
        rs, n = int(case.row_starts[i]), int(case.seq_lens[i])
        local[i, :n] = case.scores[i, rs:rs + n]
        pt_local[i] = case.page_table[case.row_to_batch[i]]
    row_local = topk_rows(local, case.seq_lens, case.k, None, None, pt_local, 1)
    assert np.array_equal(packed, row_local)


def test_sentinels_outside_windows_are_never_selected():
    case = workloads.packed_prefill_case(seed=12, prefix0=100, new_tokens=20, k=32)
    pos = topk_rows(case.scores, case.seq_lens, case.k, case.row_starts, None, None)
    for i in range(case.rows):
        rs, n = int(case.row_starts[i]), int(case.seq_lens[i])
        v = pos[i][pos[i] >= 0]
        assert np.isfinite(case.scores[i, rs + v]).all()


def test_page_transform_identity_and_permutation():
    g = np.random.default_rng(3)
    pos = np.array([5, 0, 17, -1, 9, -1])
    ident = np.arange(32)
    assert page_transform(pos, ident, 1).tolist() == pos.tolist()
    perm = g.permutation(32)
    slots = page_transform(pos, perm, 1)
    inv = np.argsort(perm)
    back = np.where(slots >= 0, inv[np.maximum(slots, 0)], -1)
    assert back.tolist() == pos.tolist()


def test_page_transform_paged():
    """page_size 4: slot = table[j // 4] * 4 + j % 4, checked by a plain loop."""
    table = np.array([7, 2, 9, 0])
    pos = np.array([0, 3, 4, 7, 15, -1, 10])
    exp = []
    for j in pos:
        if j < 0:
            exp.append(-1)
            continue
        page, off = divmod(int(j), 4)
        exp.append(int(table[page]) * 4 + off)
    assert page_transform(pos, table, 4).tolist() == exp


def test_negative_zero_generated_cases_live():
    """The 1/16-grid snapping of the decode workload produces -0.0 values."""
    case = workloads.decode_rows_case(seed=101)
    fin = case.scores[np.isfinite(case.scores)]
    assert ((fin == 0) & np.signbit(fin)).any()


@pytest.mark.parametrize("seed", range(10))
def test_kv_offset_against_brute_force(seed):
    """A call over one chunk of each row's KV: the kept positions are the
    window's best (heapq.nlargest keyed on (value, -position)) shifted by the
    row's offset, then mapped; -1 padding stays -1."""
    g = np.random.default_rng(300 + seed)
    rows, stride, k = 4, 64, int(g.integers(1, 20))
    buf = np.round(g.standard_normal((rows, stride)) * 2) / 2  # ties
    lens = g.integers(0, 40, size=rows).astype(np.int32)
    starts = g.integers(0, stride - 40, size=rows).astype(np.int32)
    off = g.integers(0, 500, size=rows).astype(np.int32)
    pt = g.permutation(4096).reshape(4, 1024).astype(np.int32)
    r2b = g.integers(0, 4, size=rows).astype(np.int32)
    got = topk_rows(buf, lens, k, starts, r2b, pt, 1, kv_offset=off)
    for i in range(rows):
        n, s0 = int(lens[i]), int(starts[i])
        best = heapq.nlargest(k, range(n), key=lambda t: (buf[i, s0 + t], -t))
        exp = [int(pt[r2b[i], t + off[i]]) for t in best] + [-1] * (k - len(best))
        assert got[i].tolist() == exp
