"""Every-row oracle checks of the full-size workloads.

The GPU outputs of a full-size call are split into tasks of a few rows; a
worker of the oracle pool (tests/_oracle_pool.py) draws each row's inputs
again from the seeds, runs the oracle on it and applies the acceptance rule:

* top-k over a given score buffer: the slot set equals the oracle's exactly
  (and, for sorted output, the whole sequence);
* fused indexer rows: ``check_fused_row`` (count, distinctness, every
  selected score >= the oracle's k-th score minus the tolerance, returned
  scores within the tolerance);
* block rows: the block-score criterion and the exact slot lists;
* unfused score rows: every score within the tolerance.

A worker computes an indexer row's oracle scores from the row's keys in
token order (identity block table); the GPU's slots are mapped back to token
positions through the row's real block table, so the paging is checked too.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads
from tests import _oracle_pool
from tests._helpers import check_fused_row, check_scores, log

_KEYS = {}  # per worker: the keys of the request drawn last


def _result(fails, rows, overlaps=()):
    return {"fails": fails, "rows": rows, "min_overlap": min(overlaps) if overlaps else 1.0}


def run(fn, tasks, label: str) -> int:
    """Run fn over the tasks in the oracle pool; fail with the first bad rows."""
    fails, rows, ov = [], 0, 1.0
    for r in _oracle_pool.get().imap_unordered(fn, tasks):
        fails += r["fails"]
        rows += r["rows"]
        ov = min(ov, r["min_overlap"])
    log(f"{label}: {rows} rows checked against the oracle, {len(fails)} failures, min overlap {ov:.4f}")
    assert not fails, f"{label}: {len(fails)} rows fail, first: {fails[:5]}"
    return rows


# ---------------------------------------------------------------------------
# Top-k over a given score buffer (packed prefill)
# ---------------------------------------------------------------------------


def packed_rows_task(t):
    """t: seed, tie_frac, k, rows, lens, r2b, page_table, got [m, k], sorted_got [m, k] or None."""
    fails = []
    for idx, i in enumerate(t["rows"]):
        n = int(t["lens"][idx])
        v = workloads.window_values(t["seed"], int(i), n, t["tie_frac"])
        exp = oracle.topk_rows(v[None, :], np.array([n]), t["k"], row_to_batch=np.array([t["r2b"][idx]]),
                               page_table=t["page_table"], page_size=1)[0]
        if not np.array_equal(np.sort(t["got"][idx]), np.sort(exp)):
            fails.append((int(i), "set"))
        elif t["sorted_got"] is not None and not np.array_equal(t["sorted_got"][idx], exp):
            fails.append((int(i), "sorted order"))
    return _result(fails, len(t["rows"]))


def packed_tasks(case, got, sorted_got=None, per_task=256, seed=None, tie_frac=0.01):
    seed = workloads.SEEDS["c3"] if seed is None else seed
    rows = int(case.seq_lens.shape[0])  # (the score buffer may already be freed)
    for i0 in range(0, rows, per_task):
        sl = slice(i0, min(rows, i0 + per_task))
        yield {"seed": seed, "tie_frac": tie_frac, "k": case.k, "rows": np.arange(sl.start, sl.stop),
               "lens": case.seq_lens[sl], "r2b": case.row_to_batch[sl], "page_table": case.page_table,
               "got": got[sl], "sorted_got": None if sorted_got is None else sorted_got[sl]}


# ---------------------------------------------------------------------------
# Indexer rows
# ---------------------------------------------------------------------------


def _row_scores(spec, b, page_size):
    """Oracle scores of row b (float64) from its own draws, and its length."""
    r = workloads.row_inputs(spec, b, _KEYS)
    npg = -(-max(r.n, 1) // page_size)
    ident = np.arange(npg, dtype=np.int64)
    if spec["bf16"]:
        S = oracle.index_scores_bf16(r.q, r.w, r.keys, ident, page_size, r.n)
    else:
        S = oracle.index_scores(r.q, r.q_scale, r.w, r.keys, r.k_scale, ident, page_size, r.n)
    return S, r


def fused_rows_task(t):
    """t: spec, page_size, k, rows, bt_rows, slots [m, k], scores [m, k] or
    None, gpu_scores (list of score rows, or None)."""
    fails, ov = [], []
    P = t["page_size"]
    for idx, b in enumerate(t["rows"]):
        S, r = _row_scores(t["spec"], int(b), P)
        try:
            if t.get("gpu_scores") is not None:
                check_scores(t["gpu_scores"][idx][:r.n], S)
            ts = oracle.token_slots(t["bt_rows"][idx], P, r.n)
            ov.append(check_fused_row(t["slots"][idx], None if t["scores"] is None else t["scores"][idx], S, ts,
                                      t["k"]))
        except AssertionError as e:
            fails.append((int(b), str(e)[:200]))
    return _result(fails, len(t["rows"]), ov)


def fused_tasks(case, slots, scores=None, per_task=1, rows=None, gpu_scores=None):
    """Tasks over `rows` (default: all); gpu_scores(rows) -> list of the
    unfused score rows to check as well."""
    spec = workloads.row_spec(case)
    rows = np.arange(case.batch) if rows is None else np.asarray(rows)
    r2b = case.row_to_batch
    for i0 in range(0, rows.shape[0], per_task):
        rr = rows[i0:i0 + per_task]
        prow = rr if r2b is None else r2b[rr]
        yield {"spec": spec, "page_size": case.page_size, "k": case.k, "rows": rr,
               "bt_rows": case.block_table[prow], "slots": slots[rr],
               "scores": None if scores is None else scores[rr],
               "gpu_scores": None if gpu_scores is None else gpu_scores(rr)}


def _block_check(S_col, n, bs, top, bt_row, blocks_row, slots_row):
    """Block-score criterion for one selection: distinct blocks, every
    selected block's score >= the oracle's top-th minus the tolerance, and
    each block's slot list exact."""
    bsv = oracle.block_scores(S_col, bs) if n > 0 else np.zeros(0)
    nb = bsv.shape[0]
    page_to_blk = {int(bt_row[c]): c for c in range(nb)}
    m = min(nb, top)
    assert (np.asarray(blocks_row[m:]) == -1).all(), "padding"
    if m == 0:
        return
    sel = [page_to_blk[int(p)] for p in blocks_row[:m]]
    assert len(set(sel)) == m, "duplicate block"
    sigma = max(float(np.sqrt(np.mean(S_col * S_col))), 1e-30)
    kth = np.sort(bsv)[::-1][m - 1]
    assert (bsv[sel] >= kth - 1e-3 * max(abs(kth), sigma)).all(), "block below the top-th minus tolerance"
    if slots_row is not None:
        for i, c in enumerate(sel):
            exp = np.full(bs, -1, np.int64)
            hi = min(bs, n - c * bs)
            exp[:hi] = int(bt_row[c]) * bs + np.arange(hi)
            assert np.array_equal(slots_row[i * bs:(i + 1) * bs], exp), "slot list"


def block_rows_task(t):
    """t: spec, page_size, bs, top, rows, bt_rows, blocks, slots, per_head."""
    fails = []
    P, bs, top = t["page_size"], t["bs"], t["top"]
    for idx, b in enumerate(t["rows"]):
        try:
            if t["per_head"]:
                r = workloads.row_inputs(t["spec"], int(b), _KEYS)
                npg = -(-max(r.n, 1) // P)
                T = oracle.index_head_scores(r.q, r.q_scale, r.w, r.keys, r.k_scale, np.arange(npg), P, r.n)
                for h in range(T.shape[1]):
                    _block_check(T[:, h], r.n, bs, top, t["bt_rows"][idx], t["blocks"][idx][h],
                                 None if t["slots"] is None else t["slots"][idx][h])
            else:
                S, r = _row_scores(t["spec"], int(b), P)
                _block_check(S, r.n, bs, top, t["bt_rows"][idx], t["blocks"][idx],
                             None if t["slots"] is None else t["slots"][idx])
        except AssertionError as e:
            fails.append((int(b), str(e)[:200]))
    return _result(fails, len(t["rows"]))


def block_tasks(case, blocks, slots, per_head=False, per_task=4):
    spec = workloads.row_spec(case)
    r2b = case.row_to_batch
    for i0 in range(0, case.batch, per_task):
        rr = np.arange(i0, min(case.batch, i0 + per_task))
        prow = rr if r2b is None else r2b[rr]
        yield {"spec": spec, "page_size": case.page_size, "bs": case.block_size, "top": case.top_blocks,
               "rows": rr, "bt_rows": case.block_table[prow], "blocks": blocks[rr],
               "slots": None if slots is None else slots[rr], "per_head": per_head}
