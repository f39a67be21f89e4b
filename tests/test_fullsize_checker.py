"""The every-row checker of the full-size parity tests (tests/_fullsize.py),
on the CPU: the oracle's own outputs pass, and a planted mistake in the
checked outputs is reported for exactly the row that holds it."""
import numpy as np

import oracle
import workloads
from tests import _fullsize


def _fails(r):
    return sorted({row for row, _ in r["fails"]})


def test_packed_rows_checker():
    case = workloads.packed_prefill_case(seed=91, prefix0=1500, new_tokens=48, k=32)
    ref = oracle.topk_rows(case.scores, case.seq_lens, case.k, case.row_starts, case.row_to_batch,
                           case.page_table, 1)
    task = lambda got, srt: next(iter(_fullsize.packed_tasks(case, got, srt, per_task=case.rows, seed=91)))
    r = _fullsize.packed_rows_task(task(ref, ref))
    assert r["rows"] == case.rows and r["fails"] == []
    # order within a row does not matter for the set check
    assert _fullsize.packed_rows_task(task(ref[:, ::-1].copy(), None))["fails"] == []
    bad = ref.copy()
    row = 50  # request 0's row 50 (n = 1551 > k)
    unsel = np.setdiff1d(case.page_table[0], bad[row])[0]
    bad[row, 3] = unsel
    assert _fails(_fullsize.packed_rows_task(task(bad, None))) == [row]
    srt = ref.copy()
    srt[7, [0, 1]] = srt[7, [1, 0]]
    assert _fails(_fullsize.packed_rows_task(task(ref, srt))) == [7]


def test_fused_rows_checker():
    case = workloads.indexer_case(92, batch=4, n_lo=300, n_hi=3000, page_size=16, k=200, heads=16)
    slots, pos, scores = oracle.fused_topk(case)
    sc = np.stack([np.where(p >= 0, S[np.maximum(p, 0)], -np.inf) for p, S in zip(pos, scores)]).astype(np.float32)
    tasks = list(_fullsize.fused_tasks(case, slots, sc, per_task=2))
    assert all(_fullsize.fused_rows_task(t)["fails"] == [] for t in tasks)
    # the worst unselected token in place of a selected one
    b = 2
    n = int(case.seq_lens[b])
    worst = int(np.argmin(scores[b]))
    bad = slots.copy()
    bad[b, 0] = oracle.token_slots(case.block_table[b], case.page_size, n)[worst]
    assert _fails(_fullsize.fused_rows_task(next(iter(_fullsize.fused_tasks(case, bad, None, per_task=4))))) == [b]
    # a score off by more than the tolerance
    bad_sc = sc.copy()
    bad_sc[1, 5] *= 1.01
    assert _fails(_fullsize.fused_rows_task(next(iter(_fullsize.fused_tasks(case, slots, bad_sc, per_task=4))))) \
        == [1]
    # unfused scores checked as well
    gpu = lambda rr: [scores[i].astype(np.float32) for i in rr]
    assert _fullsize.fused_rows_task(next(iter(_fullsize.fused_tasks(case, slots, None, per_task=4,
                                                                     gpu_scores=gpu))))["fails"] == []


def test_fused_rows_checker_multi_query_and_bf16():
    mq = workloads.multi_query_case(93, requests=2, next_n=3, n_lo=500, n_hi=2500, page_size=64, k=100, heads=16)
    slots, _, _ = oracle.fused_topk(mq)
    assert _fullsize.fused_rows_task(next(iter(_fullsize.fused_tasks(mq, slots, per_task=6))))["fails"] == []
    bf = workloads.indexer_case(94, batch=2, n_lo=500, n_hi=2500, page_size=64, k=100, heads=16,
                                cache_dtype="bf16")
    slots, _, _ = oracle.fused_topk(bf)
    assert _fullsize.fused_rows_task(next(iter(_fullsize.fused_tasks(bf, slots, per_task=2))))["fails"] == []


def test_block_rows_checker():
    case = workloads.indexer_case(95, batch=3, n_lo=900, n_hi=3000, page_size=64, k=0, heads=16, block_size=64,
                                  top_blocks=5, fixed_lens=np.array([0, 1000, 3000], np.int32))
    blocks, slots, _, _ = oracle.block_topk(case)
    task = lambda bl, sl, ph=False: next(iter(_fullsize.block_tasks(case, bl, sl, per_head=ph, per_task=3)))
    assert _fullsize.block_rows_task(task(blocks, slots))["fails"] == []
    bad = slots.copy()
    bad[2, 64 * 2 + 7] += 1
    assert _fails(_fullsize.block_rows_task(task(blocks, bad))) == [2]
    hb, hs = oracle.block_topk_heads(case)
    assert _fullsize.block_rows_task(task(hb, hs, True))["fails"] == []
    bad = hb.copy()
    bad[1, 3, [0, 1]] = bad[1, 3, [1, 1]]
    assert _fails(_fullsize.block_rows_task(task(bad, hs, True))) == [1]
