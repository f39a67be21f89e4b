"""GPU parity of idx_score_topk_prefill (fused prefill indexer) against the
oracle and against the unfused path (idx_score_fp8 + topk_rows)."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.indexer import case_scores
from tests._helpers import check_fused_row, dev, log, rms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    from sparse_attention_indexer_fp8_amd import ops as _ops

    torch.cuda.set_device(0)
    return _ops


def _inputs(case):
    return (dev(case.q), dev(case.q_scale), dev(case.w), dev(case.kcache), dev(case.k_scale),
            dev(case.block_table), dev(case.seq_lens))


def _prefill(ops, case, k=None, sorted_out=False, ws=None):
    import torch

    slots, sc = ops.idx_score_topk_prefill(*_inputs(case), case.page_size, case.max_seq_len,
                                           case.k if k is None else k, return_scores=True, workspace=ws,
                                           row_to_batch=dev(case.row_to_batch), sorted=sorted_out)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), sc.cpu().numpy()


def _unfused(ops, case, k=None):
    """The unfused path on the same inputs: the score rows, then topk_rows
    through the block table (slots, and the score rows on the host)."""
    import torch

    r2b = dev(case.row_to_batch)
    scores = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len, row_to_batch=r2b)
    slots = ops.topk_rows(scores, dev(case.seq_lens), case.k if k is None else k, row_to_batch=r2b,
                          page_table=dev(case.block_table), page_size=case.page_size)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), scores


def _prefill_case(seed, requests, next_n, n_lo, n_hi, page_size, k, heads=64, lens=None):
    """Packed prefill rows: request r extends its context by next_n tokens,
    its query rows see causal lengths L_r - next_n + 1 .. L_r."""
    return workloads.multi_query_case(seed, requests=requests, next_n=next_n, n_lo=n_lo, n_hi=n_hi,
                                      page_size=page_size, k=k, heads=heads, name="prefill-test", fixed_lens=lens)


def _exactify(case, seed):
    """Codes of +-0.5, +-1, +-2 and 0, unit scales, power-of-two weights:
    every product and partial sum is a multiple of 1/4 below 2^10, so the
    GPU's fp32 scores equal the oracle's float64 ones and the selected sets
    must agree exactly, ties included."""
    g = np.random.default_rng(seed + 1000)
    codes = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)
    case.q[:] = g.choice(codes, size=case.q.shape)
    case.q_scale[:] = 1.0
    case.w[:] = g.choice(np.array([0.5, 1.0, 2.0, -1.0], np.float32), size=case.w.shape)
    real = case.k_scale < workloads.SENTINEL_KEY_SCALE
    case.kcache[real] = g.choice(codes, size=(int(real.sum()), case.dim))
    case.k_scale[real] = 1.0
    return case


def _check_exact(case, slots, sc, k, sorted_out=False):
    ref_slots, ref_pos, scores = oracle.fused_topk(case, k=k)
    for b in range(case.batch):
        if sorted_out:
            assert np.array_equal(slots[b], ref_slots[b]), b
        else:
            assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), b
        m = min(int(case.seq_lens[b]), k)
        assert np.array_equal(np.sort(sc[b][:m].astype(np.float64)), np.sort(scores[b][ref_pos[b][:m]])), b
        assert (sc[b][m:] == -np.inf).all(), b


# requests x next_n rows; next_n not a multiple of 4 puts quads across two
# requests (rows scored in pairs or alone); lens include rows shorter than k
@pytest.mark.parametrize("heads,page_size,k,requests,next_n,n_hi", [
    (64, 64, 512, 3, 200, 12000),
    (16, 16, 100, 5, 7, 9000),
    (32, 128, 2048, 4, 5, 30000),
    (64, 32, 300, 9, 2, 20000),
    (64, 64, 1, 2, 33, 5000),
    (16, 48, 700, 3, 64, 3000),
])
def test_prefill_exact_sets(ops, heads, page_size, k, requests, next_n, n_hi):
    case = _exactify(_prefill_case(700 + k + page_size, requests, next_n, 1, n_hi, page_size, k, heads), 700 + k)
    log(f"prefill exact: rows={case.batch} heads={heads} P={page_size} k={k} max n={case.max_seq_len}")
    slots, sc = _prefill(ops, case)
    _check_exact(case, slots, sc, k)


@pytest.mark.parametrize("page_size,k,requests,next_n,n_lo,n_hi", [
    (64, 512, 2, 300, 20000, 70000),
    (16, 256, 3, 50, 1, 20000),
    (128, 2048, 2, 40, 30000, 90000),
])
def test_prefill_equals_unfused(ops, page_size, k, requests, next_n, n_lo, n_hi):
    """Random fp8 inputs: the fused selection equals the unfused path's
    exactly (both score with the same fp32 arithmetic and break ties by
    position), and the returned scores equal the score rows."""
    import torch

    case = _prefill_case(720 + page_size, requests, next_n, n_lo, n_hi, page_size, k)
    log(f"prefill vs unfused: rows={case.batch} P={page_size} k={k} max n={case.max_seq_len}")
    slots, sc = _prefill(ops, case)
    ref, scores = _unfused(ops, case)
    assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))
    host = scores.cpu().numpy()
    del scores
    torch.cuda.empty_cache()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        m = min(n, k)
        assert np.array_equal(np.sort(sc[b][:m]), np.sort(host[b, :n])[::-1][:m][::-1]), b
    rows = [0, case.batch // 2, case.batch - 1]
    bsig = rms(np.concatenate([case_scores(case, b) for b in rows]))
    for b in rows:
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[case.row_to_batch[b]], case.page_size, n)
        check_fused_row(slots[b], sc[b], case_scores(case, b), ts, k, batch_sigma=bsig)


def _crowded(case):
    """Exact-arithmetic rows whose best tokens all sit at the end of the
    context: query 1.0 in every dimension, only head 0 weighted (1.0), unit
    scales, and token j's key holds 1.0 in its first m_j = 1 + 127 j // L
    dimensions (L the request's context), so S[j] = m_j grows with the
    position (ties in runs). The last chunks of a long row hold its whole top
    k, so the sampled bounds there lie above the row's k-th value and the
    row is scored again in full."""
    case.q[:] = 0x38
    case.q_scale[:] = 1.0
    case.w[:] = 0.0
    case.w[:, 0] = 1.0
    for r in range(case.block_table.shape[0]):
        L = int(case.seq_lens[case.row_to_batch == r].max())
        ts = oracle.token_slots(case.block_table[r], case.page_size, L)
        m = 1 + (127 * np.arange(L)) // max(L, 1)
        case.kcache[ts] = np.where(np.arange(case.dim)[None, :] < m[:, None], 0x38, 0x00).astype(np.uint8)
        case.k_scale[ts] = 1.0
    return case


@pytest.mark.parametrize("requests,next_n", [(4, 64), (5, 52), (8, 33), (7, 39)])
def test_prefill_schedule_boundary(ops, requests, next_n):
    """Around the switch between the two chunk schedules: 64 row quads
    (256 rows: the balanced schedule, chunk sizes taken on the device from
    the rows' lengths), 65 quads (260 rows: the chunk-major grid, two rows
    per wave), 66 quads whose row pairs straddle requests, and 273 rows (an
    odd count: the last pair wave holds one row). Each equals the unfused
    path's selection exactly, with the returned scores equal to the score
    rows."""
    import torch

    case = _prefill_case(760 + requests, requests, next_n, 1, 6000, 64, 300)
    log(f"prefill schedule boundary: rows={case.batch} quads={(case.batch + 3) // 4}")
    slots, sc = _prefill(ops, case)
    ref, scores = _unfused(ops, case)
    assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))
    host = scores.cpu().numpy()
    del scores
    torch.cuda.empty_cache()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        m = min(n, case.k)
        assert np.array_equal(np.sort(sc[b][:m]), np.sort(host[b, :n])[::-1][:m][::-1]), b


@pytest.mark.parametrize("sorted_out", [False, True])
@pytest.mark.parametrize("page_size,k,n_hi", [(64, 512, 30000), (16, 300, 9000), (128, 2048, 40000)])
def test_prefill_rows_rescored(ops, page_size, k, n_hi, sorted_out):
    """Rows whose top k crowd into their last chunks: the merge queues them
    and the fallback scores them again; the result is the oracle's exact
    selection (and order, when sorted)."""
    case = _crowded(_prefill_case(740 + page_size, 3, 9, n_hi // 2, n_hi, page_size, k, heads=16))
    log(f"prefill crowded: rows={case.batch} P={page_size} k={k} sorted={sorted_out}")
    slots, sc = _prefill(ops, case, sorted_out=sorted_out)
    _check_exact(case, slots, sc, k, sorted_out)


def test_prefill_all_scores_tied(ops):
    """Every key is the same vector: all scores of a row tie, each chunk
    keeps its whole range (more candidates than the list holds for the long
    rows), and the k lowest positions are selected."""
    case = _exactify(_prefill_case(760, 2, 6, 3000, 12000, 64, 300, heads=16), 760)
    real = case.k_scale < workloads.SENTINEL_KEY_SCALE
    case.kcache[real] = case.kcache[real][0]
    slots, sc = _prefill(ops, case)
    ref_slots, ref_pos, _ = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(ref_pos[b]), np.arange(case.k)), b
        assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), b


@pytest.mark.parametrize("k", [64, 512, 2048])
def test_prefill_sorted_exact_order(ops, k):
    case = _exactify(_prefill_case(780 + k, 3, 40, 1, 15000, 64, k), 780 + k)
    case.seq_lens[:3] = [0, k - 1, k]
    slots, sc = _prefill(ops, case, sorted_out=True)
    _check_exact(case, slots, sc, k, sorted_out=True)


def test_prefill_dirty_workspace_and_reuse(ops):
    """The workspace needs no particular contents: a buffer of 0xFF bytes,
    then the same buffer again with a smaller call, give the oracle's exact
    results."""
    import torch

    from sparse_attention_indexer_fp8_amd import ops as o

    big = _exactify(_prefill_case(800, 3, 30, 5000, 20000, 64, 512), 800)
    small = _exactify(_prefill_case(801, 2, 9, 100, 3000, 16, 100, heads=32), 801)
    ws = o.Workspace()
    nbytes = o.workspace_bytes(o._lib.OP_SCORE_TOPK_PREFILL, big.batch, big.k, big.max_seq_len)
    ws.get(nbytes).fill_(0xFF)
    torch.cuda.synchronize()
    for case in (big, small):
        slots, sc = _prefill(ops, case, ws=ws)
        _check_exact(case, slots, sc, case.k)


@pytest.mark.timeout(900)
def test_prefill_fused_full_size(ops):
    """The prefill workload at full size (16384 rows, contexts 70000 and
    8192, k 512) through the fused call the benchmark times: every row
    equals the unfused path's selection exactly, and every row meets the
    oracle criterion in the oracle pool (scores within the tolerance)."""
    import torch

    from tests import _fullsize

    case = workloads.prefill_indexer()
    log(f"prefill fused full size: rows={case.batch} max n={case.max_seq_len}")
    slots, sc = _prefill(ops, case)
    ref, scores = _unfused(ops, case)
    del scores
    torch.cuda.empty_cache()
    same = np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))
    log(f"fused equals unfused on every row: {same}")
    assert same

    def tasks():
        yield from _fullsize.fused_tasks(case, slots, sc, rows=np.arange(0, 8192), per_task=32)
        yield from _fullsize.fused_tasks(case, slots, sc, rows=np.arange(8192, case.batch), per_task=512)

    n = _fullsize.run(_fullsize.fused_rows_task, tasks(), case.name + " fused")
    assert n == case.batch


@pytest.mark.timeout(600)
def test_prefill_call_on_multi_token_decode_full_size(ops):
    """The multi-token decode workload (16 requests x 4 query rows, contexts
    16K..64K, k 2048) through the row-group call, as the benchmark times it
    (small chunks: few row quads): every row against the oracle criterion,
    and the same selection as the per-row fused call (same fp32 scores)."""
    from tests import _fullsize

    case = workloads.mtp_decode()
    log(f"mtp through the row-group call: rows={case.batch} max n={case.max_seq_len}")
    slots, sc = _prefill(ops, case)
    import torch

    ref, _ = ops.idx_score_topk_fused(*_inputs(case), case.page_size, case.max_seq_len, case.k, return_scores=True,
                                      row_to_batch=dev(case.row_to_batch))
    torch.cuda.synchronize()
    assert np.array_equal(np.sort(slots, axis=1), np.sort(ref.cpu().numpy(), axis=1))
    n = _fullsize.run(_fullsize.fused_rows_task, _fullsize.fused_tasks(case, slots, sc), case.name + " row-group")
    assert n == case.batch


def test_prefill_edge_shapes(ops):
    """Shapes at the edges of the row-group call, each against the oracle's
    exact selection on exact inputs: every row empty; max_seq_len 0; no
    row_to_batch (each row its own block-table row: rows scored one at a
    time); a batch that is not a multiple of four; k above every row's
    length; a single row."""
    import torch

    base = _exactify(_prefill_case(820, 3, 7, 1, 5000, 64, 300, heads=16), 820)

    def run(case, k, r2b=True):
        slots, sc = ops.idx_score_topk_prefill(*_inputs(case), case.page_size, case.max_seq_len, k,
                                               return_scores=True,
                                               row_to_batch=dev(case.row_to_batch) if r2b else None)
        torch.cuda.synchronize()
        return slots.cpu().numpy(), sc.cpu().numpy()

    # every row empty (max_seq_len kept), then max_seq_len 0
    import copy

    empty = copy.copy(base)
    empty.seq_lens = np.zeros_like(base.seq_lens)
    for msl in (base.max_seq_len, 0):
        empty.max_seq_len = msl
        slots, sc = run(empty, 300)
        assert (slots == -1).all() and (sc == -np.inf).all(), msl
    # no row_to_batch: the block table expanded to one row per query row
    flat = copy.copy(base)
    flat.block_table = np.ascontiguousarray(base.block_table[base.row_to_batch])
    flat.row_to_batch = np.arange(base.batch, dtype=np.int32)
    slots, sc = run(flat, 300, r2b=False)
    _check_exact(flat, slots, sc, 300)
    # 21 rows (not a multiple of 4), one row, and k above every length
    short = _exactify(_prefill_case(821, 3, 7, 1, 1500, 64, 2048, heads=16), 821)
    for case, rows, k in ((base, base.batch, 300), (base, 1, 300), (short, short.batch, 2048)):
        part = copy.copy(case)
        part.q, part.q_scale, part.w = case.q[:rows], case.q_scale[:rows], case.w[:rows]
        part.seq_lens, part.row_to_batch = case.seq_lens[:rows], case.row_to_batch[:rows]
        slots, sc = run(part, k)
        _check_exact(part, slots, sc, k)
