"""GPU parity of idx_score_fp8, idx_score_topk_fused and block_topk against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.indexer import case_scores
from tests._helpers import check_fused_row, check_scores, dev, log, rms

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


def _r2b(case):
    r2b = getattr(case, "row_to_batch", None)
    return None if r2b is None else dev(r2b)


def _fused(ops, case, k=None, ws=None):
    import torch

    slots, sc = ops.idx_score_topk_fused(*_inputs(case), case.page_size, case.max_seq_len,
                                         case.k if k is None else k, return_scores=True, workspace=ws,
                                         row_to_batch=_r2b(case))
    torch.cuda.synchronize()
    return slots.cpu().numpy(), sc.cpu().numpy()


def _lens(seed, batch, n_lo, n_hi, first=()):
    lens = workloads.rng(seed, workloads.synth.STREAM_LEN).integers(n_lo, n_hi + 1, size=batch).astype(np.int32)
    lens[:len(first)] = first
    return lens


def _exact_case(seed, batch, n_lo, n_hi, page_size, heads=16, k=64, first=(), **kw):
    """Inputs whose fp32 scores are exact: codes of +-0.5, +-1, +-2 and 0, unit
    scales, power-of-two weights. Every product and partial sum is a multiple of
    1/4 below 2^10, so the GPU's fp32 scores equal the oracle's float64 ones
    and the selected sets must agree exactly, ties included."""
    case = workloads.indexer_case(seed, batch=batch, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k,
                                  heads=heads, fixed_lens=_lens(seed, batch, n_lo, n_hi, first), **kw)
    g = np.random.default_rng(seed + 1000)
    codes = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)
    case.q[:] = g.choice(codes, size=case.q.shape)
    case.q_scale[:] = 1.0
    case.w[:] = g.choice(np.array([0.5, 1.0, 2.0, -1.0], np.float32), size=case.w.shape)
    real = case.k_scale < workloads.SENTINEL_KEY_SCALE
    case.kcache[real] = g.choice(codes, size=(int(real.sum()), case.dim))
    case.k_scale[real] = 1.0
    return case


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("page_size", [1, 16, 48, 64])
def test_score_tolerance(ops, heads, page_size):
    import torch

    seed = 200 + heads + page_size
    case = workloads.indexer_case(seed, batch=3, n_lo=1, n_hi=3000, page_size=page_size, k=64, heads=heads,
                                  fixed_lens=_lens(seed, 3, 1, 3000, first=(1,)))
    out = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        check_scores(out[b, :n], rows[b], bsig)
        assert np.isnan(out[b, n:]).all(), "cells past n_b must stay untouched"


def test_score_exact_values(ops):
    import torch

    case = _exact_case(301, batch=2, n_lo=500, n_hi=2000, page_size=64)
    out = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        assert np.array_equal(out[b, :n].astype(np.float64), case_scores(case, b))


@pytest.mark.parametrize("page_size,heads,k", [(64, 64, 64), (16, 16, 200), (1, 32, 300), (48, 64, 1000),
                                               (128, 128, 100)])
def test_fused_exact_sets(ops, page_size, heads, k):
    """Exact arithmetic: the fused selection equals the oracle's set exactly
    (heavy ties are resolved toward the lower position)."""
    case = _exact_case(400 + page_size, batch=5, n_lo=1, n_hi=12000, page_size=page_size, heads=heads, k=k,
                       first=(0, k - 1, k))
    slots, sc = _fused(ops, case)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), b
        m = min(int(case.seq_lens[b]), k)
        got_s = np.sort(sc[b][:m].astype(np.float64))
        exp_s = np.sort(scores[b][ref_pos[b][:m]]) if m else np.zeros(0)
        assert np.array_equal(got_s, exp_s)


@pytest.mark.parametrize("page_size,k,n_lo,n_hi", [(64, 2048, 1, 20000), (64, 256, 3000, 40000),
                                                   (16, 512, 100, 9000), (100, 64, 1, 500)])
def test_fused_tolerance_random(ops, page_size, k, n_lo, n_hi):
    case = workloads.indexer_case(500 + k, batch=6, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k)
    slots, sc = _fused(ops, case)
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[b], case.page_size, n)
        ov = check_fused_row(slots[b], sc[b], rows[b], ts, k, batch_sigma=bsig)
        log(f"row {b} n={n} overlap={ov:.4f}")


def test_fused_workspace_reuse_smaller_second_call(ops):
    """Calls sharing one workspace do not depend on what an earlier call left
    in it: a second call with a smaller input is exact."""
    from sparse_attention_indexer_fp8_amd import ops as o

    ws = o.Workspace()
    big = _exact_case(601, batch=8, n_lo=5000, n_hi=30000, page_size=64, k=500)
    small = _exact_case(602, batch=3, n_lo=100, n_hi=3000, page_size=64, k=500)
    for case in (big, small, big):
        slots, _ = _fused(ops, case, ws=ws)
        ref, _, _ = oracle.fused_topk(case)
        assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))


def test_default_workspace_per_stream(ops):
    """Fused and block calls made on two streams at once with default
    workspaces get one workspace per stream: both results stay exact."""
    import torch

    fa = _exact_case(611, batch=6, n_lo=3000, n_hi=20000, page_size=64, k=700)
    fb = _exact_case(612, batch=5, n_lo=2000, n_hi=18000, page_size=64, k=300)
    ba = _exact_case(613, batch=6, n_lo=3000, n_hi=9000, page_size=128, k=0, block_size=128, top_blocks=9)
    ref_a, _, _ = oracle.fused_topk(fa)
    ref_b, _, _ = oracle.fused_topk(fb)
    ref_blk = oracle.block_topk(ba)
    ins = {id(c): _inputs(c) for c in (fa, fb, ba)}
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            oa = ops.idx_score_topk_fused(*ins[id(fa)], fa.page_size, fa.max_seq_len, fa.k)
            ob = ops.block_topk(*ins[id(ba)], ba.page_size, ba.max_seq_len, ba.block_size, ba.top_blocks,
                                return_slots=False)
        with torch.cuda.stream(s2):
            oc = ops.idx_score_topk_fused(*ins[id(fb)], fb.page_size, fb.max_seq_len, fb.k)
            od = ops.block_topk(*ins[id(ba)], ba.page_size, ba.max_seq_len, ba.block_size, ba.top_blocks,
                                return_slots=False)
        outs.append((oa, ob, oc, od))
    torch.cuda.synchronize()
    keys = {k for k in ops._default_ws if k[1] in (s1.cuda_stream, s2.cuda_stream)}
    assert len(keys) == 2, "one default workspace per stream"
    for oa, ob, oc, od in outs:
        assert np.array_equal(np.sort(oa.cpu().numpy(), axis=1), np.sort(ref_a, axis=1))
        assert np.array_equal(np.sort(oc.cpu().numpy(), axis=1), np.sort(ref_b, axis=1))
        for o in (ob, od):
            assert np.array_equal(np.sort(o.cpu().numpy(), axis=1), np.sort(ref_blk[0], axis=1))


# Batches of more than this many tokens never fit one resident wave of the
# fused path's chunk workgroups (at most 8192 tokens each, at most 8 per
# compute unit on 256 units): they take the guided chunk schedule
FUSED_GUIDED_TOKENS = 1 << 24


def _guided_variant(case):
    """The same case with a max_seq_len (an upper bound on every row length)
    large enough to send it down the guided chunk schedule. The block table gets
    zero columns so it covers that bound, as the API requires; no row reads
    them."""
    import copy

    big = copy.copy(case)
    big.max_seq_len = FUSED_GUIDED_TOKENS // case.batch + 1
    cols = -(-big.max_seq_len // case.page_size)
    bt = np.zeros((case.block_table.shape[0], cols), np.int32)
    bt[:, :case.block_table.shape[1]] = case.block_table
    big.block_table = bt
    return big


@pytest.mark.parametrize("page_size,heads,k", [(64, 64, 2048), (16, 32, 300), (1, 16, 100)])
def test_fused_both_variants_exact(ops, page_size, heads, k):
    """Both chunk schedules of the fused path (resident chunks and the guided
    schedule) select the oracle's exact set on the same inputs."""
    case = _exact_case(450 + page_size, batch=6, n_lo=1, n_hi=16000, page_size=page_size, heads=heads, k=k,
                       first=(0, k - 1, k, 16000))
    assert case.batch * case.max_seq_len <= FUSED_GUIDED_TOKENS
    ref_slots, _, _ = oracle.fused_topk(case)
    big = _guided_variant(case)
    for c in (case, big):
        log(f"fused variant check: batch={c.batch} max_seq_len={c.max_seq_len} k={k} page_size={page_size}")
        slots, _ = _fused(ops, c)
        for b in range(case.batch):
            assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), (c.max_seq_len, b)


def test_fused_workspace_reuse_across_variants(ops):
    """Calls of both chunk schedules share one workspace in any order."""
    from sparse_attention_indexer_fp8_amd import ops as o

    ws = o.Workspace()
    a = _exact_case(611, batch=4, n_lo=3000, n_hi=20000, page_size=64, k=700)
    b = _exact_case(612, batch=3, n_lo=100, n_hi=5000, page_size=16, k=300)
    a_big = _guided_variant(a)
    for case in (a, a_big, b, a_big, a):
        slots, _ = _fused(ops, case, ws=ws)
        ref, _, _ = oracle.fused_topk(case)
        assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))


def test_fused_all_scores_tied(ops):
    """Every key of a row is the same vector, so all its scores tie and the
    threshold bin holds the whole row (more keys than the merge buffers):
    the k lowest positions are selected."""
    case = _exact_case(620, batch=3, n_lo=9000, n_hi=12000, page_size=64, k=1500, first=(12000, 5000))
    real = case.k_scale < workloads.SENTINEL_KEY_SCALE
    case.kcache[real] = case.kcache[real][0]
    ref_slots, ref_pos, _ = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(ref_pos[b]), np.arange(case.k)), b
    for c in (case, _guided_variant(case)):
        slots, _ = _fused(ops, c)
        for b in range(case.batch):
            assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), (c.max_seq_len, b)


def _crowded_case(seed, batch, n_lo, n_hi, page_size, k, heads=16):
    """Exact-arithmetic rows whose best tokens all sit at the end of the row:
    query 1.0 in every dimension, only head 0 weighted (1.0), unit scales,
    and token j's key holds 1.0 in its first m_j = 1 + 127 j // n dimensions
    and 0 elsewhere, so S[j] = m_j grows with the position (ties in runs).
    The chunks at the end of a row hold its whole top k, far more than their
    share, so the merge's check fails and it scores the row again."""
    case = workloads.indexer_case(seed, batch=batch, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k, heads=heads,
                                  fixed_lens=_lens(seed, batch, n_lo, n_hi))
    case.q[:] = 0x38
    case.q_scale[:] = 1.0
    case.w[:] = 0.0
    case.w[:, 0] = 1.0
    for b in range(batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[b], case.page_size, n)
        m = 1 + (127 * np.arange(n)) // max(n, 1)
        keys = np.where(np.arange(case.dim)[None, :] < m[:, None], 0x38, 0x00).astype(np.uint8)
        case.kcache[ts] = keys
        case.k_scale[ts] = 1.0
    return case


@pytest.mark.parametrize("batch,n,k", [(16, 16384, 2048), (12, 30000, 2048)])
def test_fused_exact_many_chunks(ops, batch, n, k):
    """Exact arithmetic on rows of 32 to 64 chunks with more than 4096
    candidates each: the merge adds the chunks' candidate-count windows to
    its histogram instead of counting every candidate; the sets and scores
    equal the oracle's exactly (ties by position included)."""
    case = _exact_case(660 + batch, batch=batch, n_lo=n, n_hi=n, page_size=64, heads=64, k=k)
    slots, sc = _fused(ops, case)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), b
        assert np.array_equal(np.sort(sc[b].astype(np.float64)), np.sort(scores[b][ref_pos[b]])), b


def _tied_case(seed, batch, n, page_size, k, top, tied, heads=64):
    """Exact-arithmetic rows of n tokens with integer scores S[j] = m_j (query
    1.0 in every dimension, only head 0 weighted, unit scales, key j holding
    1.0 in its first m_j dimensions): `top` tokens at random positions score
    60..127, `tied` others score exactly 50, and the rest 0..45. The value 50
    is alone in its histogram bin and in its sub-bin."""
    case = workloads.indexer_case(seed, batch=batch, n_lo=n, n_hi=n, page_size=page_size, k=k, heads=heads,
                                  fixed_lens=np.full(batch, n, np.int32))
    case.q[:] = 0x38
    case.q_scale[:] = 1.0
    case.w[:] = 0.0
    case.w[:, 0] = 1.0
    g = np.random.default_rng(seed + 7)
    for b in range(batch):
        m = g.integers(0, 46, size=n)
        perm = g.permutation(n)
        m[perm[:top]] = g.integers(60, 128, size=top)
        m[perm[top:top + tied]] = 50
        ts = oracle.token_slots(case.block_table[b], case.page_size, n)
        case.kcache[ts] = np.where(np.arange(case.dim)[None, :] < m[:, None], 0x38, 0x00).astype(np.uint8)
        case.k_scale[ts] = 1.0
    return case


@pytest.mark.parametrize("top,tied,k", [(50, 50, 100), (50, 40, 70), (50, 300, 100), (50, 1500, 100),
                                        (50, 3000, 100)])
def test_fused_threshold_bin_ties(ops, top, tied, k):
    """The row's k-th score is shared by `tied` tokens, so the merge's
    threshold bin (and its sub-bin) holds exactly those: all of them are
    taken (k = top + tied), a few (at most 64) are ranked against each
    other, more go through the workgroup select over the sub-bin's keys
    (threshold bins of up to 2048 keys held in LDS), and beyond that the
    merge selects from the candidates themselves. Ties go to the lower
    positions, exactly as the oracle takes them, on both chunk schedules."""
    case = _tied_case(640 + tied, batch=3, n=6000, page_size=64, k=k, top=top, tied=tied)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.sum(scores[b][ref_pos[b]] == 50.0) == k - top, b
    for c in (case, _guided_variant(case)):
        slots, sc = _fused(ops, c)
        for b in range(case.batch):
            assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), (c.max_seq_len, b)
            assert np.array_equal(np.sort(sc[b].astype(np.float64)), np.sort(scores[b][ref_pos[b]])), b


@pytest.mark.parametrize("sorted_out", [False, True])
@pytest.mark.parametrize("page_size,k,n_lo,n_hi", [(64, 2048, 6000, 30000), (16, 300, 400, 9000),
                                                   (1, 100, 150, 4000)])
def test_fused_crowded_rows_rescored(ops, page_size, k, n_lo, n_hi, sorted_out):
    """Rows whose top k crowd into their last chunks (far beyond the chunks'
    margin): the merge scores them again and the result is still the
    oracle's exact selection, on both chunk schedules."""
    import torch

    case = _crowded_case(660 + page_size, batch=5, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for c in (case, _guided_variant(case)):
        log(f"crowded rows: max_seq_len={c.max_seq_len} k={k} page_size={page_size} sorted={sorted_out}")
        slots, sc = ops.idx_score_topk_fused(*_inputs(c), c.page_size, c.max_seq_len, k, return_scores=True,
                                             sorted=sorted_out)
        torch.cuda.synchronize()
        slots, sc = slots.cpu().numpy(), sc.cpu().numpy()
        for b in range(case.batch):
            if sorted_out:
                assert np.array_equal(slots[b], ref_slots[b]), b
            else:
                assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), b
            m = min(int(case.seq_lens[b]), k)
            assert np.array_equal(np.sort(sc[b][:m].astype(np.float64)), np.sort(scores[b][ref_pos[b][:m]])), b


def test_fused_dirty_workspace(ops):
    """The fused and block ops need no particular workspace contents: a
    workspace filled with 0xFF bytes gives the oracle's exact results."""
    import torch

    from sparse_attention_indexer_fp8_amd import ops as o

    fc = _exact_case(670, batch=5, n_lo=1, n_hi=20000, page_size=64, k=700, first=(0, 699, 700))
    bc = _exact_case(671, batch=4, n_lo=1, n_hi=9000, page_size=128, k=0, block_size=128, top_blocks=7,
                     first=(0, 128 * 7))
    for c, op in ((fc, "fused"), (_guided_variant(fc), "fused"), (bc, "block")):
        ws = o.Workspace()
        if op == "fused":
            buf = ws.get(ops.workspace_bytes(o._lib.OP_SCORE_TOPK_FUSED, c.batch, c.k, c.max_seq_len))
        else:
            buf = ws.get(ops.workspace_bytes(o._lib.OP_BLOCK_TOPK, c.batch, c.block_size, c.max_seq_len))
        buf.fill_(0xFF)
        if op == "fused":
            slots, _ = _fused(ops, c, ws=ws)
            ref, _, _ = oracle.fused_topk(c)
            assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))
        else:
            blocks, sl = ops.block_topk(*_inputs(c), c.page_size, c.max_seq_len, c.block_size, c.top_blocks,
                                        workspace=ws)
            torch.cuda.synchronize()
            rb, rs, _, _ = oracle.block_topk(c)
            assert np.array_equal(np.sort(blocks.cpu().numpy(), axis=1), np.sort(rb, axis=1))


@pytest.mark.parametrize("page_size,k,n_lo,n_hi,batch", [(64, 2048, 1, 20000, 6), (16, 300, 100, 9000, 5),
                                                         (1, 64, 1, 3000, 4), (16, 64, 0, 700, 300),
                                                         (64, 100, 0, 3000, 40)])
def test_fused_equals_unfused(ops, page_size, k, n_lo, n_hi, batch):
    """idx_score_fp8 then topk_rows through the block table (the unfused
    path) computes the same fp32 score per token as the fused kernels, so
    both chunk schedules of the fused path (chunks sized for one resident
    wave of workgroups, and the guided schedule of the large max_seq_len
    variant) select exactly its set, ties included, also for batches with
    empty rows and a batch of 300 short rows."""
    import torch

    case = workloads.indexer_case(800 + k, batch=batch, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k)
    scores = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len)
    ref = ops.topk_rows(scores, dev(case.seq_lens), k, page_table=dev(case.block_table), page_size=page_size)
    torch.cuda.synchronize()
    ref = np.sort(ref.cpu().numpy(), axis=1)
    for c in (case, _guided_variant(case)):
        slots, _ = _fused(ops, c)
        assert np.array_equal(np.sort(slots, axis=1), ref), c.max_seq_len


def test_fused_never_reads_outside_windows(ops):
    """Sentinel keys (+448, scale 1e3) fill every slot no row owns; selecting
    one of them would map to no token of the row and fail the inverse map."""
    case = workloads.indexer_case(701, batch=4, n_lo=1, n_hi=700, page_size=64, k=128)
    slots, sc = _fused(ops, case)
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[b], case.page_size, n)
        check_fused_row(slots[b], sc[b], rows[b], ts, case.k, batch_sigma=bsig)


# (the wave merge for most; the last two cases take the workgroup merge: more
# than 256 kept blocks, more than 1024 blocks per row)
@pytest.mark.parametrize("bs,top,n_hi", [(128, 32, 9000), (64, 5, 9000), (16, 40, 9000), (16, 300, 9000),
                                         (16, 40, 20000)])
def test_block_exact(ops, bs, top, n_hi):
    import torch

    case = _exact_case(800 + bs + top, batch=5, n_lo=1, n_hi=n_hi, page_size=bs, k=0, block_size=bs,
                       top_blocks=top, first=(0, bs * top - 5, bs * top + 1))
    blocks, slots = ops.block_topk(*_inputs(case), case.page_size, case.max_seq_len, bs, top)
    torch.cuda.synchronize()
    blocks, slots = blocks.cpu().numpy(), slots.cpu().numpy()
    rb, rs, rl, _ = oracle.block_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(blocks[b]), np.sort(rb[b])), b
        # slot lists: compare per selected block
        got = {int(blocks[b, i]): slots[b, i * bs:(i + 1) * bs].tolist() for i in range(top) if blocks[b, i] >= 0}
        exp = {int(rb[b, i]): rs[b, i * bs:(i + 1) * bs].tolist() for i in range(top) if rb[b, i] >= 0}
        assert got == exp
        assert (slots[b, len(got) * bs:] == -1).all()


def test_block_random_tolerance(ops):
    """Random fp8 inputs: every chosen block's oracle block score is within tol
    of the oracle's top-th block score."""
    import torch

    bs, top = 128, 32
    case = workloads.indexer_case(900, batch=6, n_lo=bs, n_hi=40000, page_size=bs, k=0, block_size=bs,
                                  top_blocks=top)
    blocks = ops.block_topk(*_inputs(case), case.page_size, case.max_seq_len, bs, top, return_slots=False)
    torch.cuda.synchronize()
    blocks = blocks.cpu().numpy()
    for b in range(case.batch):
        S = case_scores(case, b)
        bsv = oracle.block_scores(S, bs)
        nb = bsv.shape[0]
        m = min(nb, top)
        page_to_blk = {int(case.block_table[b, c]): c for c in range(nb)}
        sel = [page_to_blk[int(p)] for p in blocks[b, :m]]
        assert len(set(sel)) == m and (blocks[b, m:] == -1).all()
        sigma = float(np.sqrt(np.mean(S * S)))
        kth = np.sort(bsv)[::-1][m - 1]
        assert (bsv[sel] >= kth - 1e-3 * max(abs(kth), sigma)).all()


def test_fused_decode_full_size(ops):
    """Full-size fused decode (B=32, n in [8192, 16384], k=2048): every row
    against the oracle criterion, returned scores within the tolerance."""
    from tests import _fullsize

    case = workloads.c2_fused_decode()
    log(f"case {case.name}")
    slots, sc = _fused(ops, case)
    _fullsize.run(_fullsize.fused_rows_task, _fullsize.fused_tasks(case, slots, sc), case.name)


def test_long_decode_full_size(ops):
    """Full-size long-context decode (B=64, n up to 327680, k=2048): every
    row against the oracle criterion, returned scores within the tolerance."""
    from tests import _fullsize

    case = workloads.c5_long_decode()
    log(f"case {case.name} tokens={workloads.expected_tokens(case)}")
    slots, sc = _fused(ops, case)
    case.kcache = case.k_scale = None  # the workers draw each row's keys again
    _fullsize.run(_fullsize.fused_rows_task, _fullsize.fused_tasks(case, slots, sc), case.name)


def test_block_sparse_full_size(ops):
    """Full-size block-sparse decode (B=64, n=32768, top 32 of 256 blocks):
    every row against the block-score criterion, slot lists exact."""
    import torch

    from tests import _fullsize

    case = workloads.c4_block_sparse()
    log(f"case {case.name}")
    blocks, slots = ops.block_topk(*_inputs(case), case.page_size, case.max_seq_len, case.block_size,
                                   case.top_blocks)
    torch.cuda.synchronize()
    blocks, slots = blocks.cpu().numpy(), slots.cpu().numpy()
    _fullsize.run(_fullsize.block_rows_task, _fullsize.block_tasks(case, blocks, slots), case.name)


# ---------------------------------------------------------------------------
# Multi-token decode rows: several query rows share a block-table row
# ---------------------------------------------------------------------------


def _expanded(case):
    """The case with the indirection resolved: each query row gets its own
    copy of its block-table row."""
    import copy

    flat = copy.copy(case)
    flat.block_table = np.ascontiguousarray(case.block_table[case.row_to_batch])
    flat.row_to_batch = None
    return flat


@pytest.mark.parametrize("page_size,k", [(64, 2048), (16, 300)])
def test_multi_query_fused(ops, page_size, k):
    """Each row's selection meets the oracle criterion, and equals the run
    with the block-table rows copied out (same fp32 scores), for both fused
    variants."""
    case = workloads.multi_query_case(900 + page_size, requests=5, next_n=3, n_lo=1, n_hi=20000,
                                      page_size=page_size, k=k)
    log(f"multi-query fused: rows={case.batch} P={page_size} k={k}")
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    flat = _expanded(case)
    ref, _ = _fused(ops, flat)
    for c in (case, _guided_variant(case)):
        slots, sc = _fused(ops, c)
        assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1)), c.max_seq_len
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[case.row_to_batch[b]], case.page_size, n)
        check_fused_row(slots[b], sc[b], rows[b], ts, k, batch_sigma=bsig)


@pytest.mark.parametrize("heads,page_size,k,requests,next_n", [
    (64, 64, 2048, 8, 3),   # 24 rows: row pairs straddle requests
    (32, 16, 300, 4, 4),    # 16 rows: each quad one request
    (16, 128, 700, 6, 2),   # 12 rows: pairs within requests, quads across two
    (64, 32, 64, 3, 4),     # 12 rows, k far below the row lengths
])
def test_multi_query_fused_row_pairs(ops, heads, page_size, k, requests, next_n):
    """Rows in quads (a row count that is a multiple of 4): the fused call
    scores two rows per chunk workgroup against one key load. Its selection
    equals the per-row call's on the expanded block tables (the same fp32
    scores), on the one-wave and the guided chunk schedules, and every row
    meets the oracle criterion."""
    case = workloads.multi_query_case(940 + page_size, requests=requests, next_n=next_n, n_lo=1, n_hi=20000,
                                      page_size=page_size, k=k, heads=heads)
    assert case.batch % 4 == 0
    log(f"multi-query fused, row pairs: rows={case.batch} heads={heads} P={page_size} k={k}")
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    ref, ref_sc = _fused(ops, _expanded(case))
    for c in (case, _guided_variant(case)):
        slots, sc = _fused(ops, c)
        assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1)), c.max_seq_len
        assert np.array_equal(np.sort(sc, axis=1), np.sort(ref_sc, axis=1)), c.max_seq_len
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[case.row_to_batch[b]], case.page_size, n)
        check_fused_row(slots[b], sc[b], rows[b], ts, k, batch_sigma=bsig)


def test_multi_query_fused_row_pairs_short_rows(ops):
    """Two rows per chunk workgroup at the edges: contexts 1, 2, 3 and 16
    give rows of 0 to 3 keys (a pair with one empty row, pairs shorter than
    k) beside longer requests, so chunks hold one row of a pair and not the
    other. The selection equals the per-row call's on the expanded block
    tables and meets the oracle criterion."""
    lens = np.array([1, 2, 3, 16, 2047, 2049, 4100, 9000], np.int32)
    case = workloads.multi_query_case(960, requests=8, next_n=2, n_lo=0, n_hi=0, page_size=64, k=2048, heads=64,
                                      fixed_lens=lens)
    assert case.batch % 4 == 0 and int(case.seq_lens.min()) == 0
    log(f"multi-query fused, row pairs, short rows: rows={case.batch} lens={case.seq_lens.tolist()}")
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate([r for r in rows if r.size]))
    ref, ref_sc = _fused(ops, _expanded(case))
    slots, sc = _fused(ops, case)
    assert np.array_equal(np.sort(slots, axis=1), np.sort(ref, axis=1))
    assert np.array_equal(np.sort(sc, axis=1), np.sort(ref_sc, axis=1))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[case.row_to_batch[b]], case.page_size, n)
        check_fused_row(slots[b], sc[b], rows[b], ts, case.k, batch_sigma=bsig)


def test_multi_query_scores(ops):
    case = workloads.multi_query_case(911, requests=4, next_n=4, n_lo=1, n_hi=5000, page_size=32, k=0, heads=32)
    out = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len, row_to_batch=_r2b(case))
    flat = _expanded(case)
    out2 = ops.idx_score_fp8(*_inputs(flat), flat.page_size, flat.max_seq_len)
    import torch

    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        assert np.array_equal(out[b, :n], out2[b, :n]), b
        check_scores(out[b, :n], case_scores(case, b))


def test_multi_query_block(ops):
    bs = 64
    case = workloads.multi_query_case(912, requests=4, next_n=3, n_lo=bs, n_hi=30000, page_size=bs, k=0)
    flat = _expanded(case)
    got = ops.block_topk(*_inputs(case), bs, case.max_seq_len, bs, 20, row_to_batch=_r2b(case))
    exp = ops.block_topk(*_inputs(flat), bs, flat.max_seq_len, bs, 20)
    import torch

    torch.cuda.synchronize()
    # output order within a row is unspecified: compare the block sets, and
    # each block's slot list by block id
    gb, gs = got[0].cpu().numpy(), got[1].cpu().numpy()
    eb, es = exp[0].cpu().numpy(), exp[1].cpu().numpy()
    assert np.array_equal(np.sort(gb, axis=1), np.sort(eb, axis=1))
    for b in range(case.batch):
        gmap = {int(x): tuple(gs[b, i * bs:(i + 1) * bs]) for i, x in enumerate(gb[b]) if x >= 0}
        emap = {int(x): tuple(es[b, i * bs:(i + 1) * bs]) for i, x in enumerate(eb[b]) if x >= 0}
        assert gmap == emap, b
    blocks = gb
    top = 20
    for b in range(case.batch):
        S = case_scores(case, b)
        bsv = oracle.block_scores(S, bs)
        nb = bsv.shape[0]
        m = min(nb, top)
        bt_row = case.block_table[case.row_to_batch[b]]
        page_to_blk = {int(bt_row[c]): c for c in range(nb)}
        sel = [page_to_blk[int(p)] for p in blocks[b, :m]]
        assert len(set(sel)) == m and (blocks[b, m:] == -1).all()
        sigma = float(np.sqrt(np.mean(S * S)))
        kth = np.sort(bsv)[::-1][m - 1]
        assert (bsv[sel] >= kth - 1e-3 * max(abs(kth), sigma)).all()


@pytest.mark.parametrize("heads,page_size,next_n,requests", [(64, 64, 3, 5), (16, 16, 4, 3), (32, 128, 1, 7),
                                                            (64, 32, 300, 2)])
def test_row_pair_scores_match_per_row(ops, heads, page_size, next_n, requests):
    """With row_to_batch, idx_score_fp8 scores two rows per wave against one
    key load. Its scores are bit-identical to the one-row-per-workgroup path
    on the same case with block-table rows copied out (pairs that straddle
    two requests, odd row counts and single-row requests included)."""
    import torch

    case = workloads.multi_query_case(930 + next_n, requests=requests, next_n=next_n, n_lo=1, n_hi=6000,
                                      page_size=page_size, k=0, heads=heads)
    log(f"row pairs: rows={case.batch} heads={heads} P={page_size}")
    out = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len, row_to_batch=_r2b(case))
    flat = _expanded(case)
    out2 = ops.idx_score_fp8(*_inputs(flat), flat.page_size, flat.max_seq_len)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        assert np.array_equal(out[b, :n], out2[b, :n]), b
    for b in (0, case.batch // 2, case.batch - 1):
        n = int(case.seq_lens[b])
        check_scores(out[b, :n], case_scores(case, b))


@pytest.mark.timeout(900)
def test_prefill_indexer_full_size(ops):
    """The prefill workload at full size, in the launch configuration the
    benchmark times (idx_score_fp8 with row_to_batch, then topk_rows through
    the block table): every row's scores against the oracle's within the
    tolerance and its selection against the oracle criterion, in the oracle
    pool."""
    import torch

    from tests import _fullsize

    case = workloads.prefill_indexer()
    log(f"prefill full size: rows={case.batch} max n={case.max_seq_len}")
    r2b = _r2b(case)
    scores = ops.idx_score_fp8(*_inputs(case), case.page_size, case.max_seq_len, row_to_batch=r2b)
    slots = ops.topk_rows(scores, dev(case.seq_lens), case.k, row_to_batch=r2b, page_table=dev(case.block_table),
                          page_size=case.page_size)
    torch.cuda.synchronize()
    host = scores.cpu().numpy()
    slots = slots.cpu().numpy()
    del scores
    torch.cuda.empty_cache()
    lens = case.seq_lens

    def gpu_rows(rr):
        return [host[b, :int(lens[b])] for b in rr]

    # request 0's rows see ~62K-70K keys, request 1's 1..8192: smaller tasks
    # for the long rows keep the pool busy to the end
    def tasks():
        yield from _fullsize.fused_tasks(case, slots, rows=np.arange(0, 8192), per_task=32, gpu_scores=gpu_rows)
        yield from _fullsize.fused_tasks(case, slots, rows=np.arange(8192, case.batch), per_task=512,
                                         gpu_scores=gpu_rows)

    n = _fullsize.run(_fullsize.fused_rows_task, tasks(), case.name)
    assert n == case.batch


# Sorted output: rows in descending score order, equal scores by ascending
# position, -1 padding last. The oracle's selection is a stable descending
# sort, so its order is that order: with exact arithmetic the whole output
# sequence must match, ties included.
@pytest.mark.parametrize("variant", ["resident", "guided"])
@pytest.mark.parametrize("with_scores", [True, False])
@pytest.mark.parametrize("k", [100, 700, 3000, 8192])
def test_fused_sorted_exact_order(ops, variant, with_scores, k):
    import torch
    from sparse_attention_indexer_fp8_amd import ops as o

    case = _exact_case(640 + k, batch=5, n_lo=1, n_hi=12000, page_size=64, heads=64, k=k, first=(0, k - 1, k))
    if variant == "guided":
        case = _guided_variant(case)
    ws = o.Workspace()
    res = ops.idx_score_topk_fused(*_inputs(case), case.page_size, case.max_seq_len, case.k,
                                   return_scores=with_scores, workspace=ws, row_to_batch=_r2b(case), sorted=True)
    torch.cuda.synchronize()
    slots, sc = (res[0].cpu().numpy(), res[1].cpu().numpy()) if with_scores else (res.cpu().numpy(), None)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(slots[b], ref_slots[b]), b
        if sc is not None:
            m = min(int(case.seq_lens[b]), case.k)
            assert np.array_equal(sc[b][:m].astype(np.float64), scores[b][ref_pos[b][:m]]), b
            assert np.all(np.isneginf(sc[b][m:])), b


def test_fused_sorted_random_order(ops):
    """Random inputs: the sorted call returns the unsorted call's selection,
    ordered by its own scores (descending), and the same slots as a set."""
    import torch

    case = workloads.indexer_case(650, batch=6, n_lo=1, n_hi=30000, page_size=64, k=2048)
    for big in (False, True):
        c = _guided_variant(case) if big else case
        s0, v0 = _fused(ops, c)
        s1, v1 = ops.idx_score_topk_fused(*_inputs(c), c.page_size, c.max_seq_len, c.k, return_scores=True,
                                          row_to_batch=_r2b(c), sorted=True)
        torch.cuda.synchronize()
        s1, v1 = s1.cpu().numpy(), v1.cpu().numpy()
        for b in range(c.batch):
            assert np.array_equal(np.sort(s1[b]), np.sort(s0[b])), b
            assert np.all(v1[b][:-1] >= v1[b][1:]), b  # (-inf padding compares equal)
            # the score that goes with each slot is unchanged by the sort
            assert dict(zip(s0[b].tolist(), v0[b].tolist())) == dict(zip(s1[b].tolist(), v1[b].tolist())), b


# Per-head block selection: every (row, head) keeps its own blocks by the
# head's term of the score.
# (the last two cases take the workgroup merge: more than 256 kept blocks,
# more than 1024 blocks per row)
@pytest.mark.parametrize("bs,top,heads,n_hi", [(128, 32, 64, 9000), (64, 7, 16, 9000), (16, 5, 128, 9000),
                                               (16, 300, 16, 9000), (16, 40, 16, 20000)])
def test_block_heads_exact(ops, bs, top, heads, n_hi):
    import torch

    case = _exact_case(1000 + bs + heads + top, batch=4, n_lo=1, n_hi=n_hi, page_size=bs, heads=heads, k=0,
                       block_size=bs, top_blocks=top, first=(0, bs * top - 5, bs * top + 1))
    blocks, slots = ops.block_topk_heads(*_inputs(case), case.page_size, case.max_seq_len, bs, top)
    torch.cuda.synchronize()
    blocks, slots = blocks.cpu().numpy(), slots.cpu().numpy()
    rb, rs = oracle.block_topk_heads(case)
    for b in range(case.batch):
        for h in range(heads):
            assert np.array_equal(np.sort(blocks[b, h]), np.sort(rb[b, h])), (b, h)
            got = {int(blocks[b, h, i]): slots[b, h, i * bs:(i + 1) * bs].tolist() for i in range(top)
                   if blocks[b, h, i] >= 0}
            exp = {int(rb[b, h, i]): rs[b, h, i * bs:(i + 1) * bs].tolist() for i in range(top) if rb[b, h, i] >= 0}
            assert got == exp, (b, h)


def test_block_heads_random_tolerance(ops):
    """Random fp8 inputs: each (row, head)'s chosen blocks are within the
    score tolerance of that head's top-th block score."""
    import torch
    from oracle.indexer import case_bt_row, index_head_scores

    bs, top = 128, 16
    case = workloads.indexer_case(1010, batch=3, n_lo=bs, n_hi=20000, page_size=bs, k=0, block_size=bs,
                                  top_blocks=top, heads=32)
    blocks = ops.block_topk_heads(*_inputs(case), case.page_size, case.max_seq_len, bs, top, return_slots=False)
    torch.cuda.synchronize()
    blocks = blocks.cpu().numpy()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        bt = case_bt_row(case, b)
        T = index_head_scores(case.q[b], case.q_scale[b], case.w[b], case.kcache, case.k_scale, bt,
                              case.page_size, n)
        nb = -(-n // bs)
        page_to_blk = {int(bt[c]): c for c in range(nb)}
        for h in range(case.heads):
            bsv = oracle.block_scores(T[:, h], bs)
            m = min(nb, top)
            sel = [page_to_blk[int(p)] for p in blocks[b, h, :m]]
            assert len(set(sel)) == m and (blocks[b, h, m:] == -1).all()
            sigma = max(float(np.sqrt(np.mean(T[:, h] ** 2))), 1e-30)
            kth = np.sort(bsv)[::-1][m - 1]
            assert (bsv[sel] >= kth - 1e-3 * max(abs(kth), sigma)).all(), (b, h)


# ---------------------------------------------------------------------------
# Full-size checks of the remaining benchmarked configurations, in the launch
# configuration bench.py times.
# ---------------------------------------------------------------------------

def test_mtp_decode_full_size(ops):
    """Multi-token decode 16 x 4 (n 16K-64K, k 2048): every row meets the
    tolerance criterion."""
    from tests import _fullsize

    case = workloads.mtp_decode()
    log(f"case {case.name}")
    slots, sc = _fused(ops, case)
    _fullsize.run(_fullsize.fused_rows_task, _fullsize.fused_tasks(case, slots, sc, per_task=4), case.name)


def test_fused_decode_full_size_sorted(ops):
    """Fused decode B32 with sorted output: the same selection as the
    unsorted call, each row in descending score order with its scores."""
    import torch

    case = workloads.c2_fused_decode()
    s0, v0 = _fused(ops, case)
    s1, v1 = ops.idx_score_topk_fused(*_inputs(case), case.page_size, case.max_seq_len, case.k, return_scores=True,
                                      sorted=True)
    torch.cuda.synchronize()
    s1, v1 = s1.cpu().numpy(), v1.cpu().numpy()
    for b in range(case.batch):
        assert np.array_equal(np.sort(s1[b]), np.sort(s0[b])), b
        assert np.all(v1[b][:-1] >= v1[b][1:]), b
        assert dict(zip(s0[b].tolist(), v0[b].tolist())) == dict(zip(s1[b].tolist(), v1[b].tolist())), b


def test_block_heads_full_size(ops):
    """Per-head selection on the block-sparse geometry (B64, n 32768, top 32,
    64 heads): every row and head against the block-score criterion, slot
    lists exact."""
    import torch

    from tests import _fullsize

    case = workloads.c4_block_sparse()
    bs, top = case.block_size, case.top_blocks
    blocks, slots = ops.block_topk_heads(*_inputs(case), case.page_size, case.max_seq_len, bs, top)
    torch.cuda.synchronize()
    blocks, slots = blocks.cpu().numpy(), slots.cpu().numpy()
    _fullsize.run(_fullsize.block_rows_task, _fullsize.block_tasks(case, blocks, slots, per_head=True, per_task=2),
                  case.name + " per head")


@pytest.mark.parametrize("entry", ["block_topk", "block_topk_heads"])
def test_block_slots_unaligned_output(ops, entry):
    """Slot lists written through an output pointer that is not 16-byte
    aligned (entries stored one by one) equal the aligned call's (four
    entries per 16-byte store), and both equal the oracle's."""
    import torch
    from sparse_attention_indexer_fp8_amd import _lib

    bs, top = 64, 9
    case = _exact_case(870 + len(entry), batch=3, n_lo=1, n_hi=9000, page_size=bs, heads=16, k=0,
                       block_size=bs, top_blocks=top, first=(0, bs * top - 5))
    ins = _inputs(case)
    fn = getattr(ops, entry)
    blocks, slots = fn(*ins, bs, case.max_seq_len, bs, top)
    args, B, H, D = ops._indexer_args(*ins)
    lead = (B, H) if entry == "block_topk_heads" else (B,)
    op = _lib.OP_BLOCK_TOPK_HEADS if entry == "block_topk_heads" else _lib.OP_BLOCK_TOPK
    rows = B * H if entry == "block_topk_heads" else B
    ws = torch.zeros(ops.workspace_bytes(op, rows, bs, case.max_seq_len), dtype=torch.uint8, device="cuda")
    out_blocks = torch.empty(lead + (top,), dtype=torch.int32, device="cuda")
    buf = torch.full((int(np.prod(lead)) * top * bs + 1,), 7, dtype=torch.int32, device="cuda")
    shifted = buf[1:]
    assert shifted.data_ptr() % 16 != 0
    st = getattr(_lib.load(), entry)(*args, bs, None, ops._ptr(ins[6]), B, H, D, case.max_seq_len, bs, top,
                                     ops._ptr(out_blocks), ops._ptr(shifted), ops._ptr(ws), ws.numel(),
                                     ops._stream())
    _lib.check(entry, st)
    torch.cuda.synchronize()
    assert int(buf[0]) == 7

    # the order of a selection's blocks is unspecified: compare each
    # selection's blocks as a set, and each block's slot list
    def lists(blk, sl):
        blk = blk.reshape(-1, top).cpu().numpy()
        sl = sl.reshape(-1, top * bs).cpu().numpy()
        return [{int(blk[r, i]): sl[r, i * bs:(i + 1) * bs].tolist() for i in range(top) if blk[r, i] >= 0}
                for r in range(blk.shape[0])], [int((blk[r] < 0).sum()) for r in range(blk.shape[0])]

    got, got_pad = lists(out_blocks, shifted)
    ref, ref_pad = lists(blocks, slots)
    assert got == ref and got_pad == ref_pad
    for r in range(len(got)):  # padding entries of the slot lists
        n_sel = top - got_pad[r]
        assert (shifted.reshape(-1, top * bs)[r, n_sel * bs:] == -1).all()
    if entry == "block_topk":
        rb, rs, _, _ = oracle.block_topk(case)
        exp, _ = lists(torch.from_numpy(np.ascontiguousarray(rb)), torch.from_numpy(np.ascontiguousarray(rs)))
        assert got == exp
