"""Pins for the oracle's paged fp8 scoring and the block variant (CPU only)."""
import math

import numpy as np
import pytest

import workloads
from oracle.fp8 import E4M3FN_TABLE
from oracle.indexer import (block_scores, block_topk, case_scores, fused_topk, index_scores,
                            token_slots, topk_order)


def _code_times_512(c: int) -> int:
    """Integer value * 2^9 of one e4m3fn byte, from its bit fields.

    Subnormal: m * 2^-9 * 2^9 = m. Normal: (8 + m)/8 * 2^(e-7) * 2^9 = (8 + m) << (e - 1).
    """
    s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 7
    mag = m if e == 0 else (8 + m) << (e - 1)
    return -mag if s else mag


INT_TABLE = np.array([_code_times_512(c) for c in range(256)], dtype=np.int64)


def _slots_loop(bt_row, P, n):
    out = []
    for j in range(n):
        out.append(int(bt_row[j // P]) * P + (j % P))
    return np.array(out, dtype=np.int64)


def test_integer_table_agrees_with_closed_form():
    ok = ~np.isnan(E4M3FN_TABLE)
    assert np.array_equal(INT_TABLE[ok].astype(np.float64), E4M3FN_TABLE[ok] * 512.0)


@pytest.mark.parametrize("seed", [0, 1])
def test_dot_exact_against_int64(seed):
    """The float64 dot equals an int64 recomputation on 2^9-scaled codes, bit for bit."""
    case = workloads.indexer_case(seed, batch=2, n_lo=70, n_hi=130, page_size=16, k=8,
                                  heads=16, dim=128)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        slots = _slots_loop(case.block_table[b], case.page_size, n)
        assert np.array_equal(slots, token_slots(case.block_table[b], case.page_size, n))
        qi = INT_TABLE[case.q[b]]  # [H, D]
        ki = INT_TABLE[case.kcache[slots]]  # [n, D]
        dot_int = np.zeros((n, case.heads), np.int64)
        for h in range(case.heads):
            dot_int[:, h] = (ki * qi[h][None, :]).sum(axis=1)
        # oracle path with unit scales and one-hot weights exposes each head's ReLU(dot)
        for h in (0, case.heads - 1):
            w = np.zeros(case.heads, np.float32)
            w[h] = 1.0
            S = index_scores(case.q[b], 1.0, w, case.kcache, np.ones_like(case.k_scale),
                             case.block_table[b], case.page_size, n)
            expect = np.maximum(dot_int[:, h], 0).astype(np.float64) / 2.0 ** 18
            assert np.array_equal(S, expect)


def test_brute_force_fsum_tiny():
    """Pure-Python loops with math.fsum on a tiny case (float64 rounding only)."""
    case = workloads.indexer_case(5, batch=1, n_lo=9, n_hi=9, page_size=4, k=4, heads=16, dim=128)
    b = 0
    n = int(case.seq_lens[b])
    S = case_scores(case, b)
    for j in range(n):
        slot = int(case.block_table[b][j // 4]) * 4 + j % 4
        terms = []
        for h in range(case.heads):
            d = math.fsum(E4M3FN_TABLE[case.q[b, h, x]] * E4M3FN_TABLE[case.kcache[slot, x]]
                          for x in range(case.dim))
            logit = d * float(case.q_scale[b]) * float(case.k_scale[slot])
            terms.append(float(case.w[b, h]) * max(0.0, logit))
        ref = math.fsum(terms)
        assert abs(S[j] - ref) <= 1e-14 * max(1.0, abs(ref))


def _tiny_case(heads=1, dim=128, n=5, P=2, seed=9):
    return workloads.indexer_case(seed, batch=1, n_lo=n, n_hi=n, page_size=P, k=2,
                                  heads=heads, dim=dim)


def test_single_head_unit_scales_is_relu_dot():
    case = _tiny_case(heads=16)
    n = int(case.seq_lens[0])
    slots = _slots_loop(case.block_table[0], case.page_size, n)
    w = np.zeros(case.heads, np.float32)
    w[3] = 1.0
    S = index_scores(case.q[0], 1.0, w, case.kcache, np.ones_like(case.k_scale),
                     case.block_table[0], case.page_size, n)
    qd = E4M3FN_TABLE[case.q[0, 3]]
    for j in range(n):
        kd = E4M3FN_TABLE[case.kcache[slots[j]]]
        assert S[j] == max(0.0, float(np.dot(qd, kd)))


def test_one_hot_query_picks_key_coordinate():
    case = _tiny_case(heads=16)
    q = np.zeros_like(case.q[0])
    for h in range(case.heads):
        q[h, (5 * h) % case.dim] = 0x38  # 1.0 at one coordinate per head
    w = np.linspace(0.5, 2.0, case.heads).astype(np.float32)
    n = int(case.seq_lens[0])
    S = index_scores(q, 1.0, w, case.kcache, np.ones_like(case.k_scale), case.block_table[0],
                     case.page_size, n)
    slots = _slots_loop(case.block_table[0], case.page_size, n)
    for j in range(n):
        kd = E4M3FN_TABLE[case.kcache[slots[j]]]
        ref = sum(float(w[h]) * max(0.0, kd[(5 * h) % case.dim]) for h in range(case.heads))
        assert abs(S[j] - ref) <= 1e-14 * max(1.0, abs(ref))


def test_scales_and_weights_behave():
    case = workloads.indexer_case(3, batch=1, n_lo=40, n_hi=40, page_size=8, k=4, heads=16)
    n = int(case.seq_lens[0])
    base = case_scores(case, 0)
    # doubling every key scale doubles every score (exact: power-of-two scaling)
    S2 = index_scores(case.q[0], case.q_scale[0], case.w[0], case.kcache, case.k_scale * 2,
                      case.block_table[0], case.page_size, n)
    assert np.array_equal(S2, 2 * base)
    # doubling the query scale doubles too
    S3 = index_scores(case.q[0], case.q_scale[0] * 2, case.w[0], case.kcache, case.k_scale,
                      case.block_table[0], case.page_size, n)
    assert np.array_equal(S3, 2 * base)
    # all-negative weights: every score <= 0, and negating weights negates scores
    Sn = index_scores(case.q[0], case.q_scale[0], -np.abs(case.w[0]), case.kcache, case.k_scale,
                      case.block_table[0], case.page_size, n)
    Sp = index_scores(case.q[0], case.q_scale[0], np.abs(case.w[0]), case.kcache, case.k_scale,
                      case.block_table[0], case.page_size, n)
    assert (Sn <= 0).all() and np.array_equal(Sn, -Sp)


def test_scores_never_touch_sentinels():
    """Every real token's key is finite-scaled; sentinel slots would score ~1e3x higher."""
    case = workloads.indexer_case(4, batch=3, n_lo=1, n_hi=200, page_size=64, k=16, heads=16)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        slots = token_slots(case.block_table[b], case.page_size, n)
        assert (case.k_scale[slots] < workloads.SENTINEL_KEY_SCALE).all()


def test_fused_topk_consistent():
    case = workloads.indexer_case(6, batch=3, n_lo=100, n_hi=400, page_size=64, k=64, heads=16)
    slots, pos, scores = fused_topk(case)
    for b in range(case.batch):
        assert pos[b].tolist() == topk_order(scores[b], case.k).tolist()
        n = int(case.seq_lens[b])
        ts = token_slots(case.block_table[b], case.page_size, n)
        assert slots[b].tolist() == [int(ts[p]) if p >= 0 else -1 for p in pos[b]]


def test_block_scores_are_block_max():
    S = np.array([1.0, 5.0, 2.0, -1.0, 7.0, 0.0, 3.0])
    assert block_scores(S, 3).tolist() == [5.0, 7.0, 3.0]
    assert block_scores(S, 1).tolist() == S.tolist()


def test_block_size_one_reduces_to_token_topk():
    case = workloads.indexer_case(8, batch=2, n_lo=50, n_hi=90, page_size=1, k=0, heads=16,
                                  block_size=1, top_blocks=12)
    blocks, slot_lists, logical, _ = block_topk(case)
    for b in range(case.batch):
        S = case_scores(case, b)
        assert logical[b].tolist() == topk_order(S, 12).tolist()
        assert np.array_equal(slot_lists[b], blocks[b])


def test_block_planted_maxima_and_ties():
    """Blocks holding a planted max key win; equal planted blocks go to the lower id."""
    case = workloads.indexer_case(10, batch=1, n_lo=16 * 20, n_hi=16 * 20, page_size=16, k=0,
                                  heads=16, block_size=16, top_blocks=3)
    n = int(case.seq_lens[0])
    slots = token_slots(case.block_table[0], 16, n)
    q = np.full_like(case.q[0], 0x38)  # all ones
    case.q[0] = q
    case.w[0] = 1.0
    # plant identical max keys (all 448) in tokens of blocks 4, 11 and 17, and
    # block 2 gets a slightly smaller planted key
    for blk, byte in ((4, 0x7E), (11, 0x7E), (17, 0x7E), (2, 0x7D)):
        case.kcache[slots[blk * 16 + 5]] = byte
        case.k_scale[slots[blk * 16 + 5]] = 1.0
    _, _, logical, bsv = block_topk(case)
    assert sorted(logical[0].tolist()) == [4, 11, 17]
    case.block_table  # unchanged
    _, _, logical2, _ = block_topk(case, top_blocks=2)
    assert logical2[0].tolist() == [4, 11]
    _, _, logical4, _ = block_topk(case, top_blocks=4)
    assert logical4[0].tolist() == [4, 11, 17, 2]


def test_block_short_row_padding():
    case = workloads.indexer_case(12, batch=2, n_lo=0, n_hi=0, page_size=128, k=0, heads=16,
                                  block_size=128, top_blocks=4, fixed_lens=np.array([0, 200]))
    blocks, slot_lists, logical, _ = block_topk(case)
    assert (blocks[0] == -1).all() and (slot_lists[0] == -1).all()
    assert sorted(logical[1][:2].tolist()) == [0, 1] and (logical[1][2:] == -1).all()
    # block 1 holds tokens 128..199: 72 visible slots then -1
    i1 = logical[1].tolist().index(1)
    sl = slot_lists[1][i1 * 128:(i1 + 1) * 128]
    assert (sl[:72] >= 0).all() and (sl[72:] == -1).all()


def _expanded(case):
    """The same case with the block-table indirection resolved: query row b
    gets its own copy of block-table row row_to_batch[b]."""
    import copy

    flat = copy.copy(case)
    flat.block_table = np.ascontiguousarray(case.block_table[case.row_to_batch])
    flat.row_to_batch = None
    return flat


def test_multi_query_rows_share_the_request_cache():
    """Multi-token decode rows: row r * next_n + t of request r sees the
    request's first L_r - (next_n - 1 - t) tokens through the request's
    block-table row. Resolving the indirection by copying block-table rows
    gives identical scores and selections (the copy-versus-indirection check
    of [SGL-37889], Modifications)."""
    case = workloads.multi_query_case(31, requests=3, next_n=4, n_lo=1, n_hi=400, page_size=16, k=40, heads=16)
    R, T = 3, 4
    assert case.batch == R * T
    assert np.array_equal(case.row_to_batch, np.repeat(np.arange(R), T))
    base_lens = workloads.indexer_case(31, batch=R, n_lo=1, n_hi=400, page_size=16, k=40, heads=16).seq_lens
    for r in range(R):
        for t in range(T):
            assert case.seq_lens[r * T + t] == max(int(base_lens[r]) - (T - 1 - t), 0)
    flat = _expanded(case)
    for b in range(case.batch):
        assert np.array_equal(case_scores(case, b), case_scores(flat, b))
    s1, p1, _ = fused_topk(case)
    s2, p2, _ = fused_topk(flat)
    assert np.array_equal(s1, s2) and np.array_equal(p1, p2)
    # the last query token of a request sees the request's whole context, so
    # its scores are index_scores over the request's own block-table row
    for r in range(R):
        b = r * T + T - 1
        S = index_scores(case.q[b], case.q_scale[b], case.w[b], case.kcache, case.k_scale,
                         case.block_table[r], case.page_size, int(base_lens[r]))
        assert np.array_equal(case_scores(case, b), S)


def test_multi_query_block_variant_matches_expanded():
    case = workloads.multi_query_case(32, requests=2, next_n=3, n_lo=100, n_hi=700, page_size=16, k=0, heads=16)
    flat = _expanded(case)
    a = block_topk(case, block_size=16, top_blocks=5)
    b = block_topk(flat, block_size=16, top_blocks=5)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def test_head_terms_sum_to_index_score():
    """The per-head terms add up to the (separately pinned) index score, and
    each is the weight times a non-negative number."""
    from oracle.indexer import case_bt_row, index_head_scores, index_scores

    case = workloads.indexer_case(321, batch=2, n_lo=50, n_hi=400, page_size=16, k=8, heads=32)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        args = (case.q[b], case.q_scale[b], case.w[b], case.kcache, case.k_scale, case_bt_row(case, b),
                case.page_size, n)
        T = index_head_scores(*args)
        assert T.shape == (n, case.heads)
        np.testing.assert_allclose(T.sum(axis=1), index_scores(*args), rtol=1e-12, atol=1e-12)
        assert np.all(T * np.sign(case.w[b])[None, :] >= 0)


def test_per_head_blocks_single_head_equal_block_topk():
    """With one head of the 16 carrying weight and the rest weight 0, that
    head's selection is the head-summed block selection."""
    from oracle.indexer import block_topk, block_topk_heads

    case = workloads.indexer_case(322, batch=2, n_lo=300, n_hi=2000, page_size=64, k=0, heads=16,
                                  block_size=64, top_blocks=5)
    case.w[:] = 0.0
    case.w[:, 3] = 1.5
    hb, hs = block_topk_heads(case)
    rb, rs, _, _ = block_topk(case)
    assert np.array_equal(hb[:, 3], rb) and np.array_equal(hs[:, 3], rs)
