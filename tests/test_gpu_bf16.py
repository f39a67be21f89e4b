"""GPU parity of the bf16 index-cache entry points against the oracle.

Same bars as the fp8 tests: scores within the 1e-3 relative tolerance,
selections exact on exact-arithmetic inputs and meeting the tolerance
criterion on random ones, the cache writer bit-exact.
"""
import copy

import numpy as np
import pytest

import oracle
import workloads
from oracle.indexer import case_scores
from tests._helpers import check_fused_row, check_scores, dev, log, rms

pytestmark = pytest.mark.gpu

# batches of more than this many tokens never fit one resident wave of the
# fused path's chunk workgroups (at most 8192 tokens each, at most 8 per
# compute unit on 256 units): they take the guided chunk schedule
FUSED_GUIDED_TOKENS = 1 << 24


@pytest.fixture(scope="module")
def ops():
    import torch
    from sparse_attention_indexer_fp8_amd import ops as _ops

    torch.cuda.set_device(0)
    return _ops


def _inputs(case):
    return dev(case.q), dev(case.w), dev(case.kcache), dev(case.block_table), dev(case.seq_lens)


def _r2b(case):
    return None if case.row_to_batch is None else dev(case.row_to_batch)


def _lens(seed, batch, n_lo, n_hi, first=()):
    lens = workloads.rng(seed, workloads.synth.STREAM_LEN).integers(n_lo, n_hi + 1, size=batch).astype(np.int32)
    lens[:len(first)] = first
    return lens


# 0, +-0.5, +-1, +-2 as bf16 patterns
_EXACT = np.array([0x0000, 0x3F00, 0x3F80, 0x4000, 0xBF00, 0xBF80, 0xC000], np.uint16)


def _exact_case(seed, batch, n_lo, n_hi, page_size, heads=64, k=64, first=(), **kw):
    """bf16 inputs whose fp32 scores are exact (small multiples of 1/4 below
    2^10, power-of-two weights): the selected sets must equal the oracle's,
    ties included."""
    case = workloads.indexer_case(seed, batch=batch, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k, heads=heads,
                                  fixed_lens=_lens(seed, batch, n_lo, n_hi, first), cache_dtype="bf16", **kw)
    g = np.random.default_rng(seed + 2000)
    case.q[:] = g.choice(_EXACT, size=case.q.shape)
    case.w[:] = g.choice(np.array([0.5, 1.0, 2.0, -1.0], np.float32), size=case.w.shape)
    real = ~(case.kcache == workloads.SENTINEL_KEY_BF16).all(axis=1)
    case.kcache[real] = g.choice(_EXACT, size=(int(real.sum()), case.dim))
    return case


def _guided_variant(case):
    big = copy.copy(case)
    big.max_seq_len = FUSED_GUIDED_TOKENS // case.batch + 1
    cols = -(-big.max_seq_len // case.page_size)
    bt = np.zeros((case.block_table.shape[0], cols), np.int32)
    bt[:, :case.block_table.shape[1]] = case.block_table
    big.block_table = bt
    return big


def _fused(ops, case, sorted=False):
    import torch

    slots, sc = ops.idx_score_topk_fused_bf16(*_inputs(case), case.page_size, case.max_seq_len, case.k,
                                              return_scores=True, row_to_batch=_r2b(case), sorted=sorted)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_bf16_score_tolerance(ops, heads, page_size):
    import torch

    seed = 1200 + heads + page_size
    case = workloads.indexer_case(seed, batch=3, n_lo=1, n_hi=3000, page_size=page_size, k=64, heads=heads,
                                  fixed_lens=_lens(seed, 3, 1, 3000, first=(1,)), cache_dtype="bf16")
    out = ops.idx_score_bf16(*_inputs(case), case.page_size, case.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        check_scores(out[b, :n], rows[b], bsig)
        assert np.isnan(out[b, n:]).all(), "cells past n_b must stay untouched"


def test_bf16_score_exact_values(ops):
    import torch

    case = _exact_case(1301, batch=3, n_lo=500, n_hi=2000, page_size=64)
    out = ops.idx_score_bf16(*_inputs(case), case.page_size, case.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        assert np.array_equal(out[b, :n].astype(np.float64), case_scores(case, b))


@pytest.mark.parametrize("variant", ["resident", "guided"])
@pytest.mark.parametrize("page_size,heads,k", [(64, 64, 64), (16, 16, 300), (1, 32, 200), (48, 128, 700)])
def test_bf16_fused_exact_sets(ops, variant, page_size, heads, k):
    case = _exact_case(1400 + page_size + heads, batch=5, n_lo=1, n_hi=12000, page_size=page_size, heads=heads,
                       k=k, first=(0, k - 1, k))
    if variant == "guided":
        case = _guided_variant(case)
    slots, sc = _fused(ops, case)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(slots[b]), np.sort(ref_slots[b])), b
        m = min(int(case.seq_lens[b]), k)
        exp_s = np.sort(scores[b][ref_pos[b][:m]]) if m else np.zeros(0)
        assert np.array_equal(np.sort(sc[b][:m].astype(np.float64)), exp_s), b


@pytest.mark.parametrize("variant", ["resident", "guided"])
def test_bf16_fused_tolerance_random(ops, variant):
    case = workloads.indexer_case(1500, batch=6, n_lo=1, n_hi=20000, page_size=64, k=2048, cache_dtype="bf16")
    if variant == "guided":
        case = _guided_variant(case)
    slots, sc = _fused(ops, case)
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[b], case.page_size, n)
        ov = check_fused_row(slots[b], sc[b], rows[b], ts, case.k, batch_sigma=bsig)
        log(f"bf16 {variant} row {b} n={n} overlap={ov:.4f}")


def test_bf16_fused_sorted_exact_order(ops):
    case = _exact_case(1550, batch=4, n_lo=1, n_hi=9000, page_size=64, k=1000, first=(0, 999))
    slots, sc = _fused(ops, case, sorted=True)
    ref_slots, ref_pos, scores = oracle.fused_topk(case)
    for b in range(case.batch):
        assert np.array_equal(slots[b], ref_slots[b]), b
        m = min(int(case.seq_lens[b]), case.k)
        assert np.array_equal(sc[b][:m].astype(np.float64), scores[b][ref_pos[b][:m]]), b


def test_bf16_multi_query_fused(ops):
    """Multi-token decode rows from a bf16 cache: each row meets the
    tolerance criterion, and equals the run with the block-table rows copied
    out per query row."""
    case = workloads.multi_query_case(1600, requests=4, next_n=4, n_lo=3000, n_hi=20000, page_size=64, k=1024,
                                      cache_dtype="bf16")
    slots, sc = _fused(ops, case)
    flat = copy.copy(case)
    flat.block_table = np.ascontiguousarray(case.block_table[case.row_to_batch])
    flat.row_to_batch = None
    slots2, _ = _fused(ops, flat)
    assert np.array_equal(np.sort(slots, axis=1), np.sort(slots2, axis=1))
    rows = [case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[case.row_to_batch[b]], case.page_size, n)
        check_fused_row(slots[b], sc[b], rows[b], ts, case.k, batch_sigma=bsig)


@pytest.mark.parametrize("bs,top", [(128, 32), (64, 7)])
def test_bf16_block_exact(ops, bs, top):
    import torch

    case = _exact_case(1700 + bs, batch=4, n_lo=1, n_hi=9000, page_size=bs, k=0, block_size=bs, top_blocks=top,
                       first=(0, bs * top - 5, bs * top + 1))
    blocks, slots = ops.block_topk_bf16(*_inputs(case), case.page_size, case.max_seq_len, bs, top)
    torch.cuda.synchronize()
    blocks, slots = blocks.cpu().numpy(), slots.cpu().numpy()
    rb, rs, _, _ = oracle.block_topk(case)
    for b in range(case.batch):
        assert np.array_equal(np.sort(blocks[b]), np.sort(rb[b])), b
        got = {int(blocks[b, i]): slots[b, i * bs:(i + 1) * bs].tolist() for i in range(top) if blocks[b, i] >= 0}
        exp = {int(rb[b, i]): rs[b, i * bs:(i + 1) * bs].tolist() for i in range(top) if rb[b, i] >= 0}
        assert got == exp


@pytest.mark.parametrize("key_dtype", ["float32", "bfloat16"])
def test_bf16_cache_write_exact(ops, key_dtype):
    """The bf16 writer stores exactly the oracle's patterns (fp32 keys rounded
    to nearest even, bf16 keys as they are); negative slots are skipped."""
    import torch

    g = np.random.default_rng(1800)
    T, slots_n = 700, 2048
    keys = (g.standard_normal((T, 128)) * 3).astype(np.float32)
    keys[0, :8] = [1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 3e-39, 65504.0, 1e-30]  # ties, zeros, tiny
    slots = g.permutation(slots_n)[:T].astype(np.int32)
    slots[::37] = -1
    kc = np.full((slots_n, 128), 0x1234, np.uint16)
    if key_dtype == "bfloat16":
        kt = dev(keys).to(torch.bfloat16)
        ref_keys = kt.float().cpu().numpy()
    else:
        kt = dev(keys)
        ref_keys = keys
    kc_gpu = dev(kc)
    ops.idx_cache_write_bf16(kt, dev(slots), kc_gpu)
    torch.cuda.synchronize()
    ref = kc.copy()
    oracle.cache_write_bf16(ref_keys, slots, ref)
    assert np.array_equal(kc_gpu.cpu().numpy(), ref)


def test_bf16_written_cache_feeds_fused(ops):
    """Keys written by the bf16 writer give the fused call the same selection
    as the same keys written by the oracle."""
    import torch

    case = workloads.indexer_case(1900, batch=3, n_lo=500, n_hi=6000, page_size=64, k=256, cache_dtype="bf16")
    g = np.random.default_rng(1901)
    real = np.where(~(case.kcache == workloads.SENTINEL_KEY_BF16).all(axis=1))[0].astype(np.int32)
    keys = g.standard_normal((real.shape[0], 128)).astype(np.float32)
    ref = case.kcache.copy()
    oracle.cache_write_bf16(keys, real, ref)
    kc_gpu = dev(case.kcache)
    ops.idx_cache_write_bf16(dev(keys), dev(real), kc_gpu)
    torch.cuda.synchronize()
    assert np.array_equal(kc_gpu.cpu().numpy(), ref)
    written = copy.copy(case)
    written.kcache = ref
    slots, _ = _fused(ops, written)
    ref_slots, _, _ = oracle.fused_topk(written)
    rows = [case_scores(written, b) for b in range(written.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(written.batch):
        n = int(written.seq_lens[b])
        ts = oracle.token_slots(written.block_table[b], written.page_size, n)
        check_fused_row(slots[b], None, rows[b], ts, written.k, batch_sigma=bsig)


def test_bf16_decode_full_size(ops):
    """Fused decode B32 from a bf16 cache (the benchmarked configuration):
    every row meets the tolerance criterion."""
    from tests import _fullsize

    case = workloads.bf16_decode()
    log(f"case {case.name}")
    slots, sc = _fused(ops, case)
    _fullsize.run(_fullsize.fused_rows_task, _fullsize.fused_tasks(case, slots, sc), case.name)


def test_bf16_long_decode_full_size(ops):
    """Long decode B64 (n up to 327680) from a bf16 cache: every row against
    the oracle criterion, returned scores within the tolerance."""
    from tests import _fullsize

    case = workloads.bf16_long_decode()
    log(f"case {case.name} tokens={workloads.expected_tokens(case)}")
    slots, sc = _fused(ops, case)
    case.kcache = None  # the workers draw each row's keys again
    _fullsize.run(_fullsize.fused_rows_task, _fullsize.fused_tasks(case, slots, sc), case.name)
