"""Per-row regeneration of the seeded inputs equals the whole-case generators.

The every-row parity checks of the full-size workloads draw each row again in
worker processes (``workloads.window_values``, ``workloads.row_inputs``)
instead of shipping gigabytes of inputs to them. These tests show that the
rows drawn that way are byte for byte the rows of the whole case the GPU
reads.
"""
import numpy as np
import pytest

import oracle
import workloads


def test_window_values_equal_packed_rows():
    case = workloads.packed_prefill_case(seed=77, prefix0=900, new_tokens=40, k=16)
    for i in range(case.rows):
        rs, n = int(case.row_starts[i]), int(case.seq_lens[i])
        v = workloads.window_values(77, i, n, 0.01)
        assert np.array_equal(v, case.scores[i, rs:rs + n]), i
    dec = workloads.decode_rows_case(seed=78, rows=5, stride=700, n_lo=10, n_hi=700, k=8)
    for i in range(dec.rows):
        n = int(dec.seq_lens[i])
        assert np.array_equal(workloads.window_values(78, i, n, 0.05), dec.scores[i, :n]), i


def _check_rows(case):
    spec = workloads.row_spec(case)
    cache = {}
    for b in range(case.batch):
        r = workloads.row_inputs(spec, b, cache)
        assert r.n == int(case.seq_lens[b])
        assert np.array_equal(r.q, case.q[b]) and np.array_equal(r.w, case.w[b]), b
        assert r.q_scale == case.q_scale[b], b
        prow = b if case.row_to_batch is None else int(case.row_to_batch[b])
        ts = oracle.token_slots(case.block_table[prow], case.page_size, r.n)
        assert np.array_equal(r.keys[:r.n], case.kcache[ts]), b
        if case.cache_dtype == "fp8":
            assert np.array_equal(r.k_scale[:r.n], case.k_scale[ts]), b


@pytest.mark.parametrize("cache_dtype", ["fp8", "bf16"])
def test_row_inputs_equal_indexer_case(cache_dtype):
    case = workloads.indexer_case(79, batch=4, n_lo=0, n_hi=700, page_size=16, k=32, heads=16,
                                  fixed_lens=np.array([0, 1, 333, 700], np.int32), cache_dtype=cache_dtype)
    _check_rows(case)


def test_row_inputs_equal_multi_query_case():
    case = workloads.multi_query_case(80, requests=3, next_n=4, n_lo=5, n_hi=900, page_size=64, k=16, heads=32)
    _check_rows(case)
