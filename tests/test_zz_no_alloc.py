"""idx_score_topk_fused_noalloc (built-in workspace) against idx_score_topk_fused
(caller workspace): the same outputs, call after call, on the same GPU.

Two calls in a row, the second with a smaller input, for decode-size
batches and for batches of a few million tokens, plain and sorted output;
each result also meets the oracle criterion.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle.indexer import case_scores
from tests._helpers import check_fused_row, dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    from sparse_attention_indexer_fp8_amd import ops as _ops

    torch.cuda.set_device(0)
    return _ops


def _ins(case):
    return (dev(case.q), dev(case.q_scale), dev(case.w), dev(case.kcache), dev(case.k_scale),
            dev(case.block_table), dev(case.seq_lens))


def _both(ops, case, sorted_out):
    import torch

    ins = _ins(case)
    ref, ref_sc = ops.idx_score_topk_fused(*ins, case.page_size, case.max_seq_len, case.k, return_scores=True,
                                           workspace=ops.Workspace(), sorted=sorted_out)
    out = torch.full((case.batch, case.k), 7, dtype=torch.int32, device="cuda")
    sc = torch.full((case.batch, case.k), 7.0, dtype=torch.float32, device="cuda")
    ops.idx_score_topk_fused_noalloc(*ins, case.page_size, case.max_seq_len, case.k, out, sc, sorted=sorted_out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), ref_sc.cpu().numpy(), out.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("sorted_out", [False, True])
@pytest.mark.parametrize("variant", ["decode", "large"])
def test_noalloc_equals_workspace_call(ops, variant, sorted_out):
    if variant == "decode":
        cases = [workloads.indexer_case(951, batch=16, n_lo=4000, n_hi=20000, page_size=64, k=1024),
                 workloads.indexer_case(952, batch=5, n_lo=100, n_hi=3000, page_size=64, k=300)]
    else:  # about two million tokens per call
        cases = [workloads.indexer_case(953, batch=9, n_lo=200000, n_hi=260000, page_size=64, k=2048),
                 workloads.indexer_case(954, batch=8, n_lo=150000, n_hi=270000, page_size=64, k=512)]
    for i, case in enumerate(cases):
        log(f"{variant} sorted={sorted_out} call {i}: batch={case.batch} max_seq_len={case.max_seq_len} k={case.k}")
        ref, ref_sc, out, sc = _both(ops, case, sorted_out)
        if sorted_out:
            assert np.array_equal(out, ref) and np.array_equal(sc, ref_sc)
        else:
            # the order within a row is unspecified: compare (slot, score) sets
            for b in range(case.batch):
                assert dict(zip(out[b].tolist(), sc[b].tolist())) == dict(zip(ref[b].tolist(), ref_sc[b].tolist()))
        for b in range(case.batch):
            n = int(case.seq_lens[b])
            ts = oracle.token_slots(case.block_table[b], case.page_size, n)
            check_fused_row(out[b], sc[b], case_scores(case, b), ts, case.k)


def test_noalloc_refuses_larger_than_builtin(ops):
    import torch
    from sparse_attention_indexer_fp8_amd import _lib

    case = workloads.indexer_case(955, batch=2, n_lo=100, n_hi=200, page_size=64, k=64)
    big = 1 << 20
    bt = torch.zeros((64, big // 64), dtype=torch.int32, device="cuda")
    ins = list(_ins(case))
    q = torch.zeros((64, case.heads, case.dim), dtype=torch.uint8, device="cuda")
    ins[0], ins[1], ins[2] = q, torch.ones(64, device="cuda"), torch.ones((64, case.heads), device="cuda")
    ins[5], ins[6] = bt, torch.full((64,), 100, dtype=torch.int32, device="cuda")
    out = torch.empty((64, 2048), dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.IdxTopkError) as e:
        ops.idx_score_topk_fused_noalloc(*ins, 64, big, 2048, out)
    assert e.value.status == _lib.IDXTOPK_EWORKSPACE
