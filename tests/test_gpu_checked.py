"""The checked build (libidxtopk_checked.so: device-side checks of the callers'
preconditions and of internal bounds) on the full-size workloads, in the
launch configurations the benchmark times: no check fires, and every output
equals the release build's. Then one precondition broken on purpose from the
host, in a way that keeps every access in bounds, is reported."""
import os

import numpy as np
import pytest

import workloads
from tests._helpers import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import torch
    from sparse_attention_indexer_fp8_amd import _lib, ops

    torch.cuda.set_device(0)
    assert os.path.exists(_lib.CHECKED_LIB_PATH), "libidxtopk_checked.so is not built (build() builds it)"
    chk = _lib.load(_lib.CHECKED_LIB_PATH)
    assert chk.idxtopk_check_status(1) == 0
    return _lib, ops, chk


def _both(libs, fn):
    """fn() with the release build, then with the checked build: the outputs
    (numpy arrays) and the checked build's status."""
    import torch

    _lib, ops, chk = libs
    rel = fn()
    torch.cuda.synchronize()
    with _lib.using(_lib.CHECKED_LIB_PATH):
        got = fn()
        torch.cuda.synchronize()
    return rel, got, int(chk.idxtopk_check_status(1))


def _same(a, b):
    if isinstance(a, tuple):
        return all(_same(x, y) for x, y in zip(a, b))
    return np.array_equal(a, b)


def _ins(case):
    return (dev(case.q), dev(case.q_scale), dev(case.w), dev(case.kcache), dev(case.k_scale),
            dev(case.block_table), dev(case.seq_lens))


def test_checked_packed_prefill_topk(libs):
    _lib, ops, _ = libs
    case = workloads.c3_packed_prefill()
    args = (dev(case.scores), dev(case.seq_lens), case.k, dev(case.row_starts), dev(case.row_to_batch),
            dev(case.page_table), 1)
    del case
    for sorted_out in (False, True):
        rel, got, st = _both(libs, lambda: ops.topk_rows(*args, sorted=sorted_out).cpu().numpy())
        log(f"packed prefill sorted={sorted_out}: check status {st:#x}")
        assert st == 0
        assert _same(np.sort(rel, axis=1), np.sort(got, axis=1))


def test_checked_decode_topk(libs):
    _lib, ops, _ = libs
    case = workloads.c1_decode_topk()
    args = (dev(case.scores), dev(case.seq_lens), case.k, None, None, dev(case.page_table), 1)
    rel, got, st = _both(libs, lambda: ops.topk_rows(*args).cpu().numpy())
    assert st == 0 and _same(np.sort(rel, axis=1), np.sort(got, axis=1))


@pytest.mark.parametrize("name", ["c2", "c5", "mtp"])
def test_checked_fused(libs, name):
    _lib, ops, _ = libs
    case = {"c2": workloads.c2_fused_decode, "c5": workloads.c5_long_decode, "mtp": workloads.mtp_decode}[name]()
    ins = _ins(case)
    r2b = None if case.row_to_batch is None else dev(case.row_to_batch)

    def run():
        s, v = ops.idx_score_topk_fused(*ins, case.page_size, case.max_seq_len, case.k, return_scores=True,
                                        row_to_batch=r2b)
        return s.cpu().numpy(), v.cpu().numpy()

    rel, got, st = _both(libs, run)
    log(f"fused {name}: check status {st:#x}")
    assert st == 0
    for b in range(case.batch):
        assert dict(zip(rel[0][b].tolist(), rel[1][b].tolist())) == dict(zip(got[0][b].tolist(), got[1][b].tolist()))


@pytest.mark.parametrize("per_head", [False, True])
def test_checked_block_sparse(libs, per_head):
    _lib, ops, _ = libs
    case = workloads.c4_block_sparse()
    ins = _ins(case)
    fn = ops.block_topk_heads if per_head else ops.block_topk

    def run():
        b, s = fn(*ins, case.page_size, case.max_seq_len, case.block_size, case.top_blocks)
        return b.cpu().numpy(), s.cpu().numpy()

    rel, got, st = _both(libs, run)
    assert st == 0
    assert _same(np.sort(rel[0], axis=-1), np.sort(got[0], axis=-1))


def test_checked_prefill_indexer(libs):
    import torch

    _lib, ops, _ = libs
    case = workloads.prefill_indexer()
    ins = _ins(case)
    r2b = dev(case.row_to_batch)

    def run():
        sc = ops.idx_score_fp8(*ins, case.page_size, case.max_seq_len, row_to_batch=r2b)
        out = ops.topk_rows(sc, ins[6], case.k, row_to_batch=r2b, page_table=ins[5], page_size=case.page_size)
        rows = sc[::997].cpu().numpy()
        del sc
        torch.cuda.empty_cache()
        return out.cpu().numpy(), rows

    rel, got, st = _both(libs, run)
    assert st == 0
    assert _same(np.sort(rel[0], axis=1), np.sort(got[0], axis=1))
    assert np.array_equal(np.nan_to_num(rel[1]), np.nan_to_num(got[1]))


def test_checked_reports_broken_preconditions(libs):
    """Forced from the host, every access staying in bounds: a window that
    runs past its own row into the next one (topk_rows), and a row longer
    than the max_seq_len the caller promised, with every buffer sized for the
    longer row (idx_score_fp8, which then scores only up to the bound). Each
    call completes and its bit is reported."""
    import torch

    _lib, ops, chk = libs
    with _lib.using(_lib.CHECKED_LIB_PATH):
        buf = np.random.default_rng(3).standard_normal((4, 1000)).astype(np.float32)
        ops.topk_rows(dev(buf), dev(np.array([100, 100, 100, 100], np.int32)), 10,
                      row_starts=dev(np.array([0, 950, 0, 0], np.int32)))
        torch.cuda.synchronize()
        st = int(chk.idxtopk_check_status(1))
        assert st == 0x1, hex(st)  # IDXTOPK_CHK_WINDOW
        case = workloads.indexer_case(31, batch=2, n_lo=3000, n_hi=3000, page_size=64, k=64, heads=16)
        out = torch.zeros((2, 3000), dtype=torch.float32, device="cuda")
        ops.idx_score_fp8(*_ins(case), case.page_size, 2000, out=out)
        torch.cuda.synchronize()
        st = int(chk.idxtopk_check_status(1))
        assert st == 0x8, hex(st)  # IDXTOPK_CHK_SEQ_LEN
    assert int(chk.idxtopk_check_status(1)) == 0
