"""GPU parity of idx_cache_write against the oracle's cache writer (bit-exact)."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.fp8 import E4M3FN_TABLE
from tests._helpers import check_fused_row, dev, log, rms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    from sparse_attention_indexer_fp8_amd import ops as _ops

    torch.cuda.set_device(0)
    return _ops


def _run(ops, keys_t, slots, num_slots):
    """Write keys through the GPU and the oracle into caches prefilled with a
    marker; return both (codes, scales) pairs."""
    import torch

    kc = torch.full((num_slots, 128), 0xAA, dtype=torch.uint8, device="cuda")
    ks = torch.full((num_slots,), -1.0, dtype=torch.float32, device="cuda")
    ops.idx_cache_write(keys_t, dev(slots), kc, ks)
    torch.cuda.synchronize()
    keys32 = keys_t.float().cpu().numpy()
    rk = np.full((num_slots, 128), 0xAA, np.uint8)
    rs = np.full(num_slots, -1.0, np.float32)
    oracle.cache_write(keys32[:, :128], slots, rk, rs)
    return (kc.cpu().numpy(), ks.cpu().numpy()), (rk, rs)


def _keys(seed, T, width=128):
    g = np.random.default_rng(seed)
    k = g.standard_normal((T, width)).astype(np.float32)
    k *= (2.0 ** g.integers(-30, 30, size=(T, 1))).astype(np.float32)   # magnitudes from 1e-9 to 1e9
    k[0] = 0.0                                                            # all-zero key
    k[1, :] = 0.0
    k[1, 5] = -3.0                                                        # one nonzero entry
    k[2] = np.float32(1e30) * np.sign(k[2])                               # huge, all equal magnitude
    return k


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_cache_write_bit_exact(ops, dtype):
    import torch

    T, S = 3000, 5000
    g = np.random.default_rng(11)
    slots = g.permutation(S)[:T].astype(np.int32)
    slots[g.random(T) < 0.1] = -1
    keys = torch.from_numpy(_keys(12, T)).to(getattr(torch, dtype)).cuda()
    log(f"cache write: T={T} dtype={dtype}")
    (gc, gs), (rc, rs) = _run(ops, keys, slots, S)
    assert np.array_equal(gs, rs)
    assert np.array_equal(gc, rc)


def test_cache_write_strided_keys(ops):
    import torch

    T, S = 700, 900
    wide = torch.from_numpy(_keys(13, T, width=256)).cuda()
    keys = wide[:, 64:192]                     # rows 256 apart, 128 wide
    slots = np.random.default_rng(14).permutation(S)[:T].astype(np.int32)
    (gc, gs), (rc, rs) = _run(ops, keys, slots, S)
    assert np.array_equal(gs, rs) and np.array_equal(gc, rc)


def test_encoder_on_every_code_and_boundary(ops):
    """Each key holds 448 (so the scale is exactly 1) and 127 test values:
    every finite code's value, every midpoint between adjacent codes and the
    fp32 neighbours of each midpoint, both signs. (Values past 448 would
    raise the key's scale; saturation is pinned on the oracle's encoder.)"""
    import torch

    pos = E4M3FN_TABLE[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2.0).astype(np.float32)
    vals = np.concatenate([pos.astype(np.float32), mid, np.nextafter(mid, np.float32(0)),
                           np.nextafter(mid, np.float32(1e9))])
    vals = np.concatenate([vals, -vals, np.float32([-0.0])])
    n = -(-vals.size // 127)
    buf = np.zeros((n, 128), np.float32)
    flat = np.zeros(n * 127, np.float32)
    flat[:vals.size] = vals
    buf[:, 1:] = flat.reshape(n, 127)
    buf[:, 0] = 448.0
    keys = torch.from_numpy(buf).cuda()
    slots = np.arange(n, dtype=np.int32)
    (gc, gs), (rc, rs) = _run(ops, keys, slots, n)
    assert (gs == 1.0).all() and (rs == 1.0).all()
    assert np.array_equal(gc, rc)


def test_written_cache_feeds_the_indexer(ops):
    """Keys written by idx_cache_write score through idx_score_topk_fused as
    the oracle scores the same cache."""
    import torch

    case = workloads.indexer_case(15, batch=4, n_lo=100, n_hi=5000, page_size=64, k=256)
    g = np.random.default_rng(16)
    n_slots = case.kcache.shape[0]
    real = np.flatnonzero(case.k_scale < workloads.SENTINEL_KEY_SCALE).astype(np.int32)
    keys = g.standard_normal((real.size, 128)).astype(np.float32)
    kc = dev(case.kcache)
    ks = dev(case.k_scale)
    ops.idx_cache_write(torch.from_numpy(keys).cuda(), dev(real), kc, ks)
    torch.cuda.synchronize()
    oracle.cache_write(keys, real, case.kcache, case.k_scale)      # the oracle's view of the same cache
    assert np.array_equal(kc.cpu().numpy(), case.kcache) and np.array_equal(ks.cpu().numpy(), case.k_scale)
    slots, sc = ops.idx_score_topk_fused(dev(case.q), dev(case.q_scale), dev(case.w), kc, ks,
                                         dev(case.block_table), dev(case.seq_lens), case.page_size,
                                         case.max_seq_len, case.k, return_scores=True)
    torch.cuda.synchronize()
    slots, sc = slots.cpu().numpy(), sc.cpu().numpy()
    rows = [oracle.indexer.case_scores(case, b) for b in range(case.batch)]
    bsig = rms(np.concatenate(rows))
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        ts = oracle.token_slots(case.block_table[b], case.page_size, n)
        check_fused_row(slots[b], sc[b], rows[b], ts, case.k, batch_sigma=bsig)
    assert n_slots == case.kcache.shape[0]
