"""Shared helpers of the GPU parity tests (comparison logic only)."""
from __future__ import annotations

import sys

import numpy as np

import oracle

# Score tolerance: relative 1e-3 with a per-row floor sigma_b (RMS of the row's
# oracle scores), so that cancellation near zero does not make the relative
# test ill-posed. A row with fewer than MIN_ROW_FOR_SIGMA tokens has no scale
# of its own (one token's RMS is its own |S|), so it takes the RMS of the
# oracle scores of every row of the call.
REL_TOL = 1e-3
MIN_ROW_FOR_SIGMA = 64


def rms(S) -> float:
    S = np.asarray(S, dtype=np.float64)
    return float(np.sqrt(np.mean(S * S))) if S.size else 0.0


def row_sigma(S, batch_sigma=None) -> float:
    S = np.asarray(S, dtype=np.float64)
    if S.size >= MIN_ROW_FOR_SIGMA or batch_sigma is None:
        return rms(S)
    return float(batch_sigma)


def dev(a, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def sorted_rows(a: np.ndarray) -> np.ndarray:
    return np.sort(np.asarray(a, dtype=np.int64), axis=1)


def positions_from_slots(slots_row: np.ndarray, tok_slots: np.ndarray) -> np.ndarray:
    """Invert the token -> slot map of one row (slots are distinct)."""
    order = np.argsort(tok_slots)
    s_sorted = tok_slots[order]
    valid = slots_row[slots_row >= 0]
    idx = np.searchsorted(s_sorted, valid)
    assert (idx < s_sorted.shape[0]).all(), "slot outside the row's tokens"
    assert (s_sorted[idx] == valid).all(), "slot outside the row's tokens"
    return order[idx]


def check_fused_row(slots_row, scores_row, S, tok_slots, k, min_overlap=0.97, batch_sigma=None):
    """Fused-path acceptance of one row. Returns the overlap with the oracle's exact set.

    - exactly min(n, k) valid slots, distinct, all mapping to the row's tokens,
      -1 in the tail;
    - every selected token's oracle score >= oracle k-th score - tol;
    - returned scores (if any) within tol of the oracle scores.
    """
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    m = min(n, k)
    slots_row = np.asarray(slots_row, dtype=np.int64)
    assert (slots_row[:m] >= 0).all() and (slots_row[m:] == -1).all(), "valid-count / padding"
    pos = positions_from_slots(slots_row[:m], tok_slots)
    assert np.unique(pos).shape[0] == m, "duplicate selection"
    if m == 0:
        return 1.0
    sigma = row_sigma(S, batch_sigma)
    kth = float(np.partition(S, n - m)[n - m])
    tol_k = REL_TOL * max(abs(kth), sigma)
    assert (S[pos] >= kth - tol_k).all(), f"selected below k-th - tol: {S[pos].min()} < {kth - tol_k}"
    if scores_row is not None:
        sc = np.asarray(scores_row[:m], dtype=np.float64)
        tol = REL_TOL * np.maximum(np.abs(S[pos]), sigma)
        err = np.abs(sc - S[pos])
        assert (err <= tol).all(), f"score error {err.max()} above tolerance"
        assert (np.asarray(scores_row[m:]) == -np.inf).all()
    exact = oracle.topk_order(S, k)[:m]
    overlap = np.intersect1d(exact, pos).shape[0] / m
    assert overlap >= min_overlap, f"overlap with the exact set {overlap}"
    return overlap


def check_scores(S_gpu, S, batch_sigma=None):
    S = np.asarray(S, dtype=np.float64)
    sigma = row_sigma(S, batch_sigma)
    tol = REL_TOL * np.maximum(np.abs(S), sigma)
    err = np.abs(np.asarray(S_gpu, dtype=np.float64) - S)
    assert (err <= tol).all(), f"max score error {err.max()} (tol at worst {tol[np.argmax(err)]})"
    return float((err / np.maximum(np.abs(S), 1e-30)).max()) if S.size else 0.0
