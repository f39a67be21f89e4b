"""Plain float64 definition of the indexer top-k path (oracle; test infrastructure only).

Notation: row b (a query token), its window length n_b (the number of visible
keys), row-local key positions j = 0..n_b-1, physical KV-cache slots, page
size P.

Readings where the pages are silent are marked READING. The same readings are
listed in the repository's design notes.
"""
from __future__ import annotations

import numpy as np

from .bf16 import decode_bf16, encode_bf16
from .fp8 import decode_e4m3fn


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Addressing
# ---------------------------------------------------------------------------


def token_slots(bt_row: np.ndarray, page_size: int, n: int) -> np.ndarray:
    """Physical slot of each of the first n tokens of one row.

    [ATOM-1473], decode-kernel diff in the review thread: the kernel walks the
    row's blocks, reads ``page = bt_row[blk]`` (widened to int64) and
    addresses tokens ``blk * BLOCK_SIZE_K + off`` inside that page. So token j
    lives at slot ``bt_row[j // P] * P + j % P``.
    """
    P = int(page_size)
    j = np.arange(int(n), dtype=np.int64)
    return np.asarray(bt_row, dtype=np.int64)[j // P] * P + j % P


def page_transform(positions: np.ndarray, pt_row: np.ndarray, page_size: int) -> np.ndarray:
    """Map row-local positions to physical slots; -1 stays -1.

    [SGL-37889], Motivation and Modifications: the top-k "transform" maps the
    selected row-local index through the page table, and with page_size 1
    the table is the wide per-token table. For a general page size the same
    slot rule as ``token_slots`` applies.
    """
    P = int(page_size)
    pos = np.asarray(positions, dtype=np.int64)
    out = np.full(pos.shape, -1, dtype=np.int64)
    ok = pos >= 0
    p = pos[ok]
    out[ok] = np.asarray(pt_row, dtype=np.int64)[p // P] * P + p % P
    return out


def row_window(scores: np.ndarray, i: int, seq_lens, row_starts=None) -> np.ndarray:
    """fp32 window of row i, widened exactly to float64.

    [SGL-37889], Modifications, addressing table: without row_starts row i
    reads ``scores[i, :seq_lens[i]]``; with it, row i reads
    ``scores[i, row_starts[i] : row_starts[i] + seq_lens[i]]``.
    """
    n = int(seq_lens[i])
    rs = 0 if row_starts is None else int(row_starts[i])
    return _f64(scores[i, rs:rs + n])


def page_row(i: int, row_to_batch=None) -> int:
    """[SGL-37889], Modifications: page-table row is ``row_to_batch[i]`` if given, else i."""
    return int(i) if row_to_batch is None else int(row_to_batch[i])


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------


def topk_order(values: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k best values of one row, padded with -1.

    Definition: sort the whole row by value, descending, with a STABLE sort,
    so equal values keep ascending position; keep the first min(k, n); fill
    the rest of the k outputs with -1. Values compare as IEEE numbers:
    -0.0 == +0.0, +-inf allowed. NaN is outside the input domain and raises.

    READING: the pages give no tie rule. Ties go to the lower position, and
    rows shorter than k are padded with -1. [SGL-37889], Modifications: the
    selected index stays row-local until the transform.

    The outputs come in that sort's order (value descending, equal values by
    ascending position, padding last), which is also the order of the
    library's sorted-output variant.
    """
    v = _f64(values).reshape(-1)
    if np.isnan(v).any():
        raise ValueError("NaN score in top-k input")
    k = int(k)
    out = np.full(k, -1, dtype=np.int64)
    m = min(k, v.shape[0])
    if m > 0:
        order = np.argsort(-v, kind="stable")
        out[:m] = order[:m]
    return out


def topk_rows(scores: np.ndarray, seq_lens, k: int, row_starts=None, row_to_batch=None,
              page_table=None, page_size: int = 1, rows=None, kv_offset=None) -> np.ndarray:
    """Top-k with page transform over an fp32 score buffer, row by row.

    [SGL-37889], Modifications: each row's window comes from the addressing
    table (``row_window``), the best k row-local positions are kept
    (``topk_order``), and the page-table row ``page_row`` maps them to slots
    (``page_transform``). With ``page_table=None`` the row-local positions
    are returned. ``rows`` picks a subset of rows (default: all).

    ``kv_offset`` (per row, default 0): [SGL-37889] sends chunked-prefix-cache
    extend, where the plan covers the whole forward but a call sees one
    chunk, to its legacy path. READING: the window of row i then holds KV
    positions kv_offset[i] .. kv_offset[i] + seq_lens[i] - 1, so each kept
    window position gets kv_offset[i] added before the transform; -1
    padding stays -1.
    """
    rows = range(int(np.asarray(seq_lens).shape[0])) if rows is None else list(rows)
    out = []
    for i in rows:
        pos = topk_order(row_window(scores, i, seq_lens, row_starts), k)
        if kv_offset is not None:
            pos = np.where(pos >= 0, pos + int(kv_offset[i]), -1)
        if page_table is not None:
            pos = page_transform(pos, page_table[page_row(i, row_to_batch)], page_size)
        out.append(pos)
    return np.stack(out) if out else np.zeros((0, int(k)), np.int64)


# ---------------------------------------------------------------------------
# Scoring
# ---------------------------------------------------------------------------


def index_scores(q_b, q_scale_b, w_b, kcache, k_scale, bt_row, page_size: int, n: int) -> np.ndarray:
    """Indexer score of every visible key of one row, in float64.

    S[j] = sum_h w[h] * max(0, dot[h, j] * s_q * s_k[slot_j]),
    dot[h, j] = sum_d qhat[h, d] * khat[slot_j, d].

    [ATOM-1473], Pull request overview and commit "fp8 index score calculate
    in fp8": queries and index keys are fp8 and the dot product is taken on
    fp8 operands. The key of token j is fetched through the block table
    (``token_slots``).

    READING: the pages name the index score without writing it out. This
    library's score is the weighted-ReLU head sum above, with one fp32 scale
    per query row, one per cached token, and one fp32 weight per (row, head).
    The scales multiply the dot before the ReLU.

    The dot is exact in float64: every product of two e4m3 values is an
    integer multiple of 2^-18 below 448^2, so sums of 128 of them need at most
    43 significant bits.
    """
    qd = decode_e4m3fn(q_b)  # [H, D]
    slots = token_slots(bt_row, page_size, n)
    kd = decode_e4m3fn(np.asarray(kcache)[slots])  # [n, D]
    dot = kd @ qd.T  # [n, H]
    sk = _f64(np.asarray(k_scale)[slots])
    logits = dot * float(q_scale_b) * sk[:, None]
    return (np.maximum(logits, 0.0) * _f64(w_b)[None, :]).sum(axis=1)


def index_scores_bf16(q_b, w_b, kcache, bt_row, page_size: int, n: int) -> np.ndarray:
    """Indexer score of every visible key of one row from a bf16 index cache,
    in float64: S[j] = sum_h w[h] * max(0, sum_d q[h, d] * k[slot_j, d]).

    [ATOM-1473], Pull request overview: the index cache takes the model's
    dtype when the KV cache is not fp8. READING: that dtype is bf16, the
    queries are bf16 too, and there are no scales; the score is the same
    weighted-ReLU head sum as the fp8 one with unit scales. ``q_b`` [H, D]
    and ``kcache`` [slots, D] hold bf16 bit patterns.

    A product of two bf16 values has at most 16 significant bits and is
    exact in float64; the sum of 128 of them is exact whenever their
    exponents span fewer than 30 binades (always for the small-integer
    inputs of the exact tests), and otherwise within float64 rounding, far
    below any fp32 tolerance.
    """
    qd = decode_bf16(q_b)  # [H, D]
    slots = token_slots(bt_row, page_size, n)
    kd = decode_bf16(np.asarray(kcache)[slots])  # [n, D]
    dot = kd @ qd.T  # [n, H]
    return (np.maximum(dot, 0.0) * _f64(w_b)[None, :]).sum(axis=1)


def index_head_scores(q_b, q_scale_b, w_b, kcache, k_scale, bt_row, page_size: int, n: int) -> np.ndarray:
    """Each head's term of the fp8 index score, [n, H] in float64:
    T[j, h] = w[h] * max(0, s_q * s_k[slot_j] * dot(qhat_h, khat[slot_j])).

    The index score is the sum of these terms over the heads
    (``index_scores``). [ATOM-1473], Pull request overview: the partial top-k
    kernel's grid has an index-head axis. READING for the per-head variant:
    each head ranks keys by its own term.
    """
    qd = decode_e4m3fn(q_b)  # [H, D]
    slots = token_slots(bt_row, page_size, n)
    kd = decode_e4m3fn(np.asarray(kcache)[slots])  # [n, D]
    logits = (kd @ qd.T) * float(q_scale_b) * _f64(np.asarray(k_scale)[slots])[:, None]
    return np.maximum(logits, 0.0) * _f64(w_b)[None, :]


def case_bt_row(case, b: int) -> np.ndarray:
    """Block-table row of query row b: ``row_to_batch[b]`` if the case has one,
    else b. Several query rows may share a block-table row (multi-token
    decode: one row per query token of a request, each with its own causal
    length in ``seq_lens``). Same addressing rule as ``page_row`` ([SGL-37889],
    Modifications)."""
    return case.block_table[page_row(b, getattr(case, "row_to_batch", None))]


def case_scores(case, b: int) -> np.ndarray:
    """``index_scores`` (or ``index_scores_bf16`` for a bf16 index cache) of
    row b of a workloads.IndexerCase."""
    if getattr(case, "cache_dtype", "fp8") == "bf16":
        return index_scores_bf16(case.q[b], case.w[b], case.kcache, case_bt_row(case, b), case.page_size,
                                 int(case.seq_lens[b]))
    return index_scores(case.q[b], case.q_scale[b], case.w[b], case.kcache, case.k_scale,
                        case_bt_row(case, b), case.page_size, int(case.seq_lens[b]))


def fused_topk(case, rows=None, k=None):
    """Score + top-k + page transform for decode rows of an indexer case.

    [ATOM-1473], Pull request overview: the decode indexer scores the fp8
    index cache and keeps a top-k of key positions (the fused kernel only
    removes the intermediate score tensor, so it computes the same thing).
    Returns (slots [R, k] int64, positions [R, k] int64, scores list of the
    float64 score rows).
    """
    k = int(case.k if k is None else k)
    rows = range(case.batch) if rows is None else list(rows)
    slots, positions, scores = [], [], []
    for b in rows:
        S = case_scores(case, b)
        pos = topk_order(S, k)
        positions.append(pos)
        slots.append(page_transform(pos, case_bt_row(case, b), case.page_size))
        scores.append(S)
    return np.stack(slots), np.stack(positions), scores


# ---------------------------------------------------------------------------
# Block-sparse variant
# ---------------------------------------------------------------------------


def block_scores(S: np.ndarray, block_size: int) -> np.ndarray:
    """Block score = max of the token scores of the block's visible tokens.

    [ATOM-1282], title and launch script (--block-size 128): key positions are
    grouped in 128-token blocks and blocks are selected. [ATOM-1473], Pull
    request overview: an index block-score kernel produces the block scores.
    READING: the block score is the max over the block's visible tokens;
    block c covers tokens [c*bs, min((c+1)*bs, n)), for c < ceil(n / bs).
    """
    S = _f64(S)
    n = S.shape[0]
    bs = int(block_size)
    nb = -(-n // bs)
    return np.array([S[c * bs:min((c + 1) * bs, n)].max() for c in range(nb)], dtype=np.float64)


def block_topk(case, rows=None, block_size=None, top_blocks=None):
    """Top blocks per row, as physical block ids and expanded slot lists.

    [ATOM-1282], title: the sparse block list is built inside the top-k
    step. READING: keep the top_blocks best blocks (ties to the lower block
    id, via ``topk_order``). With block_size == page_size, block c is page
    ``bt[b, c]`` and its slots are ``page * bs + t`` for its visible tokens t.
    Past n_b the slot list holds -1, and missing blocks give -1 block ids and
    -1 slots.

    Returns (blocks [R, top] int64, slots [R, top*bs] int64, logical block ids
    [R, top] int64, block-score rows).
    """
    bs = int(case.block_size if block_size is None else block_size)
    top = int(case.top_blocks if top_blocks is None else top_blocks)
    rows = range(case.batch) if rows is None else list(rows)
    blocks, slot_lists, logical, bscores = [], [], [], []
    for b in rows:
        n = int(case.seq_lens[b])
        S = case_scores(case, b)
        bsv = block_scores(S, bs) if n > 0 else np.zeros(0)
        sel = topk_order(bsv, top)
        bt_row = case_bt_row(case, b)
        tok_slots = token_slots(bt_row, case.page_size, n)
        phys = np.full(top, -1, np.int64)
        sl = np.full(top * bs, -1, np.int64)
        for i, c in enumerate(sel):
            if c < 0:
                continue
            phys[i] = int(bt_row[c * bs // case.page_size])
            lo, hi = c * bs, min((c + 1) * bs, n)
            sl[i * bs:i * bs + (hi - lo)] = tok_slots[lo:hi]
        blocks.append(phys)
        slot_lists.append(sl)
        logical.append(sel)
        bscores.append(bsv)
    return np.stack(blocks), np.stack(slot_lists), np.stack(logical), bscores


def block_topk_heads(case, rows=None, block_size=None, top_blocks=None):
    """Per-head block selection: for every row b and head h, the top_blocks
    best blocks by the head's own block score (the max of its term
    ``index_head_scores`` over the block's visible tokens; ties to the lower
    block id), as physical block ids and expanded slot lists, laid out
    [R, H, top] and [R, H, top*bs] (fp8 index cache).

    READING: [ATOM-1473]'s partial top-k grid runs over (query row, index
    head, chunk); selecting per head is read as every head keeping its own
    blocks, with the block rule of ``block_scores``.
    """
    bs = int(case.block_size if block_size is None else block_size)
    top = int(case.top_blocks if top_blocks is None else top_blocks)
    rows = range(case.batch) if rows is None else list(rows)
    H = case.heads
    blocks = np.full((len(rows), H, top), -1, np.int64)
    slot_lists = np.full((len(rows), H, top * bs), -1, np.int64)
    for ri, b in enumerate(rows):
        n = int(case.seq_lens[b])
        bt_row = case_bt_row(case, b)
        tok_slots = token_slots(bt_row, case.page_size, n)
        T = index_head_scores(case.q[b], case.q_scale[b], case.w[b], case.kcache, case.k_scale, bt_row,
                              case.page_size, n)
        for h in range(H):
            bsv = block_scores(T[:, h], bs) if n > 0 else np.zeros(0)
            for i, c in enumerate(topk_order(bsv, top)):
                if c < 0:
                    continue
                blocks[ri, h, i] = int(bt_row[c * bs // case.page_size])
                lo, hi = c * bs, min((c + 1) * bs, n)
                slot_lists[ri, h, i * bs:i * bs + (hi - lo)] = tok_slots[lo:hi]
    return blocks, slot_lists


# ---------------------------------------------------------------------------
# Index-key cache writer
# ---------------------------------------------------------------------------


def quantize_key(k_row):
    """One token's cache entry: scale = fp32(max|k| / 448), or 1 if that is
    0; codes = e4m3fn(fp32(k / scale)).

    [ATOM-1473], Pull request overview and the attention-layer diffs: the
    index-key cache is allocated in fp8 and written with a key scale.
    READING: one fp32 scale per cached token, chosen so the largest
    magnitude maps to 448 (the e4m3 maximum); both divisions are fp32
    divisions rounded to nearest, then ``encode_e4m3fn``. This is the format
    every scoring function here reads (``index_scores``).
    """
    from .fp8 import encode_e4m3fn

    k = np.asarray(k_row, dtype=np.float32)
    m = np.float32(np.abs(k).max()) if k.size else np.float32(0.0)
    scale = np.float32(m / np.float32(448.0))
    if not scale > 0:
        scale = np.float32(1.0)
    return encode_e4m3fn((k / scale).astype(np.float32)), scale


def cache_write(keys, slot_mapping, kcache, k_scale) -> None:
    """Quantize each new key (``quantize_key``) and store it at its slot:
    kcache[slot] = codes, k_scale[slot] = scale. Tokens with a negative slot
    are skipped. Writes into ``kcache`` and ``k_scale`` in place."""
    keys = np.asarray(keys, dtype=np.float32)
    for t, s in enumerate(np.asarray(slot_mapping).astype(np.int64)):
        if s < 0:
            continue
        codes, scale = quantize_key(keys[t])
        kcache[s] = codes
        k_scale[s] = scale


def cache_write_bf16(keys, slot_mapping, kcache) -> None:
    """bf16 index cache writer: kcache[slot] = the nearest bf16 of each key
    value (``encode_bf16``: round to nearest, ties to even), no scale. Tokens
    with a negative slot are skipped. Writes into ``kcache`` (uint16) in
    place. [ATOM-1473], Pull request overview: the non-fp8 index cache holds
    keys in the model's dtype. A bf16 key is stored as it is."""
    keys = np.asarray(keys, dtype=np.float64)
    for t, s in enumerate(np.asarray(slot_mapping).astype(np.int64)):
        if s < 0:
            continue
        kcache[s] = encode_bf16(keys[t])
