"""Seeded synthetic inputs for the sparse-attention indexer top-k path.

This module only draws random inputs and lays them out in memory. It holds
none of the method's arithmetic (no decoding, no dot products, no scoring, no
selection), so the CPU oracle and the HIP path can both consume its output
without sharing any computation.

Every random draw comes from ``numpy.random.default_rng([seed, stream, row])``
so any single row can be regenerated on its own. The e4m3 bytes of queries and
index keys are produced by torch's ``float8_e4m3fn`` conversion (a library
cast, after clamping to the format's finite range of +-448).

Workload shapes follow the pages:
  * ROCm/ATOM PR 1473 ("enable minimax m3 fp8 index cache and fuse
    index_score_kernel with partial_topk kernel"), the decode kernel's paged
    index-key cache walked through a block table, 64-token pages;
  * sgl-project/sglang PR 37889 ("Enable GLM DSA prefill top-k to the v2
    kernel"), section Modifications: one packed fp32 score buffer shared by all
    requests of an extend batch, addressed through row_starts / row_to_batch,
    ISL 70000 and 16384-row launches (section Speed Tests and Profiling);
  * ROCm/ATOM PR 1282 ("merge build sparse block into topk"), 128-token
    blocks.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Independent random streams (second element of the rng seed list).
STREAM_LEN = 1
STREAM_VAL = 2
STREAM_SNAP = 3
STREAM_PT = 4
STREAM_Q = 5
STREAM_W = 6
STREAM_KEY = 7
STREAM_PAGE = 8
STREAM_MQ = 9
STREAM_MW = 10

E4M3_MAX = 448.0
# Values written into every cache slot and score cell that no row may read:
# key byte 0x7E is +448, the largest finite e4m3 value, and a large scale makes
# any such token score far above every real token.
SENTINEL_KEY_BYTE = 0x7E
SENTINEL_KEY_SCALE = 1.0e3
SENTINEL_SCORE = np.float32(np.inf)
# bf16 index cache: unused slots hold this key (2^23 in every dimension), far
# above any real key, so reading one would show up in the scores
SENTINEL_KEY_BF16 = 0x4B00

_POOL_THREADS = 8


def rng(seed: int, stream: int, row: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(row)])


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 values drawn from float32 ones by keeping the upper 16 bits (a
    bf16 value is the upper half of a float32 bit pattern)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """Cast float32 values to OCP e4m3fn bytes with torch (clamped to +-448)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp_(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _snap(v: np.ndarray, frac: float, g: np.random.Generator) -> None:
    """Snap a Bernoulli(frac) subset of v to the 1/16 grid (round half to even)."""
    if frac <= 0.0:
        return
    m = g.random(v.shape[0]) < frac
    v[m] = np.round(v[m] * np.float32(16.0)) / np.float32(16.0)


# --------------------------------------------------------------------------
# Top-k over a given fp32 score buffer (decode layout and packed extend layout)
# --------------------------------------------------------------------------


@dataclass
class RowsCase:
    """fp32 score rows plus the addressing of the top-k-with-transform op."""

    name: str
    scores: np.ndarray  # float32 [rows, stride]; cells outside windows are +inf
    seq_lens: np.ndarray  # int32 [rows]
    row_starts: Optional[np.ndarray]  # int32 [rows] or None (window starts at 0)
    row_to_batch: Optional[np.ndarray]  # int32 [rows] or None (page row = row)
    page_table: np.ndarray  # int32 [pt_rows, pt_width]
    page_size: int
    k: int

    @property
    def rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def stride(self) -> int:
        return int(self.scores.shape[1])


def window_values(seed: int, row: int, n: int, tie_frac: float) -> np.ndarray:
    """The n fp32 values of row ``row``'s window (its own random streams), so
    any row of a score buffer can be drawn again on its own."""
    v = rng(seed, STREAM_VAL, row).standard_normal(n, dtype=np.float32)
    _snap(v, tie_frac, rng(seed, STREAM_SNAP, row))
    return v


def _fill_row(buf_row: np.ndarray, start: int, n: int, seed: int, row: int, tie_frac: float) -> None:
    buf_row[:] = SENTINEL_SCORE
    buf_row[start:start + n] = window_values(seed, row, n, tie_frac)


def _fill_rows(scores, starts, lens, seed, tie_frac):
    rows = scores.shape[0]

    def work(r):
        _fill_row(scores[r], int(starts[r]), int(lens[r]), seed, r, tie_frac)

    if rows * scores.shape[1] < (1 << 22):
        for r in range(rows):
            work(r)
    else:
        with ThreadPoolExecutor(_POOL_THREADS) as ex:
            list(ex.map(work, range(rows)))


def decode_rows_case(seed: int = 101, rows: int = 8, stride: int = 4096, n_lo: int = 256,
                     n_hi: int = 4096, k: int = 512, tie_frac: float = 0.05,
                     pt_width: int = 65536, name: str = "decode-topk") -> RowsCase:
    """Decode layout: row i owns scores[i, :n_i] and page-table row i.

    Default sizes: 8 rows of a [8, 4096] buffer, n_i uniform on [256, 4096],
    5% of values snapped to the 1/16 grid, k = 512, page_size 1 tables made of
    independent permutations of [0, 65536).
    """
    lens = rng(seed, STREAM_LEN).integers(n_lo, n_hi + 1, size=rows).astype(np.int32)
    scores = np.empty((rows, stride), dtype=np.float32)
    _fill_rows(scores, np.zeros(rows, np.int64), lens, seed, tie_frac)
    pt = np.stack([rng(seed, STREAM_PT, i).permutation(pt_width) for i in range(rows)]).astype(np.int32)
    return RowsCase(name, scores, lens, None, None, pt, 1, k)


def packed_prefill_case(seed: int = 103, prefix0: int = 61808, new_tokens: int = 8192,
                        k: int = 512, tie_frac: float = 0.01,
                        name: str = "packed-prefill-topk") -> RowsCase:
    """Packed extend layout of two requests sharing one fp32 score buffer.

    Request 0 has a prefix of ``prefix0`` cached tokens, request 1 has none;
    each contributes ``new_tokens`` query rows and attention is causal, so row
    r of a request sees prefix + r + 1 keys. The buffer has
    ``prefix0 + new_tokens + 1`` columns (70001 at full size: not a multiple of
    4). The two windows cannot sit end to end in that width, so request 0's
    rows start at column 0 and request 1's rows start at
    ``stride - new_tokens`` (61809 at full size, odd), where its longest window
    ends on the last column. Each request owns one page-table row of width
    ``prefix0 + new_tokens``; the two rows are one permutation of
    [0, 2 * width) so slots never collide across requests.
    """
    stride = prefix0 + new_tokens + 1
    width = prefix0 + new_tokens
    rows = 2 * new_tokens
    r = np.arange(new_tokens, dtype=np.int64)
    lens = np.concatenate([prefix0 + r + 1, r + 1]).astype(np.int32)
    starts = np.concatenate([np.zeros(new_tokens, np.int64),
                             np.full(new_tokens, stride - new_tokens, np.int64)]).astype(np.int32)
    r2b = np.concatenate([np.zeros(new_tokens, np.int32), np.ones(new_tokens, np.int32)])
    scores = np.empty((rows, stride), dtype=np.float32)
    _fill_rows(scores, starts, lens, seed, tie_frac)
    pt = rng(seed, STREAM_PT).permutation(2 * width).astype(np.int32).reshape(2, width)
    return RowsCase(name, scores, lens, starts, r2b, pt, 1, k)


# --------------------------------------------------------------------------
# Indexer inputs: fp8 queries, head weights, paged fp8 index-key cache
# --------------------------------------------------------------------------


@dataclass
class IndexerCase:
    name: str
    q: np.ndarray  # uint8 (e4m3fn bytes) [B, H, D]
    q_scale: np.ndarray  # float32 [B]
    w: np.ndarray  # float32 [B, H]
    kcache: np.ndarray  # uint8 (e4m3fn bytes) [num_slots, D]
    k_scale: np.ndarray  # float32 [num_slots]
    block_table: np.ndarray  # int32 [B, max_pages]; unused entries name the sentinel page
    page_size: int
    seq_lens: np.ndarray  # int32 [B]
    k: int = 2048
    block_size: int = 0  # block-sparse variant: tokens per block
    top_blocks: int = 0  # block-sparse variant: blocks kept per row
    max_seq_len: int = 0  # upper bound on seq_lens the caller promises
    meta: dict = field(default_factory=dict)
    row_to_batch: Optional[np.ndarray] = None  # int32 [B]: block-table row of each query row
    # "fp8": q and kcache hold e4m3fn bytes with fp32 scales. "bf16": q
    # [B, H, D] and kcache [num_slots, D] hold bf16 bit patterns (uint16);
    # q_scale and k_scale are all ones and unused.
    cache_dtype: str = "fp8"

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def dim(self) -> int:
        return int(self.q.shape[2])


def query_row(seed: int, row: int, heads: int, dim: int, bf16: bool, q_stream: int = STREAM_Q,
              w_stream: int = STREAM_W):
    """Query row ``row``: (q [heads, dim] e4m3fn bytes or bf16 patterns, its
    fp32 scale (1 for bf16), head weights [heads] fp32)."""
    qf = rng(seed, q_stream, row).standard_normal((heads, dim), dtype=np.float32) * np.float32(0.5)
    w = rng(seed, w_stream, row).standard_normal(heads, dtype=np.float32) / np.float32(8.0)
    if bf16:
        return _to_bf16_bits(qf), np.float32(1.0), w
    s = np.float32(np.abs(qf).max() / np.float32(E4M3_MAX))
    return _to_e4m3_bytes(qf / s), s, w


def key_rows(seed: int, request: int, n: int, dim: int, bf16: bool):
    """The n index keys of request ``request`` in token order: (keys [n, dim]
    e4m3fn bytes or bf16 patterns, per-token fp32 scales [n] (ones for
    bf16))."""
    kf = rng(seed, STREAM_KEY, request).standard_normal((n, dim), dtype=np.float32)
    if bf16:
        return _to_bf16_bits(kf), np.ones(n, np.float32)
    s = (np.abs(kf).max(axis=1) / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    return _to_e4m3_bytes(kf / s[:, None]), s


def indexer_case(seed: int, batch: int, n_lo: int, n_hi: int, page_size: int, k: int = 2048,
                 heads: int = 64, dim: int = 128, block_size: int = 0, top_blocks: int = 0,
                 fixed_lens: Optional[np.ndarray] = None, name: str = "indexer",
                 cache_dtype: str = "fp8") -> IndexerCase:
    """Paged indexer inputs.

    fp8 (default): q ~ 0.5 N(0,1) per element with one fp32 scale per row
    (max|q| / 448); head weights ~ N(0,1) / 8; keys ~ N(0,1) per element with
    one fp32 scale per token (max|k_t| / 448). bf16: the same q and key draws
    kept as bf16 values (``_to_bf16_bits``), no scales. Every row gets
    ceil(n_b / page_size) pages drawn from one permutation of all pages; one
    extra page filled with sentinels backs every unused block-table entry,
    and unused slots of partly filled pages hold sentinels too.
    """
    assert cache_dtype in ("fp8", "bf16")
    bf16 = cache_dtype == "bf16"
    if fixed_lens is not None:
        lens = np.asarray(fixed_lens, dtype=np.int32)
        assert lens.shape == (batch,)
    else:
        lens = rng(seed, STREAM_LEN).integers(n_lo, n_hi + 1, size=batch).astype(np.int32)
    max_seq_len = int(max(n_hi, int(lens.max()) if batch else 0))
    P = int(page_size)
    npages = [(int(n) + P - 1) // P for n in lens]
    total_pages = int(sum(npages))
    perm = rng(seed, STREAM_PAGE).permutation(total_pages).astype(np.int64)
    sentinel_page = total_pages
    num_slots = (total_pages + 1) * P
    max_pages = max(1, (max_seq_len + P - 1) // P)

    q = np.empty((batch, heads, dim), np.uint16 if bf16 else np.uint8)
    q_scale = np.ones(batch, np.float32)
    w = np.empty((batch, heads), np.float32)
    for b in range(batch):
        q[b], q_scale[b], w[b] = query_row(seed, b, heads, dim, bf16)

    if bf16:
        kcache = np.full((num_slots, dim), SENTINEL_KEY_BF16, np.uint16)
        k_scale = np.ones(num_slots, np.float32)
    else:
        kcache = np.full((num_slots, dim), SENTINEL_KEY_BYTE, np.uint8)
        k_scale = np.full(num_slots, SENTINEL_KEY_SCALE, np.float32)
    bt = np.full((batch, max_pages), sentinel_page, np.int32)
    offs = np.concatenate([[0], np.cumsum(npages)]).astype(np.int64)

    def work(b):
        n = int(lens[b])
        pages = perm[offs[b]:offs[b + 1]]
        bt[b, :pages.shape[0]] = pages.astype(np.int32)
        if n == 0:
            return
        slots = (pages[:, None] * P + np.arange(P, dtype=np.int64)[None, :]).reshape(-1)[:n]
        kb, s = key_rows(seed, b, n, dim, bf16)
        kcache[slots] = kb
        if not bf16:
            k_scale[slots] = s

    if batch * max_seq_len * dim < (1 << 24):
        for b in range(batch):
            work(b)
    else:
        with ThreadPoolExecutor(_POOL_THREADS) as ex:
            list(ex.map(work, range(batch)))

    return IndexerCase(name, q, q_scale, w, kcache, k_scale, bt, P, lens, k=k,
                       block_size=block_size, top_blocks=top_blocks, max_seq_len=max_seq_len,
                       meta={"total_pages": total_pages, "sentinel_page": sentinel_page, "seed": int(seed),
                             "request_lens": lens.copy(), "q_streams": (STREAM_Q, STREAM_W)},
                       cache_dtype=cache_dtype)


def multi_query_case(seed: int, requests: int, next_n: int, n_lo: int, n_hi: int, page_size: int,
                     k: int = 2048, heads: int = 64, dim: int = 128, name: str = "multi-query",
                     fixed_lens: Optional[np.ndarray] = None, cache_dtype: str = "fp8") -> IndexerCase:
    """Multi-token decode rows: each of `requests` requests decodes `next_n`
    query tokens at once. The cache and block table are those of an
    indexer_case with one row per request (context length L_r); query row
    r * next_n + t belongs to request r (row_to_batch), sees the causal
    length L_r - (next_n - 1 - t), and draws its own query and head weights
    from the same distributions as indexer_case."""
    base = indexer_case(seed, batch=requests, n_lo=n_lo, n_hi=n_hi, page_size=page_size, k=k, heads=heads,
                        dim=dim, name=name, fixed_lens=fixed_lens, cache_dtype=cache_dtype)
    bf16 = cache_dtype == "bf16"
    rows = requests * next_n
    q = np.empty((rows, heads, dim), np.uint16 if bf16 else np.uint8)
    q_scale = np.ones(rows, np.float32)
    w = np.empty((rows, heads), np.float32)
    for r in range(rows):
        q[r], q_scale[r], w[r] = query_row(seed, r, heads, dim, bf16, STREAM_MQ, STREAM_MW)
    r2b = np.repeat(np.arange(requests, dtype=np.int32), next_n)
    t = np.tile(np.arange(next_n, dtype=np.int32), requests)
    lens = np.maximum(base.seq_lens[r2b] - (next_n - 1 - t), 0).astype(np.int32)
    return IndexerCase(name, q, q_scale, w, base.kcache, base.k_scale, base.block_table, page_size, lens, k=k,
                       max_seq_len=base.max_seq_len,
                       meta=dict(base.meta, requests=requests, next_n=next_n, q_streams=(STREAM_MQ, STREAM_MW)),
                       row_to_batch=r2b, cache_dtype=cache_dtype)


@dataclass
class RowInputs:
    """One query row of an IndexerCase drawn again on its own: its query, its
    scale and head weights, and the keys of its block-table row's request in
    token order (keys[j] is the key of the row's token j)."""

    q: np.ndarray
    q_scale: np.float32
    w: np.ndarray
    keys: np.ndarray
    k_scale: np.ndarray
    n: int


def row_spec(case: IndexerCase) -> dict:
    """What ``row_inputs`` needs to draw any row of ``case`` again (small)."""
    return {"seed": case.meta["seed"], "heads": case.heads, "dim": case.dim, "bf16": case.cache_dtype == "bf16",
            "q_streams": tuple(case.meta["q_streams"]), "request_lens": np.asarray(case.meta["request_lens"]),
            "row_to_batch": None if case.row_to_batch is None else np.asarray(case.row_to_batch),
            "seq_lens": np.asarray(case.seq_lens)}


def row_inputs(spec: dict, row: int, keys_cache: Optional[dict] = None) -> RowInputs:
    """Row ``row`` of the case ``spec`` describes, from the same draws as the
    whole case (``query_row``, ``key_rows``). ``keys_cache`` (a dict) keeps
    each request's keys for later rows of the same request."""
    request = row if spec["row_to_batch"] is None else int(spec["row_to_batch"][row])
    q, s, w = query_row(spec["seed"], row, spec["heads"], spec["dim"], spec["bf16"], *spec["q_streams"])
    key = (spec["seed"], request, spec["bf16"])
    kv = None if keys_cache is None else keys_cache.get(key)
    if kv is None:
        kv = key_rows(spec["seed"], request, int(spec["request_lens"][request]), spec["dim"], spec["bf16"])
        if keys_cache is not None:
            keys_cache.clear()
            keys_cache[key] = kv
    return RowInputs(q, s, w, kv[0], kv[1], int(spec["seq_lens"][row]))


# --------------------------------------------------------------------------
# The five named workloads (full size) and reduced versions for quick tests
# --------------------------------------------------------------------------

SEEDS = {"c1": 101, "c2": 102, "c3": 103, "c4": 104, "c5": 105, "mtp": 106, "bf16": 107, "bf16l": 108}


def c1_decode_topk() -> RowsCase:
    return decode_rows_case(seed=SEEDS["c1"], name="decode-topk-8x4096-k512")


def c2_fused_decode() -> IndexerCase:
    return indexer_case(SEEDS["c2"], batch=32, n_lo=8192, n_hi=16384, page_size=64, k=2048,
                        name="fused-decode-B32-n8k-16k-k2048")


def c3_packed_prefill() -> RowsCase:
    return packed_prefill_case(seed=SEEDS["c3"], name="packed-prefill-16384x70001-k512")


def c4_block_sparse() -> IndexerCase:
    return indexer_case(SEEDS["c4"], batch=64, n_lo=32768, n_hi=32768, page_size=128,
                        k=0, block_size=128, top_blocks=32,
                        name="block-sparse-B64-n32768-top32x128")


def c5_long_decode() -> IndexerCase:
    return indexer_case(SEEDS["c5"], batch=64, n_lo=131072, n_hi=327680, page_size=64, k=2048,
                        name="long-decode-B64-n128k-320k-k2048")


def mtp_decode() -> IndexerCase:
    """Multi-token decode: 16 requests x 4 query tokens (64 rows sharing 16
    block-table rows), contexts ~ U{16384..65536}, page_size 64, k 2048."""
    return multi_query_case(SEEDS["mtp"], requests=16, next_n=4, n_lo=16384, n_hi=65536, page_size=64, k=2048,
                            name="mtp-decode-16x4-n16k-64k-k2048")


def bf16_decode() -> IndexerCase:
    """Fused decode from a bf16 index cache: the fused-decode geometry (32
    rows, n ~ U{8192..16384}, page 64, k 2048) with bf16 queries and keys."""
    return indexer_case(SEEDS["bf16"], batch=32, n_lo=8192, n_hi=16384, page_size=64, k=2048,
                        name="fused-decode-bf16-B32-n8k-16k-k2048", cache_dtype="bf16")


def bf16_long_decode() -> IndexerCase:
    """The long-decode geometry (64 rows, n ~ U{131072..327680}, page 64, k
    2048) from a bf16 index cache."""
    return indexer_case(SEEDS["bf16l"], batch=64, n_lo=131072, n_hi=327680, page_size=64, k=2048,
                        name="long-decode-bf16-B64-n128k-320k-k2048", cache_dtype="bf16")


def prefill_indexer() -> IndexerCase:
    """Packed prefill from the fp8 cache, in the packed-prefill top-k
    geometry: request 0 has 61808 cached tokens and request 1 none, each
    extends by 8192 tokens (contexts 70000 and 8192), so the 16384 query rows
    see causal lengths 61809..70000 and 1..8192. page_size 64, k = 512."""
    return multi_query_case(SEEDS["c3"], requests=2, next_n=8192, n_lo=0, n_hi=0, page_size=64, k=512,
                            name="prefill-indexer-2x8192-ctx70000-8192-k512",
                            fixed_lens=np.array([70000, 8192], np.int32))


def expected_tokens(case: IndexerCase) -> int:
    return int(np.asarray(case.seq_lens, dtype=np.int64).sum())


def ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


__all__ = [
    "RowsCase", "IndexerCase", "decode_rows_case", "packed_prefill_case", "indexer_case", "multi_query_case",
    "c1_decode_topk", "c2_fused_decode", "c3_packed_prefill", "c4_block_sparse", "c5_long_decode", "mtp_decode",
    "prefill_indexer", "bf16_decode", "bf16_long_decode", "SENTINEL_KEY_BF16",
    "SEEDS", "SENTINEL_KEY_BYTE", "SENTINEL_KEY_SCALE", "rng", "expected_tokens", "ceil_div",
    "window_values", "query_row", "key_rows", "RowInputs", "row_spec", "row_inputs",
]
