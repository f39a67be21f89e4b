"""Torch-facing wrappers of the libidxtopk C ABI (marshalling only).

Each function checks dtypes, devices and layouts, passes raw device pointers,
sizes and torch's current HIP stream to the library, and returns the output
tensors. None of them computes anything on the host. The meaning of every
argument is documented in include/idxtopk.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_P = ctypes.c_void_p


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _P(t.data_ptr())


def _stream():
    return _P(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_F8 = (torch.uint8, torch.float8_e4m3fn)


def _as_u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def workspace_bytes(op: int, rows: int, k: int, max_seq_len: int) -> int:
    return int(_lib.load().idxtopk_workspace_bytes(op, rows, k, max_seq_len))


class Workspace:
    """A device buffer for the fused and block ops; its contents never matter.

    Calls that share one Workspace must not run concurrently. A call enqueues
    its kernels on torch's current stream; the buffer is recorded on every
    stream it is used on, so the caching allocator never hands its memory to
    another tensor while a kernel on any of those streams may still use it.
    """

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        self.buf: Optional[torch.Tensor] = None
        self._streams = set()

    def get(self, nbytes: int) -> torch.Tensor:
        stream = torch.cuda.current_stream(self.device)
        if self.buf is None or self.buf.numel() < nbytes:
            # the old buffer's memory returns to the pool only after the work
            # queued on every stream it was recorded on
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._streams = {stream.cuda_stream}
        elif stream.cuda_stream not in self._streams:
            self.buf.record_stream(stream)
            self._streams.add(stream.cuda_stream)
        return self.buf


# One default Workspace per (device, stream): calls on one stream run in
# order, so they never use the default buffer concurrently; calls on two
# streams get two buffers.
_default_ws = {}


def _workspace(ws: Optional[Workspace]) -> Workspace:
    if ws is not None:
        return ws
    dev = torch.cuda.current_device()
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    if key not in _default_ws:
        _default_ws[key] = Workspace(torch.device("cuda", dev))
    return _default_ws[key]


def topk_rows(scores: torch.Tensor, seq_lens: torch.Tensor, k: int,
              row_starts: Optional[torch.Tensor] = None, row_to_batch: Optional[torch.Tensor] = None,
              page_table: Optional[torch.Tensor] = None, page_size: int = 1,
              out: Optional[torch.Tensor] = None, sorted: bool = False,
              kv_offset: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k of each row's fp32 window, mapped through the page table.
    sorted: each row in descending score order, equal scores by ascending
    position, -1 padding last (else the order within a row is unspecified).
    kv_offset: int32 per row, the KV position of the window's first column
    when the call sees one chunk of each request's KV (default 0)."""
    _need(scores, "scores", (torch.float32,), 2, contiguous=False)
    if scores.stride(1) != 1:
        raise ValueError("scores rows must be contiguous")
    rows = scores.shape[0]
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    for name, t in (("row_starts", row_starts), ("row_to_batch", row_to_batch), ("kv_offset", kv_offset)):
        if t is not None:
            _need(t, name, (torch.int32,), 1)
    pt_stride = 0
    if page_table is not None:
        _need(page_table, "page_table", (torch.int32,), 2, contiguous=False)
        if page_table.stride(1) != 1:
            raise ValueError("page_table rows must be contiguous")
        pt_stride = page_table.stride(0)
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    _need(out, "out", (torch.int32,), 2)
    st = _lib.load().topk_rows(_ptr(scores), scores.stride(0), rows, _ptr(seq_lens), _ptr(row_starts),
                               _ptr(row_to_batch), _ptr(kv_offset), _ptr(page_table), pt_stride, int(page_size),
                               int(k),
                               _ptr(out), _lib.SORTED if sorted else 0, _stream())
    _lib.check("topk_rows", st)
    return out


def topk_page_transform(idx: torch.Tensor, page_table: torch.Tensor, page_size: int = 1,
                        row_to_batch: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(idx, "idx", (torch.int32,), 2)
    _need(page_table, "page_table", (torch.int32,), 2, contiguous=False)
    if page_table.stride(1) != 1:
        raise ValueError("page_table rows must be contiguous")
    if row_to_batch is not None:
        _need(row_to_batch, "row_to_batch", (torch.int32,), 1)
    if out is None:
        out = torch.empty_like(idx)
    _need(out, "out", (torch.int32,), 2)
    rows, k = idx.shape
    st = _lib.load().topk_page_transform(_ptr(idx), rows, k, _ptr(page_table), page_table.stride(0),
                                         int(page_size), _ptr(row_to_batch), _ptr(out), _stream())
    _lib.check("topk_page_transform", st)
    return out


def _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch=None):
    _need(q, "q", _F8, 3)
    _need(q_scale, "q_scale", (torch.float32,), 1)
    _need(w, "w", (torch.float32,), 2)
    _need(kcache, "kcache", _F8, 2)
    _need(k_scale, "k_scale", (torch.float32,), 1)
    _need(block_table, "block_table", (torch.int32,), 2, contiguous=False)
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    if row_to_batch is not None:
        _need(row_to_batch, "row_to_batch", (torch.int32,), 1)
    B, H, D = q.shape
    return [_ptr(_as_u8(q)), _ptr(q_scale), _ptr(w), _ptr(_as_u8(kcache)), _ptr(k_scale),
            _ptr(block_table), block_table.stride(0)], B, H, D


def idx_score_fp8(q, q_scale, w, kcache, k_scale, block_table, seq_lens, page_size: int,
                  max_seq_len: int, out: Optional[torch.Tensor] = None,
                  row_to_batch: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index scores S[b, j] for j < seq_lens[b] (other cells of `out` untouched).
    row_to_batch: block-table row of each query row (default: row b -> b)."""
    args, B, H, D = _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch)
    if out is None:
        out = torch.full((B, max(1, max_seq_len)), float("nan"), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 2, contiguous=False)
    st = _lib.load().idx_score_fp8(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                   int(max_seq_len),
                                   _ptr(out), out.stride(0), _stream())
    _lib.check("idx_score_fp8", st)
    return out


def idx_score_topk_fused(q, q_scale, w, kcache, k_scale, block_table, seq_lens, page_size: int,
                         max_seq_len: int, k: int, return_scores: bool = False,
                         workspace: Optional[Workspace] = None, out: Optional[torch.Tensor] = None,
                         out_scores: Optional[torch.Tensor] = None, row_to_batch: Optional[torch.Tensor] = None,
                         sorted: bool = False):
    """Fused decode indexer: top-k slots per row (and their scores if asked).
    row_to_batch: block-table row of each query row (default: row b -> b).
    sorted: rows in descending score order, equal scores by ascending
    position, -1 padding last."""
    args, B, H, D = _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if return_scores and out_scores is None:
        out_scores = torch.empty((B, k), dtype=torch.float32, device=q.device)
    nbytes = workspace_bytes(_lib.OP_SCORE_TOPK_FUSED, B, k, max_seq_len)
    ws = _workspace(workspace).get(nbytes)
    st = _lib.load().idx_score_topk_fused(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                          int(max_seq_len), int(k), _ptr(out), _ptr(out_scores),
                                          _ptr(ws), ws.numel(), _lib.SORTED if sorted else 0, _stream())
    _lib.check("idx_score_topk_fused", st)
    return (out, out_scores) if return_scores else out


def idx_score_topk_prefill(q, q_scale, w, kcache, k_scale, block_table, seq_lens, page_size: int,
                           max_seq_len: int, k: int, return_scores: bool = False,
                           workspace: Optional[Workspace] = None, out: Optional[torch.Tensor] = None,
                           out_scores: Optional[torch.Tensor] = None, row_to_batch: Optional[torch.Tensor] = None,
                           sorted: bool = False):
    """Fused prefill indexer: top-k slots of each packed prefill row (and
    their scores if asked), with no score row in device memory. Rows that
    share a block-table row (row_to_batch) are scored two at a time (four in
    calls of few rows) against each key load. sorted: rows in descending score order, equal scores by
    ascending position, -1 padding last."""
    args, B, H, D = _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if return_scores and out_scores is None:
        out_scores = torch.empty((B, k), dtype=torch.float32, device=q.device)
    nbytes = workspace_bytes(_lib.OP_SCORE_TOPK_PREFILL, B, k, max_seq_len)
    ws = _workspace(workspace).get(nbytes)
    st = _lib.load().idx_score_topk_prefill(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                            int(max_seq_len), int(k), _ptr(out), _ptr(out_scores),
                                            _ptr(ws), ws.numel(), _lib.SORTED if sorted else 0, _stream())
    _lib.check("idx_score_topk_prefill", st)
    return (out, out_scores) if return_scores else out


def idx_score_topk_fused_noalloc(q, q_scale, w, kcache, k_scale, block_table, seq_lens, page_size: int,
                                 max_seq_len: int, k: int, out: torch.Tensor, out_scores: Optional[torch.Tensor] = None,
                                 row_to_batch: Optional[torch.Tensor] = None, sorted: bool = False):
    """idx_score_topk_fused with the library's built-in workspace: the caller
    passes the outputs (out [B, k] int32, optional out_scores [B, k] fp32)
    and nothing is allocated. Calls that overlap on one GPU race."""
    args, B, H, D = _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch)
    _need(out, "out", (torch.int32,), 2)
    if out_scores is not None:
        _need(out_scores, "out_scores", (torch.float32,), 2)
    st = _lib.load().idx_score_topk_fused_noalloc(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H,
                                                  D, int(max_seq_len), int(k), _ptr(out), _ptr(out_scores),
                                                  _lib.SORTED if sorted else 0, _stream())
    _lib.check("idx_score_topk_fused_noalloc", st)
    return out


def block_topk(q, q_scale, w, kcache, k_scale, block_table, seq_lens, page_size: int,
               max_seq_len: int, block_size: int, top_blocks: int, return_slots: bool = True,
               workspace: Optional[Workspace] = None, row_to_batch: Optional[torch.Tensor] = None):
    """Top blocks per row as physical block ids (and expanded slot lists).
    row_to_batch: block-table row of each query row (default: row b -> b)."""
    args, B, H, D = _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch)
    out_blocks = torch.empty((B, top_blocks), dtype=torch.int32, device=q.device)
    out_slots = (torch.empty((B, top_blocks * block_size), dtype=torch.int32, device=q.device)
                 if return_slots else None)
    nbytes = workspace_bytes(_lib.OP_BLOCK_TOPK, B, block_size, max_seq_len)
    ws = _workspace(workspace).get(nbytes)
    st = _lib.load().block_topk(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                int(max_seq_len),
                                int(block_size), int(top_blocks), _ptr(out_blocks), _ptr(out_slots),
                                _ptr(ws), ws.numel(), _stream())
    _lib.check("block_topk", st)
    return (out_blocks, out_slots) if return_slots else out_blocks


def block_topk_heads(q, q_scale, w, kcache, k_scale, block_table, seq_lens, page_size: int,
                     max_seq_len: int, block_size: int, top_blocks: int, return_slots: bool = True,
                     workspace: Optional[Workspace] = None, row_to_batch: Optional[torch.Tensor] = None):
    """Per-head block selection: [B, H, top] physical block ids (and
    [B, H, top * block_size] slot lists), each head ranking blocks by its own
    term of the index score."""
    args, B, H, D = _indexer_args(q, q_scale, w, kcache, k_scale, block_table, seq_lens, row_to_batch)
    out_blocks = torch.empty((B, H, top_blocks), dtype=torch.int32, device=q.device)
    out_slots = (torch.empty((B, H, top_blocks * block_size), dtype=torch.int32, device=q.device)
                 if return_slots else None)
    nbytes = workspace_bytes(_lib.OP_BLOCK_TOPK_HEADS, B * H, block_size, max_seq_len)
    ws = _workspace(workspace).get(nbytes)
    st = _lib.load().block_topk_heads(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                      int(max_seq_len), int(block_size), int(top_blocks), _ptr(out_blocks),
                                      _ptr(out_slots), _ptr(ws), ws.numel(), _stream())
    _lib.check("block_topk_heads", st)
    return (out_blocks, out_slots) if return_slots else out_blocks


def idx_cache_write(keys: torch.Tensor, slot_mapping: torch.Tensor, kcache: torch.Tensor,
                    k_scale: torch.Tensor) -> None:
    """Quantize new index keys (fp32 or bf16, [tokens, 128] with contiguous
    rows) into the paged e4m3fn cache: kcache[slot] and k_scale[slot] for
    every token whose slot is non-negative. In place."""
    if keys.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"keys: expected float32 or bfloat16, got {keys.dtype}")
    _need(keys, "keys", (keys.dtype,), 2, contiguous=False)
    if keys.stride(1) != 1:
        raise ValueError("keys rows must be contiguous")
    _need(slot_mapping, "slot_mapping", (torch.int32,), 1)
    _need(kcache, "kcache", _F8, 2)
    _need(k_scale, "k_scale", (torch.float32,), 1)
    T, D = keys.shape
    dt = _lib.KEY_BF16 if keys.dtype == torch.bfloat16 else _lib.KEY_F32
    st = _lib.load().idx_cache_write(_ptr(keys), dt, keys.stride(0), T, D, _ptr(slot_mapping),
                                     _ptr(_as_u8(kcache)), _ptr(k_scale), _stream())
    _lib.check("idx_cache_write", st)


# ---------------------------------------------------------------------------
# bf16 index cache: q [B, H, 128] and kcache [slots, 128] as bf16 (or their
# 16-bit patterns as int16 / uint16), no scales.
# ---------------------------------------------------------------------------

_BF = (torch.bfloat16, torch.int16, torch.uint16)


def _indexer_args_bf16(q, w, kcache, block_table, seq_lens, row_to_batch=None):
    _need(q, "q", _BF, 3)
    _need(w, "w", (torch.float32,), 2)
    _need(kcache, "kcache", _BF, 2)
    _need(block_table, "block_table", (torch.int32,), 2, contiguous=False)
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    if row_to_batch is not None:
        _need(row_to_batch, "row_to_batch", (torch.int32,), 1)
    B, H, D = q.shape
    return [_ptr(q), _ptr(w), _ptr(kcache), _ptr(block_table), block_table.stride(0)], B, H, D


def idx_score_bf16(q, w, kcache, block_table, seq_lens, page_size: int, max_seq_len: int,
                   out: Optional[torch.Tensor] = None, row_to_batch: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index scores from a bf16 index cache (other cells of `out` untouched)."""
    args, B, H, D = _indexer_args_bf16(q, w, kcache, block_table, seq_lens, row_to_batch)
    if out is None:
        out = torch.full((B, max(1, max_seq_len)), float("nan"), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 2, contiguous=False)
    st = _lib.load().idx_score_bf16(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                    int(max_seq_len), _ptr(out), out.stride(0), _stream())
    _lib.check("idx_score_bf16", st)
    return out


def idx_score_topk_fused_bf16(q, w, kcache, block_table, seq_lens, page_size: int, max_seq_len: int, k: int,
                              return_scores: bool = False, workspace: Optional[Workspace] = None,
                              out: Optional[torch.Tensor] = None, out_scores: Optional[torch.Tensor] = None,
                              row_to_batch: Optional[torch.Tensor] = None, sorted: bool = False):
    """Fused decode indexer from a bf16 index cache: top-k slots per row (and
    their scores if asked); `sorted` as in idx_score_topk_fused."""
    args, B, H, D = _indexer_args_bf16(q, w, kcache, block_table, seq_lens, row_to_batch)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if return_scores and out_scores is None:
        out_scores = torch.empty((B, k), dtype=torch.float32, device=q.device)
    nbytes = workspace_bytes(_lib.OP_SCORE_TOPK_FUSED, B, k, max_seq_len)
    ws = _workspace(workspace).get(nbytes)
    st = _lib.load().idx_score_topk_fused_bf16(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                               int(max_seq_len), int(k), _ptr(out), _ptr(out_scores),
                                               _ptr(ws), ws.numel(), _lib.SORTED if sorted else 0, _stream())
    _lib.check("idx_score_topk_fused_bf16", st)
    return (out, out_scores) if return_scores else out


def block_topk_bf16(q, w, kcache, block_table, seq_lens, page_size: int, max_seq_len: int, block_size: int,
                    top_blocks: int, return_slots: bool = True, workspace: Optional[Workspace] = None,
                    row_to_batch: Optional[torch.Tensor] = None):
    """Top blocks per row from a bf16 index cache (and expanded slot lists)."""
    args, B, H, D = _indexer_args_bf16(q, w, kcache, block_table, seq_lens, row_to_batch)
    out_blocks = torch.empty((B, top_blocks), dtype=torch.int32, device=q.device)
    out_slots = (torch.empty((B, top_blocks * block_size), dtype=torch.int32, device=q.device)
                 if return_slots else None)
    nbytes = workspace_bytes(_lib.OP_BLOCK_TOPK, B, block_size, max_seq_len)
    ws = _workspace(workspace).get(nbytes)
    st = _lib.load().block_topk_bf16(*args, int(page_size), _ptr(row_to_batch), _ptr(seq_lens), B, H, D,
                                     int(max_seq_len), int(block_size), int(top_blocks), _ptr(out_blocks),
                                     _ptr(out_slots), _ptr(ws), ws.numel(), _stream())
    _lib.check("block_topk_bf16", st)
    return (out_blocks, out_slots) if return_slots else out_blocks


def idx_cache_write_bf16(keys: torch.Tensor, slot_mapping: torch.Tensor, kcache: torch.Tensor) -> None:
    """Store new index keys (fp32 rounded to nearest even, or bf16 as they
    are; [tokens, 128], rows contiguous and 16-byte aligned) into the bf16
    cache at kcache[slot] for every non-negative slot. In place."""
    if keys.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"keys: expected float32 or bfloat16, got {keys.dtype}")
    _need(keys, "keys", (keys.dtype,), 2, contiguous=False)
    if keys.stride(1) != 1:
        raise ValueError("keys rows must be contiguous")
    _need(slot_mapping, "slot_mapping", (torch.int32,), 1)
    _need(kcache, "kcache", _BF, 2)
    T, D = keys.shape
    dt = _lib.KEY_BF16 if keys.dtype == torch.bfloat16 else _lib.KEY_F32
    st = _lib.load().idx_cache_write_bf16(_ptr(keys), dt, keys.stride(0), T, D, _ptr(slot_mapping), _ptr(kcache),
                                          _stream())
    _lib.check("idx_cache_write_bf16", st)
