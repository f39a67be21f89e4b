"""ctypes binding of libidxtopk (include/idxtopk.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libidxtopk.so. Tensors must live on the current HIP device. The library is
required: if libidxtopk.so has not been built, importing the ops raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidxtopk.so")
# the same library built with device-side checks (idxtopk_check_status)
CHECKED_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidxtopk_checked.so")

IDXTOPK_OK = 0
IDXTOPK_EINVAL = -1
IDXTOPK_EUNSUPPORTED = -2
IDXTOPK_EWORKSPACE = -3
IDXTOPK_ELAUNCH = -4

OP_TOPK_ROWS = 1
OP_SCORE = 2
OP_PAGE_TRANSFORM = 3
OP_SCORE_TOPK_FUSED = 4
OP_BLOCK_TOPK = 5
OP_CACHE_WRITE = 6
OP_BLOCK_TOPK_HEADS = 7
OP_SCORE_TOPK_PREFILL = 8
KEY_F32 = 0
KEY_BF16 = 1
SORTED = 1
NOALLOC_SCRATCH_BYTES = 64 << 20
CHECKS_OFF = 0x80000000

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/idxtopk.h
SIGNATURES = {
    "idx_score_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32,
                             _i32, _vp, _i64, _vp]),
    "topk_rows": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _i32, _vp]),
    "topk_page_transform": (_i32, [_vp, _i32, _i32, _vp, _i64, _i32, _vp, _vp, _vp]),
    "idx_score_topk_fused": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32,
                                    _i32, _i32, _i32, _vp, _vp, _vp, _sz, _i32, _vp]),
    "idx_score_topk_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32,
                                    _i32, _i32, _i32, _vp, _vp, _vp, _sz, _i32, _vp]),
    "idx_score_topk_fused_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32,
                                            _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "block_topk": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                          _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "block_topk_heads": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "idx_cache_write": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "idx_score_bf16": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i64, _vp]),
    "idx_score_topk_fused_bf16": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _vp, _vp, _vp, _sz, _i32, _vp]),
    "block_topk_bf16": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                               _vp, _vp, _vp, _sz, _vp]),
    "idx_cache_write_bf16": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp]),
    "idxtopk_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "idxtopk_status_str": (ctypes.c_char_p, [_i32]),
    "idxtopk_version": (_i32, []),
    "idxtopk_check_status": (ctypes.c_uint32, [_i32]),
}

_lock = threading.Lock()
_LIBS = {}
_active = [LIB_PATH]  # the library the ops call (a test may switch it, see using())


class LibraryMissing(ImportError):
    pass


def load(path: str = None) -> ctypes.CDLL:
    """Load a libidxtopk build (default: the one the ops call, normally
    libidxtopk.so) and declare its C signatures (raises if not built)."""
    path = _active[0] if path is None else path
    with _lock:
        lib = _LIBS.get(path)
        if lib is not None:
            return lib
        if not os.path.exists(path):
            raise LibraryMissing(
                f"{path} is not built; run `python -m sparse_attention_indexer_fp8_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIBS[path] = lib
        return lib


@contextlib.contextmanager
def using(path: str):
    """Make the ops call the library at `path` (e.g. CHECKED_LIB_PATH) inside
    the block."""
    load(path)
    prev = _active[0]
    _active[0] = path
    try:
        yield load(path)
    finally:
        _active[0] = prev


class IdxTopkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().idxtopk_status_str(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != IDXTOPK_OK:
        raise IdxTopkError(fn, status)
