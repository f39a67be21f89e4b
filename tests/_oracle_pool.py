"""Process pool that runs the oracle side of the full-size parity checks.

conftest starts it at session start, before any test touches the GPU, so its
workers are forked from a process that has not initialised the device: plain
CPU processes that never use it. Each worker draws the rows it checks again
from the seeds (``workloads.window_values`` / ``workloads.row_inputs``), so
no multi-gigabyte input is copied to it; only the GPU outputs of its rows
travel. BLAS runs one thread per worker.
"""
from __future__ import annotations

import multiprocessing as mp
import os

_POOL = None
MAX_WORKERS = 16


def workers() -> int:
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:
        pass


def start() -> None:
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("fork").Pool(workers(), initializer=_init_worker)


def get():
    if _POOL is None:
        raise RuntimeError("the oracle pool is started at session start, before the GPU is initialised")
    return _POOL


def stop() -> None:
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None
