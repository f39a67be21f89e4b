#!/usr/bin/env python3
"""Benchmark of the sparse-attention indexer top-k path on one MI355X.

Headline step: one topk_rows call over the packed-prefill batch, 16384 score
rows of a [16384, 70001] fp32 buffer from two requests (prefix 61808 and 0,
8192 new tokens each), k = 512, page_size 1 transform through row_to_batch.
That is the workload of the pages' kernel-level measurement: grid 16384, ISL
70000 ("[AMD] Enable GLM DSA prefill top-k to the v2 kernel", section Speed
Tests and Profiling).

The same JSON line also carries the other workloads, each with its own HBM
roofline figure:
  * decode top-k:    8 rows of [8, 4096], k 512;
  * fused decode:    B 32, n ~ U[8192, 16384], k 2048;
  * block-sparse:    B 64, n 32768, top 32 blocks of 128;
  * long decode:     B 64, n ~ U[131072, 327680], k 2048;
  * multi-token decode: 16 requests x 4 query rows, n ~ U[16384, 65536], k 2048;
  * index-key cache write: 16384 bf16 keys into a 1M-slot cache;
  * prefill indexer from the fp8 cache: the packed-prefill geometry (16384
    rows, causal lengths 61809..70000 and 1..8192), scores then top-512.
It also carries the CPU oracle's throughput on a bounded sample of the
headline workload, run on the host's cores.

Timing, per workload: SETTLE_SECONDS of untimed back-to-back launches (the
chip's clocks rise only under sustained load), W untimed warmup steps, then
exactly K timed steps between HIP events on the launch stream.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only c3|all|...] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "top-k rows/s + µs/launch and achieved HBM GB/s (% roofline), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
FLUSH_BYTES = 1 << 30
COPY_CALIBRATION_BYTES = 1 << 30
# Untimed back-to-back launches of each workload before its warmup steps. The
# chip raises its clocks only after some tens of milliseconds of sustained
# load (after an idle gap the first ~40 ms of launches run up to 1.3x slower),
# and a serving loop runs in that steady state.
SETTLE_SECONDS = 0.25
COUNTERS_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "topk_rows": ["topk_rows.hip", "select.hpp", "sort.hpp", "common.hpp"],
    "fused": ["indexer.hip", "indexer_shared.hpp", "score_mfma.hpp", "select.hpp", "common.hpp"],
    "prefill": ["prefill.hip", "indexer_shared.hpp", "score_mfma.hpp", "select.hpp", "common.hpp"],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that a changed
    comment does not mark the measured counters stale (string literals in
    these kernels hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kind: str) -> str:
    """Hash of the code (comments and spacing ignored) of the sources a
    kernel kind is built from; counters taken on other code read as stale."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "sparse_attention_indexer_fp8_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


PMC_KERNELS = {
    # counters file name -> (source kind, kernel name prefix, grid size (threads) of the workload's launch,
    # the benchmark entry it belongs to)
    "topk_rows_packed_prefill_16384x70001": ("topk_rows", "void idxtopk::topk_rows_kernel<false>", 16384 * 256,
                                             None),
    "fused_long_decode_B64_k2048": ("fused", "void idxtopk::fused_chunk_kernel<4, false>", 1310720,
                                    "long_decode_B64_k2048"),
    "fused_decode_B32_chunk": ("fused", "void idxtopk::fused_chunk_kernel<4, false>", 196608,
                               "fused_decode_B32_k2048"),
    "fused_decode_B32_merge": ("fused", "void idxtopk::fused_merge_kernel<4, false>", 32768,
                               "fused_decode_B32_k2048"),
    "mtp_decode_16x4_chunk": ("fused", "void idxtopk::fused_pair_chunk_kernel<4>", 262144,
                              "mtp_decode_16x4_k2048"),
    "mtp_decode_16x4_rowgroup_chunk": ("prefill", "void idxtopk::prefill_chunk_kernel<4, true, 4>", 65536,
                                       "mtp_decode_16x4_k2048"),
    "block_sparse_B64_chunk": ("fused", "void idxtopk::block_chunk_kernel<4, false>", 196608,
                               "block_sparse_B64_n32768_top32"),
    "block_sparse_B64_merge": ("fused", "idxtopk::block_merge_kernel", 32768, "block_sparse_B64_n32768_top32"),
    "block_heads_B64_chunk": ("fused", "void idxtopk::block_heads_chunk_kernel<4>", 524288,
                              "block_sparse_per_head_B64_H64_top32"),
    "block_heads_B64_merge": ("fused", "idxtopk::block_heads_merge_kernel", 262144,
                              "block_sparse_per_head_B64_H64_top32"),
    "prefill_scores_16384": ("fused", "void idxtopk::pair_score_kernel<4>", 4718592, "prefill_indexer_16384_k512"),
    "prefill_fused_chunk_16384": ("prefill", "void idxtopk::prefill_chunk_kernel<4, false, 2>", 4718592,
                                  "prefill_indexer_16384_k512"),
    "prefill_fused_merge_16384": ("prefill", "void idxtopk::prefill_merge_kernel", 8388608,
                                  "prefill_indexer_16384_k512"),
}


def _pmc_rows(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def write_counters_from_pmc(fetch_csv: str, write_csv: str, command: str) -> None:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) into profiles/<name>.counters.json. Each counter is scaled by
    what it reads for the 1 GiB device copy of --copy-calibration (a plain
    copy kernel that reads and writes exactly 1 GiB)."""
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _pmc_rows(path) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
        if not copies:
            raise SystemExit(f"{path}: no 1 GiB copy dispatch to calibrate {counter}")
        factor = (COPY_CALIBRATION_BYTES / 1024) / (sum(copies) / len(copies))
        for name, (kind, prefix, grid, _) in PMC_KERNELS.items():
            vals = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith(prefix)
                    and (grid is None or int(r["Grid_Size"]) == grid)]
            if vals:
                e = out.setdefault(name, {"kind": kind, "kernel": prefix})
                e[counter] = {"kib_per_dispatch": sum(vals) / len(vals), "dispatches": len(vals),
                              "copy_calibration_factor": factor,
                              "bytes_per_dispatch": sum(vals) / len(vals) * 1024 * factor}
    for name, e in out.items():
        if "FETCH_SIZE" not in e or "WRITE_SIZE" not in e:
            continue
        e["bytes_per_launch"] = round(e["FETCH_SIZE"]["bytes_per_dispatch"] + e["WRITE_SIZE"]["bytes_per_dispatch"])
        e["source_hash"] = source_hash(e["kind"])
        e["command"] = command
        with open(os.path.join(COUNTERS_DIR, f"{name}.counters.json"), "w") as f:
            json.dump(e, f, indent=1)
        log(f"wrote {name}: {e['bytes_per_launch']} bytes per launch")


def counter_traffic(name: str, kind: str):
    """HBM bytes per launch from committed rocprofv3 PMC runs, if the kernel is unchanged."""
    path = os.path.join(COUNTERS_DIR, f"{name}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(kind):
        return None
    return d.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move; see the design notes)
# ---------------------------------------------------------------------------


def rows_algorithmic_bytes(case) -> int:
    n = case.seq_lens.astype(np.int64)
    k = case.k
    read = int((4 * n[n > k]).sum())
    sel = np.minimum(n, k)
    out = case.rows * k * 4
    gathers = int((4 * sel).sum()) if case.page_table is not None else 0
    meta = 4 * case.rows * (1 + (case.row_starts is not None) + (case.row_to_batch is not None))
    return read + out + gathers + meta


def indexer_algorithmic_bytes(case, out_entries: int) -> int:
    """Keys (128 B + 4 B scale per token from an fp8 cache, 256 B from a bf16
    one), block-table entries, queries, head weights and scales, outputs.
    Query rows that share a block-table row (row_to_batch) read nested
    windows of the same keys: those count once per block-table row, at the
    longest window."""
    n = case.seq_lens.astype(np.int64)
    r2b = getattr(case, "row_to_batch", None)
    if r2b is not None:
        longest = np.zeros(case.block_table.shape[0], np.int64)
        np.maximum.at(longest, np.asarray(r2b, np.int64), n)
        n = longest
    P = case.page_size
    bf16 = getattr(case, "cache_dtype", "fp8") == "bf16"
    per_token = 2 * case.dim if bf16 else case.dim + 4
    keys = int((n * per_token).sum())
    table = int((4 * ((n + P - 1) // P)).sum())
    query = (case.batch * case.heads * (2 * case.dim + 4) + 4 * case.batch if bf16
             else case.batch * case.heads * (case.dim + 4) + 8 * case.batch)
    return keys + table + query + 4 * out_entries


# ---------------------------------------------------------------------------
# CPU oracle baseline (runs before the GPU is touched; forked workers)
# ---------------------------------------------------------------------------

_CPU_CASE = None


def _oracle_rows(rows):
    import oracle

    c = _CPU_CASE
    return oracle.topk_rows(c.scores, c.seq_lens, c.k, c.row_starts, c.row_to_batch, c.page_table,
                            c.page_size, rows=rows).shape[0]


def cpu_baseline(case, every: int = 2):
    import multiprocessing as mp

    global _CPU_CASE
    _CPU_CASE = case
    cores = min(len(os.sched_getaffinity(0)), 16)
    rows = list(range(0, case.rows, every))
    chunks = [rows[i::cores * 4] for i in range(cores * 4)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        done = sum(pool.map(_oracle_rows, chunks))
    wall = time.perf_counter() - t0
    assert done == len(rows)
    return {"value": round(len(rows) / wall, 1), "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} of {case.rows} rows (one row in {every}) of the packed-prefill buffer, "
                      f"oracle.topk_rows (float64 full stable sort per row + page transform), "
                      f"{cores} forked worker processes, wall {wall:.2f} s (~{wall * cores:.0f} core-seconds)"}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------


class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.flush_buf = None

    def flush(self):
        if self.flush_buf is None:
            self.flush_buf = self.torch.empty(FLUSH_BYTES // 4, dtype=self.torch.float32, device="cuda")
        self.flush_buf.fill_(1.0)

    def settle(self, fn, flush):
        """Launch fn back to back (with the flush, if any) for SETTLE_SECONDS
        of wall time; returns the number of launches."""
        torch = self.torch
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < SETTLE_SECONDS:
            for _ in range(8):
                if flush:
                    self.flush()
                fn()
            n += 8
            torch.cuda.synchronize()
        return n

    def run(self, fn, warmup, steps, flush=False):
        """Per-launch HIP event pairs on the current stream, plus, without a
        flush, one pair around the whole timed region: launches then run
        back to back, and the region mean (total / steps) is the average launch
        duration. Returns the wall time, the per-launch durations (µs) and the
        region mean (µs, or None with a flush between launches)."""
        torch = self.torch
        self.settled = self.settle(fn, flush)
        for _ in range(warmup):
            if flush:
                self.flush()
            fn()
        torch.cuda.synchronize()
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r0.record()
        for i in range(steps):
            if flush:
                self.flush()
            ev0[i].record()
            fn()
            ev1[i].record()
        r1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in zip(ev0, ev1)])
        region = None if flush else r0.elapsed_time(r1) * 1e3 / steps
        return wall, us, region


def summary(us, nbytes, rows, region=None, settled=None):
    med = float(np.median(us))
    mean = float(np.mean(us)) if region is None else float(region)
    gbps = nbytes / (mean * 1e-6) / 1e9
    return {"us_per_launch_mean": round(mean, 2), "us_per_launch_median": round(med, 2),
            "us_p10": round(float(np.percentile(us, 10)), 2), "us_p90": round(float(np.percentile(us, 90)), 2),
            "rows_per_s": round(rows / (mean * 1e-6), 1), "algorithmic_bytes": int(nbytes),
            "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "settle_launches": settled}


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bench_rows(torch, ops, timer, case, warmup, steps, flush, sorted=False):
    sc = dev(torch, case.scores)
    sl = dev(torch, case.seq_lens)
    rs = None if case.row_starts is None else dev(torch, case.row_starts)
    rb = None if case.row_to_batch is None else dev(torch, case.row_to_batch)
    pt = dev(torch, case.page_table)
    out = torch.empty((case.rows, case.k), dtype=torch.int32, device="cuda")

    def step():
        ops.topk_rows(sc, sl, case.k, rs, rb, pt, case.page_size, out=out, sorted=sorted)

    wall, us, region = timer.run(step, warmup, steps, flush)
    res = summary(us, rows_algorithmic_bytes(case), case.rows, region, timer.settled)
    del sc
    torch.cuda.empty_cache()
    return wall, us, res


def bench_fused(torch, ops, timer, case, warmup, steps, flush, sorted=False):
    bf16 = getattr(case, "cache_dtype", "fp8") == "bf16"
    fields = ((case.q, case.w, case.kcache, case.block_table, case.seq_lens) if bf16 else
              (case.q, case.q_scale, case.w, case.kcache, case.k_scale, case.block_table, case.seq_lens))
    args = [dev(torch, x) for x in fields]
    out = torch.empty((case.batch, case.k), dtype=torch.int32, device="cuda")
    ws = ops.Workspace()
    fused = ops.idx_score_topk_fused_bf16 if bf16 else ops.idx_score_topk_fused

    def step():
        fused(*args, case.page_size, case.max_seq_len, case.k, workspace=ws, out=out, sorted=sorted)

    wall, us, region = timer.run(step, warmup, steps, flush)
    res = summary(us, indexer_algorithmic_bytes(case, case.batch * case.k), case.batch, region, timer.settled)
    res["tokens"] = int(case.seq_lens.astype(np.int64).sum())
    del args
    torch.cuda.empty_cache()
    return res


def bench_fused_mq(torch, ops, timer, case, warmup, steps, flush):
    """Fused path on multi-token decode rows (row_to_batch shares block-table
    rows between a request's query tokens)."""
    args = [dev(torch, x) for x in (case.q, case.q_scale, case.w, case.kcache, case.k_scale,
                                    case.block_table, case.seq_lens)]
    r2b = dev(torch, case.row_to_batch)
    out = torch.empty((case.batch, case.k), dtype=torch.int32, device="cuda")
    ws = ops.Workspace()

    def step():
        ops.idx_score_topk_fused(*args, case.page_size, case.max_seq_len, case.k, workspace=ws, out=out,
                                 row_to_batch=r2b)

    def step_rows():
        ops.idx_score_topk_prefill(*args, case.page_size, case.max_seq_len, case.k, workspace=ws, out=out,
                                   row_to_batch=r2b)

    nbytes = indexer_algorithmic_bytes(case, case.batch * case.k)
    wall, us, region = timer.run(step, warmup, steps, flush)
    res = summary(us, nbytes, case.batch, region, timer.settled)
    res["call"] = ("idx_score_topk_fused (two rows of a request per chunk workgroup against one key load; "
                   "a request's rows on one XCD, keys shared through its L2)")
    res["rows"] = case.batch
    res["row_tokens"] = int(case.seq_lens.astype(np.int64).sum())
    # the row-group call on the same rows (each key group loaded once for a
    # request's four rows), for comparison
    wall, us, region = timer.run(step_rows, warmup, steps, flush)
    res["row_group_call"] = summary(us, nbytes, case.batch, region, timer.settled)
    del args
    torch.cuda.empty_cache()
    return res


def bench_cache_write(torch, ops, timer, warmup, steps, flush, tokens=16384, num_slots=1 << 20):
    """Index-key cache writer: `tokens` new bf16 keys (one prefill chunk)
    quantized into a cache of num_slots slots at distinct random slots.
    Algorithmic bytes: keys read (2 B x 128) + slot ids read (4 B) + codes
    (128 B) and scales (4 B) written, per token."""
    g = np.random.default_rng(workloads.SEEDS["c3"])
    keys = torch.from_numpy(g.standard_normal((tokens, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    slots = torch.from_numpy(g.permutation(num_slots)[:tokens].astype(np.int32)).cuda()
    kc = torch.zeros((num_slots, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((num_slots,), dtype=torch.float32, device="cuda")

    def step():
        ops.idx_cache_write(keys, slots, kc, ks)

    wall, us, region = timer.run(step, warmup, steps, flush)
    res = summary(us, tokens * (2 * 128 + 4 + 128 + 4), tokens, region, timer.settled)
    res["tokens"] = tokens
    del keys, slots, kc, ks
    torch.cuda.empty_cache()
    return res


FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak


def bench_prefill(torch, ops, timer, case, warmup, steps):
    """Prefill indexer from the fp8 cache: idx_score_fp8 with row_to_batch
    (two rows per wave against one key load) writes the score rows, then
    topk_rows selects k per row and maps through the block table. The score
    step is a dense contraction, measured against the fp8 matrix peak
    (2 * heads * 128 flops per (row, key)); the top-k step against HBM."""
    args = [dev(torch, x) for x in (case.q, case.q_scale, case.w, case.kcache, case.k_scale,
                                    case.block_table, case.seq_lens)]
    r2b = dev(torch, case.row_to_batch)
    bt, sl = args[5], args[6]
    scores = torch.empty((case.batch, case.max_seq_len), dtype=torch.float32, device="cuda")
    out = torch.empty((case.batch, case.k), dtype=torch.int32, device="cuda")

    def score():
        ops.idx_score_fp8(*args, case.page_size, case.max_seq_len, out=scores, row_to_batch=r2b)

    def topk():
        ops.topk_rows(scores, sl, case.k, row_to_batch=r2b, page_table=bt, page_size=case.page_size, out=out)

    n = case.seq_lens.astype(np.int64)
    flops = 2 * case.heads * case.dim * int(n.sum())
    _, us_s, reg_s = timer.run(score, warmup, steps, False)
    settled_s = timer.settled
    _, us_t, reg_t = timer.run(topk, warmup, steps, False)
    s_us = float(reg_s)
    tflops = flops / (s_us * 1e-6) / 1e12
    topk_bytes = int((4 * n[n > case.k]).sum()) + case.batch * case.k * 4 + int((4 * np.minimum(n, case.k)).sum()) \
        + 8 * case.batch
    res_t = summary(us_t, topk_bytes, case.batch, reg_t, timer.settled)
    res = {"rows": case.batch, "row_tokens": int(n.sum()), "k": case.k,
           "score": {"us_per_launch_mean": round(s_us, 2), "us_per_launch_median": round(float(np.median(us_s)), 2),
                     "flops": flops, "achieved_TFLOPs": round(tflops, 1),
                     "mfma_frac": round(tflops / FP8_PEAK_TFLOPS, 4), "bound": "mfma (fp8)",
                     "settle_launches": settled_s},
           "topk": res_t,
           "us_per_call_total": round(s_us + res_t["us_per_launch_mean"], 2),
           "score_buffer_bytes": int(scores.numel() * 4)}
    del scores
    torch.cuda.empty_cache()

    # The fused call: no score buffer (its workspace holds candidate lists).
    ws = ops.Workspace()
    ws_bytes = ops.workspace_bytes(ops._lib.OP_SCORE_TOPK_PREFILL, case.batch, case.k, case.max_seq_len)
    ws.get(ws_bytes)

    def fused():
        ops.idx_score_topk_prefill(*args, case.page_size, case.max_seq_len, case.k, workspace=ws, out=out,
                                   row_to_batch=r2b)

    _, us_f, reg_f = timer.run(fused, warmup, steps, False)
    f_us = float(reg_f)
    res["fused"] = {"us_per_call_mean": round(f_us, 2), "us_per_call_median": round(float(np.median(us_f)), 2),
                    "row_tokens_per_s": round(float(n.sum()) / (f_us * 1e-6), 1),
                    "score_flops_TFLOPs": round(flops / (f_us * 1e-6) / 1e12, 1),
                    "workspace_bytes": int(ws_bytes), "score_buffer_bytes": 0,
                    "settle_launches": timer.settled}
    del args, ws
    torch.cuda.empty_cache()
    return res


def bench_unfused(torch, ops, timer, case, warmup, steps, flush):
    """The unfused path on the same inputs: idx_score_fp8 writes the score
    rows, then topk_rows selects and maps through the block table (the pages'
    "before" of the fusion). Same algorithmic bytes as the fused call, so the
    two figures compare directly."""
    args = [dev(torch, x) for x in (case.q, case.q_scale, case.w, case.kcache, case.k_scale,
                                    case.block_table, case.seq_lens)]
    scores = torch.empty((case.batch, max(1, case.max_seq_len)), dtype=torch.float32, device="cuda")
    out = torch.empty((case.batch, case.k), dtype=torch.int32, device="cuda")
    bt, sl = args[5], args[6]

    def step():
        ops.idx_score_fp8(*args, case.page_size, case.max_seq_len, out=scores)
        ops.topk_rows(scores, sl, case.k, page_table=bt, page_size=case.page_size, out=out)

    wall, us, region = timer.run(step, warmup, steps, flush)
    res = summary(us, indexer_algorithmic_bytes(case, case.batch * case.k), case.batch, region, timer.settled)
    res["score_buffer_bytes"] = int(scores.numel() * 4)
    del args, scores
    torch.cuda.empty_cache()
    return res


def bench_block(torch, ops, timer, case, warmup, steps, flush, per_head=False):
    """Block selection (per_head: one selection per (row, head), outputs
    H times larger)."""
    args = [dev(torch, x) for x in (case.q, case.q_scale, case.w, case.kcache, case.k_scale,
                                    case.block_table, case.seq_lens)]
    ws = ops.Workspace()
    op = ops.block_topk_heads if per_head else ops.block_topk

    def step():
        op(*args, case.page_size, case.max_seq_len, case.block_size, case.top_blocks, workspace=ws)

    wall, us, region = timer.run(step, warmup, steps, flush)
    out_entries = case.batch * (case.heads if per_head else 1) * case.top_blocks * (1 + case.block_size)
    res = summary(us, indexer_algorithmic_bytes(case, out_entries), case.batch, region, timer.settled)
    res["tokens"] = int(case.seq_lens.astype(np.int64).sum())
    del args
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all", help="comma list of c1..c5, mtp, cw, pf, bf16, bf16l, or all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for PMC byte-counter calibration)")
    ap.add_argument("--from-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/*.counters.json from two rocprofv3 --pmc counter_collection.csv "
                         "files (FETCH_SIZE run, WRITE_SIZE run) and exit")
    ap.add_argument("--pmc-command", default="", help="the command the --pmc runs used (recorded)")
    a = ap.parse_args(argv)
    if a.from_pmc:
        write_counters_from_pmc(a.from_pmc[0], a.from_pmc[1], a.pmc_command)
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the indexer top-k path here runs on a single MI355X "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        return 2
    only = ({"c1", "c2", "c3", "c4", "c5", "mtp", "cw", "pf", "bf16", "bf16l"} if a.only == "all"
            else set(a.only.split(",")))

    case3 = None
    cpu = None
    if "c3" in only:
        log("generating packed-prefill 16384x70001 ...")
        case3 = workloads.c3_packed_prefill()
        if not a.no_cpu:
            log("cpu oracle baseline ...")
            cpu = cpu_baseline(case3)
            log(f"cpu baseline {cpu['value']} rows/s on {cpu['cores']} cores")

    import torch
    from sparse_attention_indexer_fp8_amd import ops

    torch.cuda.set_device(0)
    timer = Timer(torch)
    also = {}
    line = None

    if a.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1 GiB")
        del src, dst

    if case3 is not None:
        log("timing packed-prefill top-k ...")
        wall, us, res = bench_rows(torch, ops, timer, case3, a.warmup, a.steps, flush=False)
        traffic = counter_traffic("topk_rows_packed_prefill_16384x70001", "topk_rows")
        roof = {"bound": "hbm", "achieved": res["achieved_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(res["achieved_GBps"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "topk_rows_kernel",
                "per_launch": {"algorithmic_bytes": res["algorithmic_bytes"],
                               "avg_kernel_us": res["us_per_launch_mean"],
                               "timing": "HIP events around the timed region of back-to-back launches, / steps"}}
        line = {
            "metric": METRIC,
            "value": round(case3.rows * a.steps / wall, 1),
            "unit": "rows/s",
            "n_gpus": 1,
            "steps": a.steps,
            "warmup": a.warmup,
            "ms_per_step": round(wall / a.steps * 1e3, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "packed-prefill-topk: 16384 rows x 70001 fp32 (2 requests, prefix 61808/0, "
                                   "8192 new tokens each), k=512, page_size 1, row_starts/row_to_batch",
                       "rows": case3.rows, "stride": case3.stride, "k": case3.k,
                       "sum_seq_len": int(case3.seq_lens.astype(np.int64).sum())},
            "roofline": roof,
            "cpu_baseline": cpu,
            "us_per_launch": res["us_per_launch_mean"],
            "us_per_launch_median": res["us_per_launch_median"],
            "achieved_GBps": res["achieved_GBps"],
        }
        log("timing packed-prefill top-k, sorted output ...")
        _, _, also["packed_prefill_topk_sorted"] = bench_rows(torch, ops, timer, case3, a.warmup, a.steps,
                                                              flush=False, sorted=True)
        del case3
    if "c1" in only:
        log("timing decode top-k ...")
        c1 = workloads.c1_decode_topk()
        _, _, also["decode_topk_8x4096_k512"] = bench_rows(torch, ops, timer, c1, a.warmup, max(a.steps, 50),
                                                           flush=True)
    if "c2" in only:
        log("timing fused decode B32 ...")
        c2 = workloads.c2_fused_decode()
        also["fused_decode_B32_k2048"] = bench_fused(torch, ops, timer, c2, a.warmup, max(a.steps, 50), True)
        log("timing fused decode B32, sorted output ...")
        also["fused_decode_B32_k2048_sorted"] = bench_fused(torch, ops, timer, c2, a.warmup, max(a.steps, 50), True,
                                                            sorted=True)
        log("timing fused decode B32, unfused path ...")
        also["fused_decode_B32_k2048_unfused"] = bench_unfused(torch, ops, timer, c2, a.warmup, max(a.steps, 50),
                                                               True)
        del c2
    if "pf" in only:
        log("generating prefill indexer inputs ...")
        pf = workloads.prefill_indexer()
        log("timing prefill indexer (row-pair scores + top-k) ...")
        also["prefill_indexer_16384_k512"] = bench_prefill(torch, ops, timer, pf, a.warmup, a.steps)
        del pf
    if "cw" in only:
        log("timing index-key cache write ...")
        also["cache_write_16384_bf16"] = bench_cache_write(torch, ops, timer, a.warmup, max(a.steps, 50), True)
    if "mtp" in only:
        log("timing multi-token decode 16x4 ...")
        mq = workloads.mtp_decode()
        also["mtp_decode_16x4_k2048"] = bench_fused_mq(torch, ops, timer, mq, a.warmup, max(a.steps, 50), True)
        del mq
    if "c4" in only:
        log("timing block-sparse B64 ...")
        c4 = workloads.c4_block_sparse()
        also["block_sparse_B64_n32768_top32"] = bench_block(torch, ops, timer, c4, a.warmup, max(a.steps, 50),
                                                            True)
        log("timing block-sparse B64, per-head selection ...")
        also["block_sparse_per_head_B64_H64_top32"] = bench_block(torch, ops, timer, c4, a.warmup,
                                                                  max(a.steps, 50), True, per_head=True)
        del c4
    if "bf16" in only:
        log("timing fused decode B32 from a bf16 cache ...")
        bc = workloads.bf16_decode()
        also["fused_decode_bf16_B32_k2048"] = bench_fused(torch, ops, timer, bc, a.warmup, max(a.steps, 50), True)
        del bc
    if "bf16l" in only:
        log("generating long decode B64 from a bf16 cache ...")
        bl = workloads.bf16_long_decode()
        log("timing long decode B64 from a bf16 cache ...")
        also["long_decode_bf16_B64_k2048"] = bench_fused(torch, ops, timer, bl, a.warmup, a.steps, False)
        del bl
    if "c5" in only:
        log("generating long decode B64 ...")
        c5 = workloads.c5_long_decode()
        log("timing long decode B64 ...")
        also["long_decode_B64_k2048"] = bench_fused(torch, ops, timer, c5, a.warmup, a.steps, False)
        log("timing long decode B64, unfused path ...")
        also["long_decode_B64_k2048_unfused"] = bench_unfused(torch, ops, timer, c5, a.warmup, a.steps, False)
        del c5
    # HBM bytes per launch of each kernel with committed counters (null when
    # the kernel's code changed since they were taken)
    for name, (kind, _, _, key) in PMC_KERNELS.items():
        if key in also:
            also[key].setdefault("counter_traffic_bytes", {})[name] = counter_traffic(name, kind)
    if line is None:
        line = {"metric": METRIC, "value": None, "unit": "rows/s", "n_gpus": 1, "steps": a.steps,
                "warmup": a.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "f32", "data": "synthetic", "config": {"workload": "partial run: " + a.only}}
    line["also"] = also
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
