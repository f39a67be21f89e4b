"""Build libidxtopk.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m sparse_attention_indexer_fp8_amd.build [--debug] [--checked] [-j N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["api.hip", "topk_rows.hip", "page_transform.hip", "indexer.hip", "cache_write.hip", "sort_rows.hip", "prefill.hip"]
LIB_NAME = "libidxtopk.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the same library with device-side checks (IDXTOPK_CHECKS=1)
CHECKED_LIB_PATH = os.path.join(PKG, "libidxtopk_checked.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# Packed fp32 instructions stay off: hipcc would otherwise form them from
# plain float code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results go straight to VGPRs (no accumulator-register reads)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(debug: bool = False, jobs: int = 4, verbose: bool = False, checked: bool = False) -> str:
    """Build libidxtopk.so (or, with checked=True, libidxtopk_checked.so:
    -O3 plus the device-side checks)."""
    hipcc = _hipcc()
    bdir = os.path.join(BUILD_DIR, "checked") if checked else BUILD_DIR
    out_path = CHECKED_LIB_PATH if checked else LIB_PATH
    os.makedirs(bdir, exist_ok=True)
    opt = ["-O1", "-g"] if debug else ["-O3"]
    if checked:
        opt = opt + ["-DIDXTOPK_CHECKS=1"]
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON_FLAGS, *opt, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max(1, jobs)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = out_path + ".tmp"
    _run([hipcc, *COMMON_FLAGS, "-shared", *objs, "-o", tmp])
    os.replace(tmp, out_path)
    return out_path


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--checked", action="store_true", help="build libidxtopk_checked.so (device-side checks)")
    ap.add_argument("-j", "--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(debug=a.debug, jobs=a.jobs, verbose=a.verbose, checked=a.checked)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
