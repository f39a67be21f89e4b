"""The C-ABI library loads, exports what include/idxtopk.h declares, and rejects
bad arguments on the host (every call here returns before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idxtopk.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def _defines():
    out = {}
    for m in re.finditer(r"#define\s+(IDXTOPK_[A-Z0-9_]+)\s+\(?(-?(?:0x[0-9a-fA-F]+|\d+))u?\)?", open(HEADER).read()):
        out[m.group(1)] = int(m.group(2), 0)
    return out


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_indexer_fp8_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_indexer_fp8_amd import build
        build.build()
    return _lib.load()


def test_header_declares_the_ops():
    names = _declared_functions()
    for op in ("idx_score_fp8", "topk_rows", "idx_score_topk_fused", "topk_page_transform", "block_topk",
               "idx_cache_write", "idx_score_topk_prefill"):
        assert op in names
    assert {"idxtopk_workspace_bytes", "idxtopk_status_str", "idxtopk_version"} <= set(names)


def test_every_declared_symbol_is_exported(lib):
    from sparse_attention_indexer_fp8_amd import _lib
    names = _declared_functions()
    assert set(names) == set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_status_codes_and_version(lib):
    d = _defines()
    from sparse_attention_indexer_fp8_amd import _lib
    assert (d["IDXTOPK_OK"], d["IDXTOPK_EINVAL"], d["IDXTOPK_EUNSUPPORTED"], d["IDXTOPK_EWORKSPACE"],
            d["IDXTOPK_ELAUNCH"]) == (_lib.IDXTOPK_OK, _lib.IDXTOPK_EINVAL, _lib.IDXTOPK_EUNSUPPORTED,
                                      _lib.IDXTOPK_EWORKSPACE, _lib.IDXTOPK_ELAUNCH)
    assert lib.idxtopk_version() == d["IDXTOPK_VERSION"]
    texts = {lib.idxtopk_status_str(s).decode() for s in (0, -1, -2, -3, -4, 7)}
    assert len(texts) == 6


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails host validation
NULL = None


def _topk_rows(lib, **kw):
    a = dict(scores=FAKE, stride=4096, rows=8, seq_lens=FAKE, rs=NULL, r2b=NULL, pt=NULL, pts=0, P=1,
             k=512, out=FAKE, flags=0)
    a.update(kw)
    return lib.topk_rows(a["scores"], a["stride"], a["rows"], a["seq_lens"], a["rs"], a["r2b"], NULL, a["pt"],
                         a["pts"], a["P"], a["k"], a["out"], a["flags"], NULL)


def test_topk_rows_validation(lib):
    assert _topk_rows(lib, rows=-1) == -1
    assert _topk_rows(lib, k=0) == -1
    assert _topk_rows(lib, stride=-5) == -1
    assert _topk_rows(lib, scores=NULL) == -1
    assert _topk_rows(lib, seq_lens=NULL) == -1
    assert _topk_rows(lib, out=NULL) == -1
    assert _topk_rows(lib, pt=FAKE, P=0) == -1
    assert _topk_rows(lib, pt=FAKE, pts=-1) == -1
    assert _topk_rows(lib, k=8193) == -2
    assert _topk_rows(lib, flags=2) == -1          # unknown flag bit
    assert _topk_rows(lib, flags=1, rows=-1) == -1
    assert _topk_rows(lib, rows=0) == 0  # nothing to do, nothing enqueued
    assert _topk_rows(lib, rows=0, flags=1) == 0


def test_page_transform_validation(lib):
    f = lib.topk_page_transform
    assert f(FAKE, -1, 4, FAKE, 10, 1, NULL, FAKE, NULL) == -1
    assert f(FAKE, 2, 0, FAKE, 10, 1, NULL, FAKE, NULL) == -1
    assert f(FAKE, 2, 4, FAKE, 10, 0, NULL, FAKE, NULL) == -1
    assert f(NULL, 2, 4, FAKE, 10, 1, NULL, FAKE, NULL) == -1
    assert f(FAKE, 2, 4, NULL, 10, 1, NULL, FAKE, NULL) == -1
    assert f(FAKE, 0, 4, FAKE, 10, 1, NULL, FAKE, NULL) == 0


def _indexer(**kw):
    a = dict(q=FAKE, qs=FAKE, w=FAKE, kc=FAKE, ks=FAKE, bt=FAKE, bts=256, P=64, r2b=NULL, sl=FAKE, B=32, H=64,
             D=128, msl=16384)
    a.update(kw)
    return [a["q"], a["qs"], a["w"], a["kc"], a["ks"], a["bt"], a["bts"], a["P"], a["r2b"], a["sl"], a["B"],
            a["H"], a["D"], a["msl"]]


def test_score_validation(lib):
    f = lambda out=FAKE, ss=16384, **kw: lib.idx_score_fp8(*_indexer(**kw), out, ss, NULL)
    assert f(D=64) == -2
    assert f(H=48) == -2
    assert f(H=0) == -1
    assert f(P=0) == -1
    assert f(q=NULL) == -1
    assert f(kc=NULL) == -1
    assert f(out=NULL) == -1
    assert f(ss=100) == -1          # max_seq_len beyond the score row
    assert f(bts=10) == -1          # block table too narrow for max_seq_len
    assert f(B=0) == 0


def test_fused_validation_and_workspace(lib):
    need = lib.idxtopk_workspace_bytes(4, 32, 2048, 16384)
    assert need > 32 * 16384 * 8
    f = lambda k=2048, out=FAKE, ws=FAKE, nb=need, flags=0, **kw: lib.idx_score_topk_fused(
        *_indexer(**kw), k, out, NULL, ws, nb, flags, NULL)
    assert f(k=0) == -1
    assert f(k=8193) == -2
    assert f(out=NULL) == -1
    assert f(ws=NULL) == -3
    assert f(nb=need - 1) == -3
    assert f(D=256) == -2
    assert f(flags=4) == -1         # unknown flag bit
    assert f(B=0) == 0
    assert f(B=0, flags=1) == 0
    # the sorted output's score area: rows x k floats on top of the rest
    assert lib.idxtopk_workspace_bytes(4, 32, 2048, 16384) - lib.idxtopk_workspace_bytes(4, 32, 1024, 16384) \
        == 32 * 1024 * 4


def test_prefill_validation_and_workspace(lib):
    """The fused prefill indexer: argument checks and a workspace far below
    the score buffer it replaces (16384 rows x 70001 fp32 = 4.59 GB)."""
    rows, k, msl = 16384, 512, 70001
    need = lib.idxtopk_workspace_bytes(8, rows, k, msl)
    assert rows * k * 8 < need < rows * msl * 4 // 4
    assert lib.idxtopk_workspace_bytes(8, rows, 0, msl) == 0
    small = lib.idxtopk_workspace_bytes(8, 32, 512, 16384)
    f = lambda k=512, out=FAKE, ws=FAKE, nb=small, flags=0, **kw: lib.idx_score_topk_prefill(
        *_indexer(**kw), k, out, NULL, ws, nb, flags, NULL)
    assert f(k=0) == -1
    assert f(k=2049) == -2
    assert f(out=NULL) == -1
    assert f(ws=NULL) == -3
    assert f(nb=small - 1) == -3
    assert f(H=128) == -2           # 16, 32 or 64 heads
    assert f(P=8, bts=2048) == -2   # pages of whole 16-token groups
    assert f(D=256) == -2
    assert f(flags=4) == -1
    assert f(B=0) == 0


def test_block_validation(lib):
    need = lib.idxtopk_workspace_bytes(5, 32, 128, 32768)
    assert need >= 32 * 256 * 4
    f = lambda bs=128, top=32, out=FAKE, ws=FAKE, nb=need, **kw: lib.block_topk(
        *_indexer(**{"P": 128, "msl": 32768, "bts": 256, **kw}), bs, top, out, NULL, ws, nb, NULL)
    assert f(bs=64) == -2          # block size must equal page size
    assert f(top=0) == -1
    assert f(top=5000) == -2
    assert f(out=NULL) == -1
    assert f(nb=need - 1) == -3
    assert f(B=0) == 0


def test_cache_write_validation(lib):
    f = lambda keys=FAKE, dt=0, ks=128, T=16, D=128, sm=FAKE, kc=FAKE, sc=FAKE: lib.idx_cache_write(
        keys, dt, ks, T, D, sm, kc, sc, NULL)
    assert f(D=64) == -2
    assert f(dt=2) == -2
    assert f(T=-1) == -1
    assert f(keys=NULL) == -1
    assert f(sm=NULL) == -1
    assert f(kc=NULL) == -1
    assert f(sc=NULL) == -1
    assert f(ks=100) == -1            # stride shorter than a key
    assert f(ks=129) == -1            # odd stride breaks row alignment
    assert f(keys=ctypes.c_void_p(0x1004)) == -1     # fp32 rows need 8-byte alignment
    assert f(keys=ctypes.c_void_p(0x1002), dt=1) == -1  # bf16 rows need 4-byte alignment
    assert f(T=0) == 0
    assert lib.idxtopk_workspace_bytes(6, 16, 0, 128) == 0


def test_workspace_bytes_rules(lib):
    wb = lib.idxtopk_workspace_bytes
    assert wb(1, 8, 512, 4096) == 0          # topk_rows needs none
    assert wb(3, 8, 512, 4096) == 0
    assert wb(4, -1, 2048, 100) == 0
    assert wb(4, 64, 2048, 327680) >= 64 * 327680 * 8
    assert wb(4, 64, 2048, 327680) > wb(4, 32, 2048, 327680)
    assert wb(5, 64, 0, 32768) == 0


def test_binding_imports_without_gpu():
    import sparse_attention_indexer_fp8_amd as pkg
    from sparse_attention_indexer_fp8_amd import ops

    assert pkg.topk_rows is ops.topk_rows and pkg.ops is ops


def _indexer_bf16(**kw):
    a = dict(q=FAKE, w=FAKE, kc=FAKE, bt=FAKE, bts=256, P=64, r2b=NULL, sl=FAKE, B=32, H=64, D=128, msl=16384)
    a.update(kw)
    return [a["q"], a["w"], a["kc"], a["bt"], a["bts"], a["P"], a["r2b"], a["sl"], a["B"], a["H"], a["D"], a["msl"]]


MISALIGNED = ctypes.c_void_p(0x1008)


def test_bf16_validation(lib):
    f = lambda out=FAKE, ss=16384, **kw: lib.idx_score_bf16(*_indexer_bf16(**kw), out, ss, NULL)
    assert f(q=MISALIGNED) == -1     # 16-byte rows
    assert f(kc=MISALIGNED) == -1
    assert f(w=NULL) == -1
    assert f(H=48) == -2
    assert f(D=64) == -2
    assert f(ss=100) == -1
    assert f(B=0) == 0
    need = lib.idxtopk_workspace_bytes(4, 32, 2048, 16384)
    g = lambda k=2048, ws=FAKE, nb=need, flags=0, **kw: lib.idx_score_topk_fused_bf16(
        *_indexer_bf16(**kw), k, FAKE, NULL, ws, nb, flags, NULL)
    assert g(k=0) == -1
    assert g(k=8193) == -2
    assert g(flags=2) == -1
    assert g(ws=NULL) == -3
    assert g(kc=MISALIGNED) == -1
    assert g(B=0) == 0
    nb = lib.idxtopk_workspace_bytes(5, 32, 128, 32768)
    h = lambda bs=128, top=32, **kw: lib.block_topk_bf16(*_indexer_bf16(**{"P": 128, "msl": 32768, **kw}), bs, top,
                                                         FAKE, NULL, FAKE, nb, NULL)
    assert h(bs=64) == -2
    assert h(top=0) == -1
    assert h(q=MISALIGNED) == -1
    assert h(B=0) == 0


def test_cache_write_bf16_validation(lib):
    f = lambda keys=FAKE, dt=0, ks=128, T=16, D=128, sm=FAKE, kc=FAKE: lib.idx_cache_write_bf16(
        keys, dt, ks, T, D, sm, kc, NULL)
    assert f(dt=5) == -2
    assert f(D=64) == -2
    assert f(T=-1) == -1
    assert f(keys=NULL) == -1
    assert f(ks=100) == -1                # stride below dim
    assert f(ks=130) == -1                # fp32 rows 520 bytes apart: not 16-byte aligned
    assert f(dt=1, ks=132) == -1          # bf16 rows 264 bytes apart
    assert f(keys=MISALIGNED) == -1
    assert f(kc=MISALIGNED) == -1
    assert f(T=0) == 0


def test_block_heads_validation(lib):
    need = lib.idxtopk_workspace_bytes(7, 32 * 64, 128, 32768)
    assert need == lib.idxtopk_workspace_bytes(5, 32 * 64, 128, 32768)
    f = lambda bs=128, top=32, nb=need, **kw: lib.block_topk_heads(
        *_indexer(**{"P": 128, "msl": 32768, "bts": 256, **kw}), bs, top, FAKE, NULL, FAKE, nb, NULL)
    assert f(bs=64) == -2
    assert f(top=0) == -1
    assert f(nb=need - 1) == -3        # sized for batch * heads selections
    assert f(H=48) == -2
    assert f(B=0) == 0


def test_fused_noalloc_validation(lib):
    """Host-side checks of the built-in-workspace entry point (each returns
    before any HIP call): bad arguments, and a call larger than the built-in
    workspace."""
    from sparse_attention_indexer_fp8_amd import _lib

    d = _defines()

    def call(batch=4, heads=64, dim=128, msl=4096, k=256, out=FAKE, flags=0, P=64, bts=64):
        return lib.idx_score_topk_fused_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bts, P, NULL, FAKE, batch, heads,
                                                dim, msl, k, out, NULL, flags, NULL)

    assert call(batch=-1) == -1
    assert call(k=0) == -1
    assert call(out=NULL) == -1
    assert call(flags=2) == -1
    assert call(dim=64) == -2
    assert call(k=d["IDXTOPK_MAX_K_FUSED"] + 1) == -2
    assert call(batch=0) == 0
    # more than the built-in workspace holds
    big = 1 << 20
    need = lib.idxtopk_workspace_bytes(_lib.OP_SCORE_TOPK_FUSED, 64, 2048, big)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert call(batch=64, msl=big, k=2048, bts=big // 64) == -3


def test_release_build_has_no_checks(lib):
    """The release library reports that no device-side checks are compiled in
    (without touching the device); the checked build is a separate file."""
    from sparse_attention_indexer_fp8_amd import _lib

    d = _defines()
    assert lib.idxtopk_check_status(0) == _lib.CHECKS_OFF == 0x80000000
    assert (d["IDXTOPK_CHK_WINDOW"], d["IDXTOPK_CHK_SEQ_LEN"]) == (0x1, 0x8)
    assert _lib.CHECKED_LIB_PATH != _lib.LIB_PATH
