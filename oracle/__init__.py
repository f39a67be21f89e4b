"""CPU oracle for the sparse-attention indexer top-k path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The library (``sparse_attention_indexer_fp8_amd``) never does, and
this package imports nothing from the library. The two share no code. They
share only the seeded inputs from ``workloads``, which hold none of the
method's arithmetic.

The oracle is plain, slow and meant to be checked by eye:

* e4m3 decoding from the OCP 8-bit floating-point definition (``fp8.py``);
* e4m3 encoding by nearest-value search over the same table (``fp8.py``);
* bf16 decoding and encoding from the format's definition (``bf16.py``);
* float64 scoring (fp8 and bf16 index caches), page gathering, top-k by a
  full stable sort, the page transform, the block variant and the key-cache
  writers (``indexer.py``).

Each function names the passage of the pages it follows. Pages:

* [ATOM-1473] ROCm/ATOM pull request 1473, "enable minimax m3 fp8 index cache
  and fuse index_score_kernel with partial_topk kernel";
* [SGL-37889] sgl-project/sglang pull request 37889, "[AMD] Enable GLM DSA
  prefill top-k to the v2 kernel";
* [ATOM-1282] ROCm/ATOM pull request 1282, "merge build sparse block into
  topk".

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py``. Those tests check closed forms, a library cast, an
independent integer recomputation, brute force on tiny inputs, invariants and
hand-built cases. None is "parity unpinned".
"""
from . import bf16, fp8, indexer  # noqa: F401
from .bf16 import BF16_TABLE, decode_bf16, encode_bf16  # noqa: F401
from .fp8 import E4M3FN_TABLE, decode_e4m3fn, encode_e4m3fn  # noqa: F401
from .indexer import (  # noqa: F401
    block_scores,
    block_topk,
    block_topk_heads,
    cache_write,
    cache_write_bf16,
    index_scores_bf16,
    quantize_key,
    fused_topk,
    index_head_scores,
    index_scores,
    page_transform,
    token_slots,
    topk_order,
    topk_rows,
)
