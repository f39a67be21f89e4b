"""libidxtopk: sparse-attention indexer top-k (fp8) for AMD Instinct MI355X.

The compute path is the HIP library ``libidxtopk.so`` (C ABI in
``include/idxtopk.h``). This package only builds it and marshals torch tensors
into its calls.
"""
from ._lib import (IdxTopkError, LibraryMissing, OP_BLOCK_TOPK, OP_SCORE_TOPK_FUSED, LIB_PATH,  # noqa: F401
                   load)

__all__ = [
    "load", "LIB_PATH", "IdxTopkError", "LibraryMissing", "ops",
    "topk_rows", "topk_page_transform", "idx_score_fp8", "idx_score_topk_fused", "block_topk",
    "workspace_bytes", "Workspace",
]


def __getattr__(name):
    # ops imports torch; keep `import sparse_attention_indexer_fp8_amd` light
    if name in ("ops", "topk_rows", "topk_page_transform", "idx_score_fp8", "idx_score_topk_fused",
                "block_topk", "workspace_bytes", "Workspace"):
        import importlib

        mod = importlib.import_module(__name__ + ".ops")
        return mod if name == "ops" else getattr(mod, name)
    raise AttributeError(name)
