"""MI355X (gfx950) DeepSeek sparse-attention decode path: HIP kernels behind a C ABI.

    from sparse_attention_14_amd import dsa            # the binding (same names as dsa.h)
    from sparse_attention_14_amd.step import decode_step

Importing fails loudly if libdsa.so has not been built; there is no fallback path.
"""
from . import dsa  # noqa: F401  (loads libdsa.so)
from .dsa import (Batch, make_batch, dsa_indexer_prolog, dsa_indexer_scores, dsa_indexer_dots_i32,
                  dsa_topk, dsa_topk_workspace_size, dsa_sparse_attn_decode,
                  dsa_sparse_attn_workspace_size, dsa_last_error, dsa_version)

__all__ = ["dsa", "Batch", "make_batch", "dsa_indexer_prolog", "dsa_indexer_scores",
           "dsa_indexer_dots_i32", "dsa_topk", "dsa_topk_workspace_size", "dsa_sparse_attn_decode",
           "dsa_sparse_attn_workspace_size", "dsa_last_error", "dsa_version"]
