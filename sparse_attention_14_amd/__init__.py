"""MI355X (gfx950) DeepSeek sparse-attention decode path: HIP kernels behind a C ABI.

    from sparse_attention_14_amd import dsa            # the binding (same names as dsa.h)
    from sparse_attention_14_amd.step import decode_step

The binding loads libdsa.so when it is first used and raises ImportError if the library has
not been built (python -m sparse_attention_14_amd.build); there is no fallback path.  The
package itself imports without the library so that the build module can run.
"""
import importlib

_EXPORTS = ("Batch", "make_batch", "dsa_indexer_prolog", "dsa_indexer_scores",
            "dsa_indexer_dots_i32", "dsa_e4m3_dots", "dsa_indexer_prolog_topk", "dsa_topk", "dsa_topk_workspace_size", "dsa_sparse_attn_decode",
            "dsa_sparse_attn_workspace_size", "dsa_indexer_attention",
            "dsa_indexer_attention_workspace_size", "dsa_last_error", "dsa_version")

__all__ = ["dsa", *_EXPORTS]


def __getattr__(name):
    if name == "dsa":
        return importlib.import_module(".dsa", __name__)
    if name in _EXPORTS:
        return getattr(importlib.import_module(".dsa", __name__), name)
    raise AttributeError(name)
