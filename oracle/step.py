"""One DSA decode step end to end (oracle; test-only).

[DIA] the decode layer is the indexer prolog, the Lightning Indexer with its TopK, and
Sparse Flash Attention (the MLA prolog that produces the attention query and latent KV
needs trained projection weights and is not part of this path; its outputs are inputs).

The cache state: every cache row's key has gone through the prolog (earlier steps wrote
the old rows; this step writes the rows of its own query tokens), so each query token
sees positions 0 .. p_t, itself included.
Pins: tests/test_oracle_compose.py (the step against a brute-force walk through the
definitions; every cache row and query token quantized with the rotary table of its own
position).
"""
import numpy as np

from .formats import bf16_decode
from .prolog import indexer_prolog
from .indexer import indexer_scores
from .topk import topk_select
from .sfa import sparse_attention


def prolog_inputs_f64(wl):
    """Raw prolog inputs of a workload as float values (bf16 bits widened exactly)."""
    if wl.in_dtype == "bf16":
        return bf16_decode(wl.idx_q_in).astype(np.float32), bf16_decode(wl.idx_k_in).astype(np.float32)
    return wl.idx_q_in, wl.idx_k_in


def quantize_workload(wl):
    """The prolog over every query token and every cache row of a workload."""
    sp = wl.spec
    q_in, k_in = prolog_inputs_f64(wl)
    rope = sp.rope_dim if sp.full_prolog else 0
    return indexer_prolog(q_in, k_in, wl.q_cos, wl.q_sin, wl.k_cos, wl.k_sin, rope,
                          sp.rope_offset, sp.rope_interleaved, sp.full_prolog, sp.code,
                          sp.scale_dt)


def decode_step(wl, quant=None):
    """Returns dict(quant, scores (list), idx [T, k], out [T, Hq, 512] float64)."""
    sp = wl.spec
    if quant is None:
        quant = quantize_workload(wl)
    scores = indexer_scores(quant["q_codes"], quant["q_scale"], wl.w, quant["k_codes"],
                            quant["k_scale"], sp.code, wl.q_seq, wl.q_pos, wl.kv_start)
    idx = topk_select(scores, sp.k)
    out = sparse_attention(wl.q, wl.kv, idx, wl.q_seq, wl.kv_start, wl.sink, wl.scale)
    return {"quant": quant, "scores": scores, "idx": idx, "out": out}
