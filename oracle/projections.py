"""Upstream projections of the Indexer Prolog (oracle; test-only).

[PRO] "Indexer Prolog", formulas and quantization strategy:
  * indexer query:  q_pre = DeQuant(q . w_qb), with q and w_qb both int8 (the W8A8 linear);
    the result then goes through RoPE -> Hadamard -> per-token-head quant (prolog.py);
  * indexer key:    k_pre = LayerNorm(x . w_k), then the same chain into the cache;
  * indexer weight: weight = (x . w_proj) * scale, not quantized, stored as FP16;
  * dequant factors are stored in FP16.
[AQ] "Int8 GEMM" (same page as [AQ], the int8 matmul operator): int8 x int8 -> int32, cast to
float, multiplied by the per-row scale of A and the per-column scale of B.

Readings (where the pages leave a step open):
  * The W8A8 scales are per row of q (per token) and per output channel of w_qb; the int32
    product is exact, the dequant is (acc * a_scale[t]) * b_scale[n] with the scales read from
    their stored (fp16) values.
  * LayerNorm is the textbook one over the D dims of a token's key: (v - mean) / sqrt(var + eps)
    * gamma + beta, population variance; gamma, beta and eps are inputs.
  * x, w_k and w_proj are bf16 values; the products are exact and the sums are real-valued
    (computed here in float64).  Weights are stored as [out, in] rows.
  * The weight's final cast to FP16 rounds to nearest even.
Pins: tests/test_oracle_projections.py.
"""
import numpy as np

from .formats import fp16_round


def w8a8_dequant(a_i8: np.ndarray, a_scale: np.ndarray, b_i8: np.ndarray,
                 b_scale: np.ndarray) -> np.ndarray:
    """[M, K] int8 . ([N, K] int8)^T -> int64 exact, then * a_scale[m] * b_scale[n] (float64)."""
    acc = np.asarray(a_i8, dtype=np.int64) @ np.asarray(b_i8, dtype=np.int64).T
    return acc.astype(np.float64) * np.asarray(a_scale, np.float64)[:, None] \
        * np.asarray(b_scale, np.float64)[None, :]


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [M, K] . (w [N, K])^T in float64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def layer_norm(v: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis (float64)."""
    v = np.asarray(v, dtype=np.float64)
    mean = v.mean(axis=-1, keepdims=True)
    var = ((v - mean) ** 2).mean(axis=-1, keepdims=True)
    return (v - mean) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def indexer_projections(qa_i8, qa_scale, w_qb_i8, w_qb_scale, x, w_k, gamma, beta, eps,
                        w_proj, weight_scale):
    """The three projections: q_pre [T, H*D], k_pre [T, D] (float64) and weight [T, H] (float64
    values of the fp16 result)."""
    q_pre = w8a8_dequant(qa_i8, qa_scale, w_qb_i8, w_qb_scale)
    k_pre = layer_norm(linear(x, w_k), gamma, beta, eps)
    weight = fp16_round(linear(x, w_proj) * weight_scale)
    return q_pre, k_pre, weight
