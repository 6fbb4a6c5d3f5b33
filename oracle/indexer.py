"""Lightning Indexer scores (oracle; test-only).

[LI] the indexer multiplies the quantized query of every head against the quantized key
cache, applies ReLU and a per-head weighting, and sums over heads; TopK follows.  [PRO]
supplies the operands: per-token-head q codes with scales, per-token k codes with
scales (C8), and FP16 head weights.  The formula itself sits in a figure the text does
not carry; the reading used here (and in the HIP path) is

    D[t, h, s] = sum_d q[t, h, d] * k[s, d]                 (exact integer for int8 codes)
    I[t, s]    = sum_h w[t, h] * ReLU(q_scale[t, h] * k_scale[s] * D[t, h, s])

for the keys s = 0 .. p_t of token t's own sequence (causal), with the stored (fp16 or
fp32) scale values.  No further softmax scale is applied.
Pins: tests/test_oracle_indexer.py (brute-force loops, homogeneity, degenerate cases).
"""
import numpy as np

from .formats import e4m3_decode


def code_values(codes: np.ndarray, code: str) -> np.ndarray:
    """Code array -> float64 values (int8 as integers, e4m3 decoded exactly)."""
    if code == "i8":
        return np.asarray(codes).astype(np.int8).astype(np.float64)
    return e4m3_decode(codes)


def indexer_dots(q_codes, k_codes, code, q_seq, q_pos, kv_start):
    """D[t] = q[t] (H x D) times k_rows(t)^T -> list of float64 [H, p_t + 1] arrays.

    Exact: int8 partial sums stay below 2^53 and e4m3 products are multiples of 2^-18
    bounded by 448^2, so float64 sums are exact in any order.
    """
    qv = code_values(q_codes, code)
    kv = code_values(k_codes, code)
    out = []
    for t in range(qv.shape[0]):
        r0 = int(kv_start[q_seq[t]])
        rows = kv[r0:r0 + int(q_pos[t]) + 1]
        out.append(qv[t] @ rows.T)
    return out


def indexer_scores(q_codes, q_scale, w, k_codes, k_scale, code, q_seq, q_pos, kv_start):
    """I[t, 0..p_t] as a list of float64 vectors (one per query token)."""
    dots = indexer_dots(q_codes, k_codes, code, q_seq, q_pos, kv_start)
    qs = np.asarray(q_scale, dtype=np.float64)
    ks = np.asarray(k_scale, dtype=np.float64)
    wv = np.asarray(w, dtype=np.float64)
    out = []
    for t, d in enumerate(dots):
        r0 = int(kv_start[q_seq[t]])
        kst = ks[r0:r0 + d.shape[1]]
        inner = qs[t][:, None] * kst[None, :] * d                   # scales inside the ReLU
        out.append(np.sum(wv[t][:, None] * np.maximum(inner, 0.0), axis=0))
    return out
