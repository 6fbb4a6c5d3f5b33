"""Top-k token selection (oracle; test-only).

[LI] the indexer ends in a TopK over each query token's scores; [SFA] step 2 consumes
`topk_idxs [b, m, k]` and treats slots past the selection as -1 ("invalid, skip").

Readings: each token t keeps k_eff = min(k, p_t + 1) positions with the largest scores
among 0 .. p_t; ties go to the lower position (a stable sort on descending score); the
selected set is emitted in ascending position order and the remaining k - k_eff slots
are -1.
Pins: tests/test_oracle_topk.py (full sort, short rows, permutation, ties).
"""
import numpy as np


def topk_select(scores_rows, k: int) -> np.ndarray:
    """scores_rows: list of 1-D arrays (token t: scores for positions 0..p_t). -> [T, k] int32."""
    T = len(scores_rows)
    out = np.full((T, k), -1, dtype=np.int32)
    for t, s in enumerate(scores_rows):
        s = np.asarray(s, dtype=np.float64)
        n = min(k, s.shape[0])
        order = np.argsort(-s, kind="stable")[:n]
        out[t, :n] = np.sort(order)
    return out


def kth_score(scores_row, k: int) -> float:
    """The k_eff-th largest score of one row (the selection boundary I_k)."""
    s = np.sort(np.asarray(scores_row, dtype=np.float64))[::-1]
    return float(s[min(k, s.shape[0]) - 1])
