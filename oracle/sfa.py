"""Sparse Flash Attention with a per-head attention sink (oracle; test-only).

[SFA] inputs: query [b, m, h, d], key/value [b, n, d], topk_idxs [b, m, k], attn_sink [h];
output [b, m, h, d].  Steps 2-7: build the index list (positions past the selection are
-1 and contribute nothing), scores = query . key^T times the softmax scale, a softmax
kept online (running max and sum), then score . value, a final rescale, and the
attention-sink term for each query head.  The tiling and the online form are how the
kernel gets there; the oracle writes out the result they reach:

    z_j = scale * q[t, h, :576] . kv[row_j, :576]           for j in J_t = {idx != -1}
    m   = max(max_j z_j, sink_h)
    o   = sum_j e^(z_j - m) kv[row_j, :512] / (sum_j e^(z_j - m) + e^(sink_h - m))

Readings: the sink is a per-head logit in the scaled-score domain that joins the softmax
denominator only (the printed sink line is garbled; dividing by e^(sink - max) as
printed would not reduce to plain softmax when the sink is -inf, which the method's own
"no sink" case requires); MLA latent rows are absorbed MQA: the key is all 576 columns
(512 nope + 64 rope) and the value is the first 512 columns of the same row, shared by
every query head; an empty J gives o = 0; duplicate indices count with multiplicity;
`sink=None` means no sink (-inf).  Index j is a position inside token t's sequence;
its row is kv_start[seq(t)] + j.
Pins: tests/test_oracle_sfa.py (dense softmax, closed form with sink, single key,
permutation, convexity, torch SDPA on CPU).
"""
import numpy as np

from .formats import bf16_decode

D_V = 512


def sparse_attention(q_bits, kv_bits, idx, q_seq, kv_start, sink, scale):
    """q_bits [T, Hq, 576] bf16 bits, kv_bits [N, 576] bf16 bits, idx [T, k] int32
    -> float64 [T, Hq, 512]."""
    q = bf16_decode(q_bits)
    T, Hq, _ = q.shape
    out = np.zeros((T, Hq, D_V), dtype=np.float64)
    snk = np.full(Hq, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    for t in range(T):
        J = idx[t][idx[t] >= 0].astype(np.int64)
        if J.size == 0:
            continue
        rows = bf16_decode(kv_bits[int(kv_start[q_seq[t]]) + J])       # [|J|, 576]
        z = scale * (q[t] @ rows.T)                                    # [Hq, |J|]
        m = np.maximum(z.max(axis=1), snk)                             # [Hq]
        p = np.exp(z - m[:, None])
        den = p.sum(axis=1) + np.exp(snk - m)
        out[t] = (p @ rows[:, :D_V]) / den[:, None]
    return out
