"""Pins for the oracle's compositions: the prolog chain's order (RoPE, then Hadamard, then the
quantizer), the per-token broadcast of the rotary tables over query heads, and the whole decode
step against a brute-force walk through its definitions.

Each pin uses values fixed by the mathematics rather than by re-running the oracle's own
formula: a unit input vector through an orthonormal Sylvester Hadamard gives +-1/sqrt(D)
everywhere, so the quantizer's codes are known in closed form; a rotated unit vector has
closed-form coordinates when the caller's cos/sin are (0.6, 0.8).
"""
import math

import numpy as np

import oracle
from oracle.formats import bf16_decode
from oracle.prolog import indexer_prolog, prolog_rows
from workloads import Spec, make

D = 128


def _sylvester_sign(i: int, j: int) -> int:
    """Sign of H[i, j] for the Sylvester Hadamard matrix: (-1)^popcount(i & j)."""
    return -1 if bin(i & j).count("1") % 2 else 1


def test_unit_vector_at_position_zero_gives_full_scale_hadamard_codes():
    """[PRO] Indexer Prolog: e_i -> RoPE at position 0 (cos 1, sin 0) is e_i; times the
    orthonormal Hadamard it is row i of H, every entry +-1/sqrt(128).  The row's amax is
    1/sqrt(128), so every int8 code is +-127 with H's signs and the scale is (1/sqrt(128))/127.
    A dropped Hadamard would give a single non-zero code."""
    rows = [0, 5, 63, 64, 100, 127]
    x = np.zeros((len(rows), D), dtype=np.float32)
    for r, i in enumerate(rows):
        x[r, i] = 1.0
    cos = np.ones((len(rows), 32), dtype=np.float32)
    sin = np.zeros((len(rows), 32), dtype=np.float32)
    codes, stored, s = prolog_rows(x, cos, sin, 64, 64, False, True, "i8", "f32")
    expect_s = np.float32(np.float32(1.0 / math.sqrt(128.0)) / np.float32(127.0))
    for r, i in enumerate(rows):
        want = [127 * _sylvester_sign(i, j) for j in range(D)]
        assert codes[r].astype(int).tolist() == want, f"row e_{i}"
        assert s[r] == expect_s


def test_rotated_unit_vector_then_hadamard_closed_form():
    """RoPE before the Hadamard.  e_j with j in the first half of the rotated pairs
    (j = 64 + i, partner j + 32) and the caller's cos/sin = (0.6, 0.8) becomes
    0.6 e_j + 0.8 e_{j+32}; times H its entries are (0.6 s_j + 0.8 s_{j+32}) / sqrt(128) with
    s = +-1: +-1.4/sqrt(128) or +-0.2/sqrt(128).  amax = 1.4/sqrt(128), so the codes are +-127
    where the signs agree and +-round(127 * 0.2 / 1.4) = +-18 where they differ.  The Hadamard
    applied first, or no Hadamard, gives different codes."""
    for i in (0, 7, 31):
        j = 64 + i
        x = np.zeros((1, D), dtype=np.float32)
        x[0, j] = 1.0
        cos = np.zeros((1, 32), dtype=np.float32)
        sin = np.zeros((1, 32), dtype=np.float32)
        cos[:] = 1.0
        cos[0, i], sin[0, i] = 0.6, 0.8
        codes, _, s = prolog_rows(x, cos, sin, 64, 64, False, True, "i8", "f32")
        want = []
        for c in range(D):
            a, b = _sylvester_sign(j, c), _sylvester_sign(j + 32, c)
            want.append(127 * a if a == b else 18 * (1 if 0.6 * a + 0.8 * b > 0 else -1))
        assert codes[0].astype(int).tolist() == want, f"pair {i}"
        assert abs(float(s[0]) - 1.4 / math.sqrt(128.0) / 127.0) <= 1e-6 * float(s[0])
        # the second element of the pair: e_{j+32} -> -0.8 e_j + 0.6 e_{j+32}
        x2 = np.zeros((1, D), dtype=np.float32)
        x2[0, j + 32] = 1.0
        codes2, _, _ = prolog_rows(x2, cos, sin, 64, 64, False, True, "i8", "f32")
        want2 = []
        for c in range(D):
            a, b = _sylvester_sign(j, c), _sylvester_sign(j + 32, c)
            v = -0.8 * a + 0.6 * b
            want2.append(127 * (1 if v > 0 else -1) if a != b else 18 * (1 if v > 0 else -1))
        assert codes2[0].astype(int).tolist() == want2, f"pair {i}, second element"


def test_query_heads_take_their_tokens_rotary_tables(rng):
    """[PRO]: every head of query token t is rotated with token t's position.  If each head row
    of token t equals key row r_t and token t's cos/sin equal key row r_t's, every head's codes
    and scale equal that key row's.  Three tokens at distinct positions and four heads: a table
    broadcast in the wrong order (per head instead of per token) breaks it."""
    T, H = 3, 4
    k_in = rng.standard_normal((T, D)).astype(np.float32)
    ang = np.array([3.0, 1000.0, 40000.0])[:, None] * (10000.0 ** (-np.arange(32) * 2 / 64))[None, :]
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    q_in = np.repeat(k_in[:, None, :], H, axis=1)
    for code in ("i8", "e4m3"):
        out = indexer_prolog(q_in, k_in, cos, sin, cos, sin, 64, 64, False, True, code, "f16")
        for t in range(T):
            for h in range(H):
                assert np.array_equal(out["q_codes"][t, h], out["k_codes"][t]), (code, t, h)
                assert out["q_scale"][t, h] == out["k_scale"][t]


def _brute_step(wl, k):
    """The decode step from its definitions, one token, head and key at a time:
    [PRO] per-row prolog (quant only for this workload) -> [LI] scores over the token's own
    sequence, s = 0 .. p_t -> TopK by a full sort (ties to the lower position) -> [SFA]
    softmax over the selected rows with the sink in the denominator."""
    sp = wl.spec
    kc, ks, qc, qs = {}, {}, {}, {}
    for r in range(wl.N):
        c, s, _ = prolog_rows(wl.idx_k_in[r:r + 1], None, None, 0, 0, False, False, sp.code, sp.scale_dt)
        kc[r], ks[r] = c[0].astype(np.float64), float(s[0])
    for t in range(wl.T):
        for h in range(sp.H):
            c, s, _ = prolog_rows(wl.idx_q_in[t, h:h + 1], None, None, 0, 0, False, False, sp.code,
                                  sp.scale_dt)
            qc[t, h], qs[t, h] = c[0].astype(np.float64), float(s[0])
    q = bf16_decode(wl.q)
    kv = bf16_decode(wl.kv)
    idx = np.full((wl.T, k), -1, dtype=np.int32)
    out = np.zeros((wl.T, sp.Hq, 512))
    scores = []
    for t in range(wl.T):
        b, p = int(wl.q_seq[t]), int(wl.q_pos[t])
        row0 = int(wl.kv_start[b])
        I = []
        for s_ in range(p + 1):
            tot = 0.0
            for h in range(sp.H):
                d = sum(qc[t, h][j] * kc[row0 + s_][j] for j in range(sp.D))
                tot += float(wl.w[t, h]) * max(qs[t, h] * ks[row0 + s_] * d, 0.0)
            I.append(tot)
        scores.append(np.array(I))
        order = sorted(range(p + 1), key=lambda s_: (-I[s_], s_))[:min(k, p + 1)]
        sel = sorted(order)
        idx[t, :len(sel)] = sel
        for h in range(sp.Hq):
            z = [wl.scale * float(np.dot(q[t, h], kv[row0 + j])) for j in sel]
            snk = float(wl.sink[h]) if wl.sink is not None else -math.inf
            m = max(max(z), snk)
            e = [math.exp(v - m) for v in z]
            den = sum(e) + (math.exp(snk - m) if snk > -math.inf else 0.0)
            out[t, h] = sum(ei * kv[row0 + j, :512] for ei, j in zip(e, sel)) / den
    return scores, idx, out


def test_decode_step_equals_brute_force_composition():
    """[DIA] the decode layer = prolog -> indexer -> TopK -> SFA.  Two sequences of different
    lengths (the second with two query tokens), a k that truncates the longer rows and pads the
    shortest, a sink on 16 heads: the oracle's step must reproduce the brute-force walk."""
    sp = Spec("compose_tiny", 4242, [23, 41], [1, 2], H=4, D=16, scale_dt="f32", k=24, Hq=16)
    wl = make(sp)
    ref = oracle.decode_step(wl)
    scores, idx, out = _brute_step(wl, sp.k)
    for t in range(wl.T):
        assert np.allclose(ref["scores"][t], scores[t], rtol=1e-12, atol=1e-12)
    assert np.array_equal(ref["idx"], idx)
    assert np.allclose(ref["out"], out, rtol=1e-10, atol=1e-12)
    # the shortest row (p = 22 < k) keeps every position and pads with -1
    assert idx[0, :23].tolist() == list(range(23)) and np.all(idx[0, 23:] == -1)


def test_quantize_workload_rows_follow_their_positions():
    """With the full prolog, cache row r of sequence b carries position r - kv_start[b]: each
    key row quantized alone with the rotary table of that position must match the workload's
    cache, and each query token with the table of q_pos."""
    sp = Spec("compose_fp8", 4243, [9, 6], [2, 1], code="e4m3", full_prolog=True, k=4, Hq=16)
    wl = make(sp)
    q = oracle.step.quantize_workload(wl)
    kin = bf16_decode(wl.idx_k_in).astype(np.float32)
    qin = bf16_decode(wl.idx_q_in).astype(np.float32)
    inv = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    for b, L in enumerate(wl.seq_lens):
        for pos in range(int(L)):
            r = int(wl.kv_start[b]) + pos
            c, s = np.cos(pos * inv).astype(np.float32)[None], np.sin(pos * inv).astype(np.float32)[None]
            codes, st, _ = prolog_rows(kin[r:r + 1], c, s, 64, 64, False, True, "e4m3", "f16")
            assert np.array_equal(q["k_codes"][r], codes[0]) and q["k_scale"][r] == st[0]
    for t in range(wl.T):
        pos = int(wl.q_pos[t])
        c, s = np.cos(pos * inv).astype(np.float32)[None], np.sin(pos * inv).astype(np.float32)[None]
        for h in range(sp.H):
            codes, st, _ = prolog_rows(qin[t, h:h + 1], c, s, 64, 64, False, True, "e4m3", "f16")
            assert np.array_equal(q["q_codes"][t, h], codes[0]) and q["q_scale"][t, h] == st[0]
