"""Pins for oracle/indexer.py: brute-force loops, exact integer dots, homogeneity, degenerate cases."""
import numpy as np

from oracle.formats import e4m3_decode, e4m3_encode
from oracle.indexer import indexer_dots, indexer_scores


def _tiny(rng, code):
    lens = [7, 12]
    q_per = [2, 1]
    kv_start = np.array([0, 7])
    q_seq = np.array([0, 0, 1])
    q_pos = np.array([5, 6, 11])
    T, H, D, N = 3, 4, 8, 19
    if code == "i8":
        q = rng.integers(-127, 128, (T, H, D)).astype(np.int8)
        k = rng.integers(-127, 128, (N, D)).astype(np.int8)
    else:
        q = e4m3_encode(rng.standard_normal((T, H, D)) * 50)
        k = e4m3_encode(rng.standard_normal((N, D)) * 50)
    qs = rng.uniform(0.001, 0.05, (T, H))
    ks = rng.uniform(0.001, 0.05, N)
    w = rng.standard_normal((T, H))
    return q, qs, w, k, ks, q_seq, q_pos, kv_start


def _brute(q, qs, w, k, ks, q_seq, q_pos, kv_start, code):
    val = (lambda c: float(c)) if code == "i8" else (lambda c: float(e4m3_decode(np.array([c], np.uint8))[0]))
    out = []
    for t in range(q.shape[0]):
        row = []
        for s in range(q_pos[t] + 1):
            r = kv_start[q_seq[t]] + s
            tot = 0.0
            for h in range(q.shape[1]):
                d = sum(val(q[t, h, i]) * val(k[r, i]) for i in range(q.shape[2]))
                tot += w[t, h] * max(0.0, qs[t, h] * ks[r] * d)
            row.append(tot)
        out.append(np.array(row))
    return out


def test_scores_match_brute_force(rng):
    for code in ("i8", "e4m3"):
        args = _tiny(rng, code)
        got = indexer_scores(*args[:5], code, *args[5:])
        ref = _brute(*args, code)
        assert [g.shape for g in got] == [(6,), (7,), (12,)]
        for g, r in zip(got, ref):
            assert np.allclose(g, r, rtol=1e-12, atol=1e-15)


def test_int8_dots_exact_against_int64_matmul(rng):
    q = rng.integers(-127, 128, (3, 64, 128)).astype(np.int8)
    k = rng.integers(-127, 128, (300, 128)).astype(np.int8)
    d = indexer_dots(q, k, "i8", np.array([0, 0, 1]), np.array([99, 150, 149]), np.array([0, 150]))
    ref = np.einsum("thd,nd->thn", q.astype(np.int64), k.astype(np.int64))
    assert np.array_equal(d[0], ref[0][:, :100]) and np.array_equal(d[1], ref[1][:, :151])
    assert np.array_equal(d[2], ref[2][:, 150:300])
    # extreme codes: |D| reaches 128 * 127^2, still exact
    qq = np.full((1, 1, 128), -127, np.int8)
    kk = np.full((1, 128), -127, np.int8)
    assert indexer_dots(qq, kk, "i8", [0], [0], [0])[0][0, 0] == 128 * 127 * 127


def test_scores_homogeneous_in_w_and_scale_factoring(rng):
    q, qs, w, k, ks, q_seq, q_pos, kv_start = _tiny(rng, "i8")
    a = indexer_scores(q, qs, w, k, ks, "i8", q_seq, q_pos, kv_start)
    b = indexer_scores(q, qs, 3.0 * w, k, ks, "i8", q_seq, q_pos, kv_start)
    for x, y in zip(a, b):
        assert np.allclose(3.0 * x, y, rtol=1e-14)
    # scales are positive, so k_scale factors out of the ReLU (the form the kernel uses)
    d = indexer_dots(q, k, "i8", q_seq, q_pos, kv_start)
    for t in range(3):
        r0 = kv_start[q_seq[t]]
        alt = ks[r0:r0 + q_pos[t] + 1] * np.sum((w[t] * qs[t])[:, None] * np.maximum(d[t], 0), 0)
        assert np.allclose(a[t], alt, rtol=1e-12, atol=1e-14)


def test_scores_zero_when_all_dots_nonpositive(rng):
    q = rng.integers(0, 128, (2, 4, 8)).astype(np.int8)
    k = -rng.integers(0, 128, (10, 8)).astype(np.int8)
    out = indexer_scores(q, np.ones((2, 4)), np.ones((2, 4)), k, np.ones(10), "i8",
                         [0, 0], [8, 9], [0])
    assert all(np.all(o == 0) for o in out)
