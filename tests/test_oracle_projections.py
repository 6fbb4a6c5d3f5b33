"""Pins of oracle/projections.py (the Indexer Prolog's upstream projections) against things
other than itself: brute-force integer sums, library routines, and invariants."""
import numpy as np
import torch

import oracle
from oracle.formats import fp16_round


def _rng():
    return np.random.default_rng(4242)


def test_w8a8_contraction_is_exact_integer_sum():
    rng = _rng()
    a = rng.integers(-127, 128, (3, 40), dtype=np.int64)
    b = rng.integers(-127, 128, (5, 40), dtype=np.int64)
    got = oracle.w8a8_dequant(a.astype(np.int8), np.ones(3), b.astype(np.int8), np.ones(5))
    for m in range(3):
        for n in range(5):
            assert got[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(40))


def test_w8a8_dequant_scales_rows_and_columns():
    rng = _rng()
    a = rng.integers(-127, 128, (4, 64)).astype(np.int8)
    b = rng.integers(-127, 128, (6, 64)).astype(np.int8)
    sa = fp16_round(rng.random(4) * 0.02 + 1e-3)
    sb = fp16_round(rng.random(6) * 0.02 + 1e-3)
    base = oracle.w8a8_dequant(a, np.ones(4), b, np.ones(6))
    got = oracle.w8a8_dequant(a, sa, b, sb)
    np.testing.assert_allclose(got, base * sa[:, None] * sb[None, :], rtol=1e-15)
    # doubling one row's scale doubles exactly that row
    sa2 = sa.copy(); sa2[1] *= 2
    g2 = oracle.w8a8_dequant(a, sa2, b, sb)
    assert np.array_equal(g2[1], 2 * got[1]) and np.array_equal(np.delete(g2, 1, 0), np.delete(got, 1, 0))
    # a zero activation row gives a zero output row
    a[2] = 0
    assert not oracle.w8a8_dequant(a, sa, b, sb)[2].any()


def test_linear_matches_torch_linear():
    rng = _rng()
    x = rng.standard_normal((3, 96))
    w = rng.standard_normal((7, 96))
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    np.testing.assert_allclose(oracle.linear(x, w), ref, rtol=1e-13, atol=1e-13)


def test_layer_norm_matches_torch_and_invariants():
    rng = _rng()
    v = rng.standard_normal((4, 128)) * 3 + 1.5
    g = rng.standard_normal(128)
    bt = rng.standard_normal(128)
    eps = 1e-6
    ref = torch.nn.functional.layer_norm(torch.from_numpy(v), (128,), torch.from_numpy(g),
                                         torch.from_numpy(bt), eps).numpy()
    got = oracle.layer_norm(v, g, bt, eps)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # unit affine: zero mean, variance var / (var + eps)
    u = oracle.layer_norm(v, np.ones(128), np.zeros(128), eps)
    np.testing.assert_allclose(u.mean(axis=1), 0, atol=1e-12)
    var = v.var(axis=1)
    np.testing.assert_allclose(u.var(axis=1), var / (var + eps), rtol=1e-12)
    # shift invariance, and a constant row maps to beta
    np.testing.assert_allclose(oracle.layer_norm(v + 7.0, g, bt, eps), got, atol=1e-10)
    c = oracle.layer_norm(np.full((1, 128), 3.25), g, bt, eps)
    np.testing.assert_allclose(c[0], bt, atol=1e-12)


def test_indexer_projections_weight_is_fp16_of_scaled_linear():
    rng = _rng()
    T, R, H, D, K = 2, 64, 4, 16, 48
    qa = rng.integers(-127, 128, (T, R)).astype(np.int8)
    wqb = rng.integers(-127, 128, (H * D, R)).astype(np.int8)
    x = rng.standard_normal((T, K))
    wk, wp = rng.standard_normal((D, K)), rng.standard_normal((H, K))
    g, bt = np.ones(D), np.zeros(D)
    q, k, w = oracle.indexer_projections(qa, np.ones(T), wqb, np.ones(H * D), x, wk, g, bt, 1e-6,
                                         wp, 0.125)
    assert q.shape == (T, H * D) and k.shape == (T, D) and w.shape == (T, H)
    assert np.array_equal(w, fp16_round((x @ wp.T) * 0.125))
    # a power-of-two weight scale commutes with the fp16 rounding (no overflow or underflow here)
    _, _, w2 = oracle.indexer_projections(qa, np.ones(T), wqb, np.ones(H * D), x, wk, g, bt, 1e-6,
                                          wp, 0.25)
    assert np.array_equal(w2, 2 * w)
