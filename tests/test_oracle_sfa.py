"""Pins for oracle/sfa.py: dense softmax, sink closed form, single key, permutation, convexity."""
import numpy as np
import scipy.special
import torch

from oracle.formats import bf16_decode, bf16_encode
from oracle.sfa import sparse_attention


def _data(rng, N=40, T=2, Hq=4):
    kv = bf16_encode(rng.standard_normal((N, 576)).astype(np.float32))
    q = bf16_encode(rng.standard_normal((T, Hq, 576)).astype(np.float32))
    return kv, q


SCALE = 1 / 24.0


def test_no_sink_full_set_is_dense_softmax(rng):
    kv, q = _data(rng)
    idx = np.tile(np.arange(40, dtype=np.int32), (2, 1))
    got = sparse_attention(q, kv, idx, [0, 0], [0], None, SCALE)
    K, Q = bf16_decode(kv), bf16_decode(q)
    for t in range(2):
        p = scipy.special.softmax(SCALE * Q[t] @ K.T, axis=1)
        assert np.allclose(got[t], p @ K[:, :512], rtol=1e-12, atol=1e-14)
        sd = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[t])[None], torch.from_numpy(K)[None],
            torch.from_numpy(K[:, :512].copy())[None], scale=SCALE)[0].numpy()
        assert np.allclose(got[t], sd, rtol=1e-10, atol=1e-12)


def test_sink_closed_form(rng):
    kv, q = _data(rng)
    idx = np.tile(np.arange(0, 40, 3, dtype=np.int32), (2, 1))
    sink = rng.standard_normal(4) * 2
    plain = sparse_attention(q, kv, idx, [0, 0], [0], None, SCALE)
    withs = sparse_attention(q, kv, idx, [0, 0], [0], sink, SCALE)
    K, Q = bf16_decode(kv)[idx[0]], bf16_decode(q)
    for t in range(2):
        z = SCALE * Q[t] @ K.T
        se = np.exp(z).sum(1)
        assert np.allclose(withs[t], plain[t] * (se / (se + np.exp(sink)))[:, None], rtol=1e-12)


def test_single_key_and_large_sink(rng):
    kv, q = _data(rng)
    idx = np.full((2, 8), -1, np.int32)
    idx[:, 3] = 17
    got = sparse_attention(q, kv, idx, [0, 0], [0], None, SCALE)
    assert np.array_equal(got[0], np.tile(bf16_decode(kv[17, :512]), (4, 1)))
    big = sparse_attention(q, kv, idx, [0, 0], [0], np.full(4, 1e4), SCALE)
    assert np.all(big == 0)


def test_empty_selection_is_zero(rng):
    kv, q = _data(rng)
    idx = np.full((2, 8), -1, np.int32)
    assert not sparse_attention(q, kv, idx, [0, 0], [0], np.zeros(4), SCALE).any()
    assert not sparse_attention(q, kv, idx, [0, 0], [0], None, SCALE).any()


def test_permutation_padding_and_offsets(rng):
    kv, q = _data(rng, N=60)
    sel = np.array([3, 9, 10, 22, 31], np.int32)
    a = sparse_attention(q[:1], kv, sel[None], [1], [0, 20], None, SCALE)
    b = sparse_attention(q[:1], kv, np.array([[31, -1, 3, 22, -1, 10, 9]], np.int32), [1], [0, 20], None, SCALE)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    c = sparse_attention(q[:1], kv[20:], sel[None], [0], [0], None, SCALE)     # kv_start shift
    assert np.allclose(a, c, rtol=1e-13, atol=1e-15)


def test_duplicates_count_twice(rng):
    kv, q = _data(rng)
    a = sparse_attention(q[:1], kv, np.array([[4, 4, 7]], np.int32), [0], [0], None, SCALE)
    K, Q = bf16_decode(kv), bf16_decode(q)
    z = SCALE * Q[0] @ K[[4, 7]].T
    wts = np.exp(z) * np.array([2.0, 1.0])
    ref = (wts @ K[[4, 7], :512]) / wts.sum(1, keepdims=True)
    assert np.allclose(a[0], ref, rtol=1e-12)


def test_convexity_bound(rng):
    kv, q = _data(rng)
    idx = rng.choice(40, size=(2, 16), replace=False).astype(np.int32)
    out = sparse_attention(q, kv, idx, [0, 0], [0], rng.standard_normal(4), SCALE)
    V = bf16_decode(kv)[:, :512]
    for t in range(2):
        assert np.all(np.abs(out[t]) <= np.abs(V[idx[t]]).max(0) + 1e-12)
