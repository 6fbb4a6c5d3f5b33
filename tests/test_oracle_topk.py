"""Pins for oracle/topk.py: full sort, short rows, permutation, ties."""
import numpy as np

from oracle.topk import kth_score, topk_select


def test_topk_equals_full_sort(rng):
    rows = [rng.standard_normal(n) for n in (5000, 2048, 3000)]
    got = topk_select(rows, 256)
    for r, g in zip(rows, got):
        full = np.argsort(-r)[:256]
        assert set(g.tolist()) == set(full.tolist()) and np.all(np.diff(g) > 0)
        assert np.min(r[g]) == kth_score(r, 256) == np.sort(r)[::-1][255]


def test_topk_short_rows_pad():
    got = topk_select([np.arange(5.0), np.zeros(1)], 8)
    assert got.tolist() == [[0, 1, 2, 3, 4, -1, -1, -1], [0, -1, -1, -1, -1, -1, -1, -1]]


def test_topk_permutation_equivariant(rng):
    r = rng.standard_normal(1000)
    perm = rng.permutation(1000)
    a = set(topk_select([r], 100)[0].tolist())
    b = set(perm[topk_select([r[perm]], 100)[0]].tolist())
    assert a == b


def test_topk_ties_take_lower_positions():
    r = np.array([1.0, 2.0, 2.0, 0.5, 2.0, 2.0])
    assert topk_select([r], 3)[0].tolist() == [1, 2, 4]
    assert topk_select([np.zeros(10)], 4)[0].tolist() == [0, 1, 2, 3]
