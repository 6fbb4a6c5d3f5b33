"""Pins of oracle/paged.py: the paged row formula and the paged -> flat gather.

The row formula is checked against a brute-force walk over the blocks; the gather against
round trips through random block permutations (a paged cache built by scattering a flat
cache's blocks must gather back to the flat cache bit for bit) and identity tables.
"""
import numpy as np
import pytest

from oracle import flatten_paged, paged_rows


def _walk(block_table, block_size, seq, n):
    """Row of every position 0..n-1 by walking the blocks one row at a time."""
    rows = []
    for j in range(-(-n // block_size)):
        base = int(block_table[seq][j]) * block_size
        for r in range(block_size):
            if len(rows) < n:
                rows.append(base + r)
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("block_size", [16, 128])
def test_row_formula_matches_block_walk(block_size):
    rng = np.random.default_rng(3)
    B, bps = 3, 7
    table = rng.permutation(B * bps + 5)[:B * bps].reshape(B, bps)
    for b in range(B):
        n = int(rng.integers(1, bps * block_size + 1))
        assert np.array_equal(paged_rows(table, block_size, b, np.arange(n)), _walk(table, block_size, b, n))


def _scatter(flat, kv_start, lengths, block_size, rng, spare=3):
    """A paged copy of a flat cache: every sequence's blocks go to random physical blocks."""
    nblk = [-(-n // block_size) for n in lengths]
    total = sum(nblk) + spare
    perm = rng.permutation(total)
    bps = max(nblk)
    table = np.full((len(lengths), bps), -1, dtype=np.int32)
    paged = np.zeros((total * block_size,) + flat.shape[1:], dtype=flat.dtype)
    k = 0
    for b, n in enumerate(lengths):
        for j in range(nblk[b]):
            table[b, j] = perm[k]
            k += 1
            rows = np.arange(j * block_size, min((j + 1) * block_size, n))
            paged[table[b, j] * block_size + rows - j * block_size] = flat[kv_start[b] + rows]
    return paged, table


@pytest.mark.parametrize("block_size", [16, 64, 128])
def test_paged_round_trip(block_size):
    rng = np.random.default_rng(11)
    lengths = [1, 200, 129, 64]
    kv_start = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    flat = rng.integers(-2**15, 2**15, size=(sum(lengths), 9)).astype(np.int16)
    paged, table = _scatter(flat, kv_start, lengths, block_size, rng)
    back, ks = flatten_paged(paged, table, block_size, lengths)
    assert np.array_equal(ks, kv_start)
    assert np.array_equal(back, flat)


def test_identity_table_is_the_flat_layout():
    bs, lengths = 32, [64, 96]
    table = np.array([[0, 1, 0], [2, 3, 4]], dtype=np.int32)
    cache = np.arange(5 * bs * 2).reshape(5 * bs, 2)
    back, ks = flatten_paged(cache, table, bs, lengths)
    assert np.array_equal(back, cache[:160]) and list(ks) == [0, 64]
