"""Paged caches (oracle; test-only).

[LI] "NPU DeepSeek-V3.2-Exp PyPTO 融合算子开发优化实践" (jsqmd.com/news/787325), Lightning
Indexer performance analysis: the 4-batch 64K decode case keeps its caches in Page Attention
blocks of 128 rows.  Reading (the page names the layout, not its table): each sequence lists
its blocks in a block table, so position p of sequence b lives in cache row

    block_table[b, p // block_size] * block_size + p % block_size.

A paged cache holds the same rows as a flat one, only placed differently, so the paged
oracle is the flat oracle applied to the rows gathered back into sequence order; nothing of
the method's arithmetic changes.
Pins: tests/test_oracle_paged.py (row formula against a brute-force walk of the blocks;
paged -> flat round trip on random block permutations; identity tables).
"""
import numpy as np


def paged_rows(block_table, block_size: int, seq: int, positions) -> np.ndarray:
    """Cache rows of `positions` (int array) of sequence `seq` under a block table."""
    pos = np.asarray(positions, dtype=np.int64)
    blocks = np.asarray(block_table, dtype=np.int64)[seq][pos // block_size]
    return blocks * block_size + pos % block_size


def flatten_paged(cache, block_table, block_size: int, lengths):
    """Gather a paged cache into sequence order: returns (flat_cache, kv_start) with sequence
    b at rows kv_start[b] .. kv_start[b] + lengths[b] - 1 of flat_cache."""
    lengths = [int(x) for x in lengths]
    kv_start = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    parts = [np.asarray(cache)[paged_rows(block_table, block_size, b, np.arange(n))]
             for b, n in enumerate(lengths)]
    flat = np.concatenate(parts, axis=0) if parts else np.asarray(cache)[:0]
    return flat, kv_start
