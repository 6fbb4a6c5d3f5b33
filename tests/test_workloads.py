"""The seeded generator: shapes pinned to the pages' printed figures, determinism, layout."""
import json
import os

import numpy as np

import workloads
from workloads import NAMED, Spec, make

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")


def test_typical_shape_matches_pages():
    g = json.load(open(GOLD))
    sp = NAMED[1]
    T = sum(sp.q_per_seq)
    assert [T, sp.H * sp.D] == [g["indexer_q_matmul"]["lhs"][0], g["indexer_q_matmul"]["rhs"][1]]
    assert [T, sp.H, sp.D] == g["hadamard_batch_matmul"]["lhs"]
    assert len(sp.q_per_seq) == g["typical_shape"]["batch"]
    assert sp.q_per_seq[0] == 1 + g["typical_shape"]["mtp"]
    assert sp.seq_lens[0] == g["typical_shape"]["kv_cache_len"]
    li = g["lightning_indexer_tasks"]
    assert len(sp.seq_lens) * sp.seq_lens[0] // li["page_block"] == li["matmul_tasks"]
    assert li["matmul_tasks"] // li["l1_reuse"] == li["tasks_after_reuse"]


def test_layout_and_positions():
    wl = make(Spec("t", 7, [10, 33, 5], [2, 1, 3], H=4, D=8, k=4, Hq=16))
    assert wl.q_start.tolist() == [0, 2, 3, 6]
    assert wl.q_seq.tolist() == [0, 0, 1, 2, 2, 2]
    assert wl.q_pos.tolist() == [8, 9, 32, 2, 3, 4]
    assert wl.kv_start.tolist() == [0, 10, 43] and wl.N == 48
    assert wl.new_rows().tolist() == [8, 9, 42, 45, 46, 47]
    assert wl.kv.shape == (48, 576) and wl.q.shape == (6, 16, 576) and wl.w.dtype == np.float16


def test_deterministic_and_seed_sensitive():
    a = make(Spec("t", 5, [64], [1], H=4, D=8, k=4, Hq=16))
    b = make(Spec("t", 5, [64], [1], H=4, D=8, k=4, Hq=16))
    c = make(Spec("t", 6, [64], [1], H=4, D=8, k=4, Hq=16))
    assert np.array_equal(a.kv, b.kv) and np.array_equal(a.idx_k_in, b.idx_k_in)
    assert not np.array_equal(a.kv, c.kv)


def test_ragged_lengths_drawn_in_range():
    wl = make(Spec("r", 1002, [], [1] * 32, H=4, D=8, k=4, Hq=16))
    assert wl.seq_lens.min() >= 4096 and wl.seq_lens.max() <= 65536 and wl.B == 32


def test_prolog_workload_has_rotary_tables():
    wl = make(Spec("p", 3, [40, 50], [1, 1], H=4, D=128, code="e4m3", full_prolog=True, k=8, Hq=16))
    assert wl.in_dtype == "bf16" and wl.k_cos.shape == (90, 32) and wl.q_cos.shape == (2, 32)
    assert np.all(wl.k_cos[0] == 1.0) and np.all(wl.k_sin[0] == 0.0)      # position 0
    assert np.array_equal(wl.q_cos[1], wl.k_cos[40 + 49])                  # same position, same table
