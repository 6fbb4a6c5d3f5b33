"""dsa_indexer_attention -- the indexer (with or without its prolog), top-k and sparse attention
of a decode step in one call -- against the separate calls, in both of its schedules (forced
through DSA_DIA_SCHEDULE, and the automatic choice): the attention workgroups resolving their own
slice of the selection from the top-k select pass's state, or the top-k's finalize pass first.

[DIA] "Deepseek Indexer Attention" (jsqmd.com/news/787325): the indexer prolog, the Lightning
Indexer, its TopK and the Sparse Flash Attention run in that order.  The separate calls' parity with
the oracle is covered by the parity tests; the one-call path must reproduce them bit for bit: the
scores on every visible column, the selection, the attention output and, with the prolog, the query
codes and scales and the whole key cache.  Cases: ragged batches, rows shorter than k, one token,
more than 64 sequences, the single-split attention (k = 32; 80 tokens at 128 heads), all-equal
scores (every key a candidate: the re-read path and the lowest-position tie rule), fp8 and int8
prologs, the decode workloads, 256 tokens (the row top-k; separate kernels inside the call), and
one workspace reused across shapes (its histogram rows stay zero).
"""
import os

import numpy as np
import pytest
import torch

import workloads
from workloads import Spec, make
from sparse_attention_14_amd import dsa

from gpu_common import Gpu, check_zeroed_workspace, log
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

EXTRA = {
    "k32": Spec("small_k32", 7011, [900, 40, 2000], [1, 1, 2], H=8, D=64, scale_dt="f32", k=32, Hq=16),
    "final_80": Spec("small_final_80", 7012, [3000] * 40, [2] * 40, k=512, Hq=128),
}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def visible(g, sc):
    return sc[torch.arange(sc.shape[1], device="cuda")[None, :] <= g.d["q_pos"][:, None].long()]


def separate(g: Gpu, prolog: bool, kc, ks, qc, qs):
    c, d = g.cfg, g.d
    scores = torch.empty((g.wl.T, dsa._scores_ld(g.batch.max_kv_len)), dtype=torch.float32, device="cuda")
    if prolog:
        idx = dsa.dsa_indexer_prolog_topk(
            g.batch, c.H, c.D, c.code, c.scale_dt, q_in=d["idx_q_in"],
            k_in=d["idx_k_in"][d["new_rows"]].contiguous(), w=d["w"], q_codes=qc, q_scale=qs,
            k_cache=kc, k_scale=ks, k=c.k, q_cos=d["q_cos"], q_sin=d["q_sin"], rope_dim=c.rope_dim,
            rope_offset=c.rope_offset, rope_interleaved=c.rope_interleaved, hadamard=c.hadamard,
            scores=scores)
    else:
        idx = dsa.dsa_indexer_topk(g.batch, c.H, c.D, c.code, c.scale_dt, qc, qs, d["w"], kc, ks, c.k,
                                   scores=scores)
    out = dsa.dsa_sparse_attn_decode(g.batch, d["q"], d["kv"], idx, d["sink"] if g.wl.spec.sink else None,
                                     g.wl.scale)
    return scores, idx, out


def one_call(g: Gpu, prolog: bool, kc, ks, qc, qs, ws=None):
    c, d = g.cfg, g.d
    scores = torch.empty((g.wl.T, dsa._scores_ld(g.batch.max_kv_len)), dtype=torch.float32, device="cuda")
    extra = {}
    if prolog:
        extra = dict(q_in=d["idx_q_in"], k_in=d["idx_k_in"][d["new_rows"]].contiguous(),
                     q_cos=d["q_cos"], q_sin=d["q_sin"], rope_dim=c.rope_dim, rope_offset=c.rope_offset,
                     rope_interleaved=c.rope_interleaved, hadamard=c.hadamard)
    idx, out = dsa.dsa_indexer_attention(
        g.batch, c.H, c.D, c.code, c.scale_dt, q_codes=qc, q_scale=qs, w=d["w"], k_cache=kc,
        k_scale=ks, k=c.k, q=d["q"], kv=d["kv"], sink=d["sink"] if g.wl.spec.sink else None,
        scale=g.wl.scale, scores=scores, ws=ws, **extra)
    return scores, idx, out


def operands(g: Gpu, prolog: bool):
    kc, ks = g.k_cache.clone(), g.k_scale.clone()
    qc, qs = g.q_codes.clone(), g.q_scale.clone()
    if prolog:
        qc.fill_(0x5A); qs.fill_(-3.0)
    return kc, ks, qc, qs


def compare(g: Gpu, prolog: bool, ws=None, schedules=("slice", "finalize", None)):
    """Both paths on copies of the operands; with the prolog the query outputs start as junk."""
    ops0 = operands(g, prolog)
    s0, i0, o0 = separate(g, prolog, *ops0)
    for sched in schedules:
        if sched is None:
            os.environ.pop("DSA_DIA_SCHEDULE", None)
        else:
            os.environ["DSA_DIA_SCHEDULE"] = sched
        try:
            ops1 = operands(g, prolog)
            s1, i1, o1 = one_call(g, prolog, *ops1, ws=ws)
            torch.cuda.synchronize()
        finally:
            os.environ.pop("DSA_DIA_SCHEDULE", None)
        what = f"schedule {sched or 'auto'}"
        assert torch.equal(i0, i1), f"{what}: selection differs from the separate calls"
        assert torch.equal(visible(g, s0), visible(g, s1)), f"{what}: scores differ from the separate calls"
        assert torch.equal(o0, o1), f"{what}: attention output differs from the separate calls"
        if prolog:
            for n, a, b in zip(("k_cache", "k_scale", "q_codes", "q_scale"), ops0, ops1):
                assert torch.equal(a, b), f"{what}: {n} differs from the separate calls"
    log(f"  {g.wl.spec.name}: prolog={prolog} T={g.wl.T}: idx, scores, out bit-identical to the separate "
        f"calls ({', '.join(x or 'auto' for x in schedules)})")
    return i1


CASES = [("ragged_i8", False), ("short_rows", False), ("no_sink", False), ("many_seqs", False),
         ("k32", False), ("final_80", False), ("fp8_prolog", True), ("i8_prolog_interleaved", True),
         ("many_tokens", False)]


@pytest.mark.parametrize("name,prolog", CASES)
def test_one_call_equals_separate_calls(name, prolog):
    spec = EXTRA.get(name) or SMALL[name]
    g = Gpu(make(spec))
    log(f"case {name}: T={g.wl.T} B={g.wl.B} k={spec.k} Hq={spec.Hq} prolog={prolog}")
    compare(g, prolog)


def test_all_equal_scores_take_the_lowest_positions():
    # zero head weights: every score is 0, every key of a row is a candidate (the lists
    # overflow and the row is re-read) and the selection is the k lowest positions
    g = Gpu(make(SMALL["ragged_i8"]))
    g.d["w"].zero_()
    idx = compare(g, False).cpu().numpy()
    k = g.cfg.k
    for t, p in enumerate(g.wl.q_pos):
        keff = min(k, int(p) + 1)
        assert np.array_equal(idx[t, :keff], np.arange(keff)) and np.all(idx[t, keff:] == -1), t


@pytest.mark.parametrize("n", [1, 2, 4])
def test_decode_workloads(n):
    g = Gpu(workloads.named(n))
    log(f"workload {n}: T={g.wl.T} B={g.wl.B}")
    compare(g, prolog=g.wl.spec.full_prolog)
    if n == 1:
        compare(g, prolog=True)


def test_workspace_shared_across_shapes():
    big, small = Gpu(workloads.named(1)), Gpu(make(SMALL["ragged_i8"]))
    c = big.cfg
    ws = torch.zeros(dsa.dsa_indexer_attention_workspace_size(big.wl.T, big.batch.max_kv_len, c.k, 128),
                     dtype=torch.uint8, device="cuda")
    for g in (big, small, big, small):
        compare(g, False, ws=ws)
        torch.cuda.synchronize()
        check_zeroed_workspace(ws, big.wl.T)
        # the second-digit histograms of the slice schedule follow the first-digit ones
        first = (big.wl.T * 4 * 2048 * 4 + 255) // 256 * 256
        h2 = ws[first:first + big.wl.T * 2048 * 4]
        assert int(torch.count_nonzero(h2).item()) == 0, "second-digit histograms not left zero"


def test_ties_at_the_kth_key_without_overflow():
    # every key row of each sequence repeated in runs of 8 (same codes and scale): each score
    # appears 8 times, so the k-th largest is one of 8 equal keys and only some of them are kept
    # (the lowest positions); the candidate lists stay within the first trip, so the slice
    # schedule ranks the tied keys in its short list
    g = Gpu(make(SMALL["ragged_i8"]))
    for b in range(g.wl.B):
        r0 = int(g.wl.kv_start[b])
        n = int(g.wl.q_pos[g.wl.q_start[b + 1] - 1]) + 1
        src = r0 + (torch.arange(n, device="cuda") // 8) * 8
        g.k_cache[r0:r0 + n] = g.k_cache[src]
        g.k_scale[r0:r0 + n] = g.k_scale[src]
    idx = compare(g, False).cpu().numpy()
    sc = g.scores().cpu().numpy()
    k, ties = g.cfg.k, 0
    for t in range(g.wl.T):
        p = int(g.wl.q_pos[t])
        if p + 1 <= k:
            continue
        row = sc[t, :p + 1]
        kth = np.sort(row)[::-1][k - 1]
        kept = np.count_nonzero(row[idx[t]] == kth)
        ties += int(kept < np.count_nonzero(row == kth))
    assert ties > 0, "no row had a partly kept tie at its k-th score"


def test_crowded_threshold_digit():
    # Every tenth key row of each sequence is a copy of one row with its scale raised 64x, and the
    # head weights are made non-negative, so the copies hold every sequence's largest score.  The
    # 40000-key sequence then has ~410 copies per 4096-score chunk, all in the threshold digit:
    # more than the first trip reads per chunk at this cache length (256), within the chunk's
    # slots (512), so both the finalize and the slice schedule take their second trip; its
    # selection is the k lowest copy positions.  Every row is also checked against the oracle's
    # top-k of the same scores.
    import oracle
    g = Gpu(make(Spec("crowded_digit", 7013, [40000, 20000, 6000], [1, 1, 1], k=2048, Hq=128)))
    g.d["w"].abs_()
    for b in range(g.wl.B):
        r0 = int(g.wl.kv_start[b])
        n = int(g.wl.q_pos[g.wl.q_start[b + 1] - 1]) + 1
        dst = r0 + torch.arange(3, n, 10, device="cuda")
        g.k_cache[dst] = g.k_cache[r0 + 3].clone()
        g.k_scale[dst] = g.k_scale[r0 + 3].clone() * 64
    idx = compare(g, False).cpu().numpy()
    sc = g.scores().cpu().numpy()
    k = g.cfg.k
    assert np.array_equal(idx[0], 3 + 10 * np.arange(k)), "40000-key row: not the k lowest copies"
    rows = [sc[t, :int(g.wl.q_pos[t]) + 1].astype(np.float64) for t in range(g.wl.T)]
    assert np.array_equal(idx, oracle.topk_select(rows, k))
