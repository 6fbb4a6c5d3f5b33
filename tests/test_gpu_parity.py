"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded inputs.

Small cases span several tiles with ragged tails and hit each edge the method has (short rows
with -1 padding, exact ties, empty selections, no sink, fp8 with RoPE+Hadamard, many tokens
per sequence); the named full-size workloads run the launch configuration the benchmark uses.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Spec, make
from sparse_attention_14_amd import dsa

from gpu_common import (Gpu, check_prolog, check_scores, check_sfa, check_topk, log, oracle_quant,
                        run_e2e)

pytestmark = pytest.mark.gpu

SMALL = {
    "ragged_i8": Spec("small_ragged_i8", 7001, [5000, 777, 3001], [2, 1, 3], k=512, Hq=128),
    "short_rows": Spec("small_short_rows", 7002, [100, 3000, 256], [1, 1, 2], H=8, D=64,
                       scale_dt="f32", k=256, Hq=16),
    "fp8_prolog": Spec("small_fp8_prolog", 7003, [3000, 4500], [1, 2], code="e4m3",
                       full_prolog=True, k=512, Hq=128),
    "i8_prolog_interleaved": Spec("small_i8_prolog_il", 7004, [2000, 2100], [2, 2], full_prolog=True,
                                  rope_interleaved=True, k=300, Hq=16),
    "no_sink": Spec("small_no_sink", 7006, [2500], [1], k=2048, Hq=128, sink=False),
    "many_tokens": Spec("small_many_tokens", 7005, [4096, 4096], [128, 128], k=256, Hq=128),
    # more than 64 sequences: the kernels' per-lane batch-metadata path does not apply
    "many_seqs": Spec("small_many_seqs", 7007, [300 + 37 * i for i in range(80)], [1] * 80, H=8,
                      D=64, scale_dt="f32", k=256, Hq=16),
}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(SMALL))
def test_small_end_to_end(name):
    run_e2e(make(SMALL[name]), check_dots=True)


def test_prolog_round_scale_and_scale_dtypes(rng):
    for code in ("i8", "e4m3"):
        for sdt in ("f16", "f32"):
            sp = Spec(f"prolog_{code}_{sdt}", 7100, [700, 1300], [3, 1], code=code, scale_dt=sdt,
                      full_prolog=True, k=64, Hq=16)
            wl = make(sp)
            log(f"case prolog {code}/{sdt} round_scale")
            d = workloads.device_arrays(wl)
            ct = torch.int8 if code == "i8" else torch.uint8
            st = torch.float16 if sdt == "f16" else torch.float32
            kc = torch.empty((wl.N, 128), dtype=ct, device="cuda")
            ks = torch.empty((wl.N,), dtype=st, device="cuda")
            dsa.dsa_indexer_prolog(64, 128, code, sdt, k_in=d["idx_k_in"], k_cos=d["k_cos"],
                                   k_sin=d["k_sin"], k_slot=d["all_rows"], k_cache=kc, k_scale=ks,
                                   rope_dim=64, rope_offset=64, hadamard=True, round_scale=True)
            kin = oracle.formats.bf16_decode(wl.idx_k_in).astype(np.float32)
            c, s, _ = oracle.prolog_rows(kin, wl.k_cos, wl.k_sin, 64, 64, False, True, code, sdt,
                                         round_scale=True)
            got = kc.cpu().numpy()
            assert np.array_equal(got.astype(c.dtype), c)
            assert np.array_equal(ks.float().cpu().numpy().astype(np.float64), s)


def test_prolog_zero_rows_and_slots():
    """All-zero rows quantize to zero codes and scale 0; rows land in their slots only."""
    N, D = 64, 128
    k_in = torch.zeros((4, D), dtype=torch.float32, device="cuda")
    k_in[1] = torch.linspace(-3, 3, D, device="cuda")
    kc = torch.full((N, D), 99, dtype=torch.int8, device="cuda")
    ks = torch.full((N,), 7.0, dtype=torch.float16, device="cuda")
    slots = torch.tensor([5, 17, 40, 63], dtype=torch.int64, device="cuda")
    dsa.dsa_indexer_prolog(1, D, "i8", "f16", k_in=k_in, k_slot=slots, k_cache=kc, k_scale=ks)
    kc_h, ks_h = kc.cpu().numpy(), ks.float().cpu().numpy()
    for r, s in enumerate([5, 17, 40, 63]):
        if r == 1:
            c, st, _ = oracle.quantize_rows(k_in[1:2].cpu().numpy(), "i8", "f16")
            assert np.array_equal(kc_h[s], c[0]) and ks_h[s] == st[0]
        else:
            assert not kc_h[s].any() and ks_h[s] == 0.0
    untouched = np.setdiff1d(np.arange(N), [5, 17, 40, 63])
    assert np.all(kc_h[untouched] == 99) and np.all(ks_h[untouched] == 7.0)


def _topk_case(rng, T, L, k, kind):
    if kind == "random":
        s = rng.standard_normal((T, L)).astype(np.float32)
    elif kind == "ties":          # few distinct values: many exact ties at the threshold
        s = rng.integers(-3, 4, (T, L)).astype(np.float32)
    elif kind == "negative":      # every score below zero: the k-th key is in the lower digits
        s = (-1.0 - np.abs(rng.standard_normal((T, L)))).astype(np.float32)
    elif kind == "zeros":         # +0 and -0 only
        s = np.where(rng.random((T, L)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    elif kind == "narrow":        # narrow band: candidates overflow the chunks' slots
        s = (1000.0 + rng.random((T, L)) * 1e-3).astype(np.float32)
    else:                         # crowded: a tenth of the keys in one digit (~410 per chunk)
        s = np.where(rng.random((T, L)) < 0.1, 1.0 + 0.25 * rng.random((T, L)),
                     1e-3 * rng.random((T, L))).astype(np.float32)
    return s


@pytest.mark.parametrize("kind", ["random", "ties", "negative", "zeros", "narrow", "crowded"])
def test_topk_exact_on_identical_scores(rng, kind):
    """Same fp32 scores on both sides: the selected sets must be identical (ties -> lower
    positions), for long rows, rows shorter than k and rows of exactly k."""
    lens = [70000, 2048, 2047, 100, 40000, 2049]
    T, k = len(lens), 2048
    L = max(lens)
    s = _topk_case(rng, T, L, k, kind)
    ld = (L + 63) // 64 * 64
    sc = np.zeros((T, ld), dtype=np.float32)
    sc[:, :L] = s
    batch = dsa.make_batch(np.arange(T + 1), np.arange(T), np.array(lens) - 1, np.zeros(T))
    log(f"case topk {kind}")
    idx = dsa.dsa_topk(batch, torch.from_numpy(sc).cuda(), k).cpu().numpy()
    rows = [sc[t, :lens[t]].astype(np.float64) for t in range(T)]
    ref = oracle.topk_select(rows, k)
    assert np.array_equal(idx, ref)


@pytest.mark.parametrize("kind", ["random", "ties", "negative", "zeros", "narrow", "crowded"])
def test_row_topk_exact_on_identical_scores(rng, kind):
    """Batches of 256 or more rows take one workgroup per row (its own first-digit histogram, the
    keys at or above the threshold digit compacted in LDS in position order, or re-read from the
    scores when they do not fit).  Same fp32 scores on both sides: the selected sets must be
    identical (ties -> lower positions), for rows of one to three 65536-score segments, rows
    shorter than k and rows of exactly k."""
    T, k = 256, 2048
    lens = rng.integers(2049, 140000, size=T)
    lens[:8] = [2048, 2047, 100, 2049, 65536, 65537, 131072, 140000]
    L = int(lens.max())
    s = _topk_case(rng, T, L, k, kind)
    ld = (L + 63) // 64 * 64
    sc = np.zeros((T, ld), dtype=np.float32)
    sc[:, :L] = s
    batch = dsa.make_batch(np.arange(T + 1), np.arange(T), lens - 1, np.zeros(T))
    log(f"case row topk {kind}")
    idx = dsa.dsa_topk(batch, torch.from_numpy(sc).cuda(), k).cpu().numpy()
    rows = [sc[t, :lens[t]].astype(np.float64) for t in range(T)]
    assert np.array_equal(idx, oracle.topk_select(rows, k))


def test_indexer_topk_all_ties_take_lowest_positions():
    """Every score equal (zero head weights): every key of a row is in the threshold digit, so the
    row workgroup's ordered list holds the whole row (9000 and 2100 keys) or overflows it (70000
    keys, resolved by re-reading the row); the ties go to the lowest positions, exactly as the
    standalone top-k, and the row histograms are left zero."""
    from gpu_common import check_zeroed_workspace
    sp = Spec("all_ties", 7210, [9000, 70000, 2100], [2, 1, 1], k=2048, Hq=16)
    wl = make(sp)
    wl.w[:] = 0
    g = Gpu(wl)
    ws = torch.zeros(dsa.dsa_topk_workspace_size(wl.T, g.batch.max_kv_len, 2048), dtype=torch.uint8,
                     device="cuda")
    log("case indexer + top-k, all ties")
    _, idx = g.indexer_topk(ws)
    check_zeroed_workspace(ws, wl.T)
    got = idx.cpu().numpy()
    assert np.array_equal(got, np.tile(np.arange(2048), (wl.T, 1)))
    assert torch.equal(idx, g.topk(g.scores()))


def test_topk_all_zero_weights_select_first_positions():
    sp = Spec("ties_w0", 7200, [9000, 3000], [1, 1], k=1024, Hq=16)
    wl = make(sp)
    wl.w[:] = 0
    g = Gpu(wl)
    idx = g.topk(g.scores()).cpu().numpy()
    assert np.array_equal(idx[:, :1024], np.tile(np.arange(1024), (2, 1)))


@pytest.mark.parametrize("Hq,T,sink,pad", [(128, 3, True, 0.0), (128, 5, False, 0.3),
                                            (16, 2, True, 0.5), (128, 300, True, 0.1),
                                            (16, 40, False, 0.0)])
def test_sparse_attention_isolated(rng, Hq, T, sink, pad):
    """Random selections (with -1 holes) straight into the attention kernel."""
    lens = list(rng.integers(1500, 6000, size=T))
    sp = Spec(f"sfa_{Hq}_{T}", 7300 + T, lens, [1] * T, H=8, D=64, k=2048, Hq=Hq, sink=sink)
    wl = make(sp)
    idx = workloads.random_topk_idx(rng, wl.q_pos, 2048, pad_frac=pad)
    if T >= 3:
        idx[1, :] = -1                                   # a token with an empty selection
    log(f"case sfa Hq={Hq} T={T} sink={sink} pad={pad}")
    d = workloads.device_arrays(wl)
    batch = dsa.make_batch(wl.q_start, wl.q_seq, wl.q_pos, wl.kv_start)
    out = dsa.dsa_sparse_attn_decode(batch, d["q"], d["kv"], torch.from_numpy(idx).cuda(),
                                     d["sink"] if sink else None, wl.scale)
    ref = oracle.sparse_attention(wl.q, wl.kv, idx, wl.q_seq, wl.kv_start, wl.sink, wl.scale)
    check_sfa(out, ref)
    if T >= 3:
        assert not out[1].float().abs().sum().item()


@pytest.mark.parametrize("T,k,pad", [(256, 2048, 0.2), (300, 100, 0.0), (257, 32, 0.5), (512, 200, 0.1),
                                     (256, 64, 0.3), (256, 96, 0.0), (260, 150, 0.2), (256, 190, 0.0),
                                     (256, 250, 0.1)])
def test_sparse_attention_64_head_kernel_equals_32_head_kernel(rng, T, k, pad):
    """Batches with one split per token run the 64-head kernel (index ring in LDS, value waves that
    also gather and read a tile's V one step early); it must reproduce the 32-head kernel bit for
    bit -- the same tiles, per-head arithmetic and order -- on random selections with -1 holes,
    empty selections, every tile count from 1 to 8 (k = 32 .. 250, partial last tiles included:
    the gather schedule's start and end differ below 3 tiles, the index ring's prologue covers 5)
    and 64 tiles, and match the oracle."""
    lens = list(rng.integers(300, 5000, size=T))
    sp = Spec(f"sfa64_{T}_{k}", 7400 + T + k, lens, [1] * T, H=8, D=64, k=k, Hq=128)
    wl = make(sp)
    idx = workloads.random_topk_idx(rng, wl.q_pos, k, pad_frac=pad)
    idx[1, :] = -1                                       # an empty selection
    log(f"case sfa64 T={T} k={k} pad={pad}")
    d = workloads.device_arrays(wl)
    batch = dsa.make_batch(wl.q_start, wl.q_seq, wl.q_pos, wl.kv_start)
    it = torch.from_numpy(idx).cuda()
    out64 = dsa.dsa_sparse_attn_decode(batch, d["q"], d["kv"], it, d["sink"], wl.scale)
    os.environ["DSA_SFA_H64"] = "0"
    try:
        out32 = dsa.dsa_sparse_attn_decode(batch, d["q"], d["kv"], it, d["sink"], wl.scale)
    finally:
        os.environ.pop("DSA_SFA_H64", None)
    torch.cuda.synchronize()
    assert torch.equal(out64, out32), "64-head kernel differs from the 32-head kernel"
    sample = np.arange(0, T, 7)
    ref = oracle.sparse_attention(wl.q[sample], wl.kv, idx[sample], np.asarray(wl.q_seq)[sample], wl.kv_start,
                                  wl.sink, wl.scale)
    check_sfa(out64[torch.from_numpy(sample).cuda()], ref)


@pytest.mark.parametrize("Hq,T", [(128, 8), (16, 3), (128, 600)])
def test_sparse_attention_split_then_merge_equals_decode(rng, Hq, T):
    """The two stage entry points, run back to back, reproduce the one-call result bit for bit
    (with split partials for small T, and the direct path when one split suffices)."""
    lens = list(rng.integers(2500, 5000, size=T))
    sp = Spec(f"sfa_stages_{Hq}_{T}", 7350 + T, lens, [1] * T, H=8, D=64, k=2048, Hq=Hq)
    wl = make(sp)
    idx = torch.from_numpy(workloads.random_topk_idx(rng, wl.q_pos, 2048, pad_frac=0.1)).cuda()
    d = workloads.device_arrays(wl)
    batch = dsa.make_batch(wl.q_start, wl.q_seq, wl.q_pos, wl.kv_start)
    log(f"case sfa split+merge Hq={Hq} T={T} ws={dsa.dsa_sparse_attn_workspace_size(T, Hq, 2048)}")
    ref = dsa.dsa_sparse_attn_decode(batch, d["q"], d["kv"], idx, d["sink"], wl.scale)
    out, ws = dsa.dsa_sparse_attn_split(batch, d["q"], d["kv"], idx, d["sink"], wl.scale)
    dsa.dsa_sparse_attn_merge(batch, Hq, 2048, d["sink"], out, ws)
    assert torch.equal(out, ref)


def test_sparse_attention_strided_kv(rng):
    """kv rows with a stride larger than 576 (e.g. a wider cache row)."""
    sp = Spec("sfa_stride", 7400, [3000, 2500], [1, 1], H=8, D=64, k=1000, Hq=128)
    wl = make(sp)
    idx = workloads.random_topk_idx(rng, wl.q_pos, 1000)
    kv_wide = torch.zeros((wl.N, 640), dtype=torch.bfloat16, device="cuda")
    kv_wide[:, :576] = torch.from_numpy(wl.kv).view(torch.bfloat16).cuda()
    d = workloads.device_arrays(wl)
    batch = dsa.make_batch(wl.q_start, wl.q_seq, wl.q_pos, wl.kv_start)
    out = dsa.dsa_sparse_attn_decode(batch, d["q"], kv_wide[:, :576], torch.from_numpy(idx).cuda(),
                                     d["sink"], wl.scale)
    ref = oracle.sparse_attention(wl.q, wl.kv, idx, wl.q_seq, wl.kv_start, wl.sink, wl.scale)
    check_sfa(out, ref)


def test_empty_batch_noop():
    batch = dsa.make_batch([0], [], [], [])
    z = torch.zeros(0, device="cuda")
    assert batch.num_q == 0
    lib = dsa.lib
    b = batch.c()
    import ctypes
    assert lib.dsa_topk(ctypes.byref(b), None, 0, 2048, None, None, 0, None) == 0
    del z


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 4])
def test_named_workload_end_to_end(cfg_id):
    run_e2e(workloads.named(cfg_id), check_dots=(cfg_id == 1))


def prefill_sample(wl, n_random=40, seed=31):
    """Tokens of the prefill chunk compared with the oracle: the first and last, the two tokens
    on each side of every 512-key boundary (the indexer's key chunks), those on each side of
    every 4096-position boundary (the top-k's score chunks), and seeded random ones."""
    T = wl.T
    p0 = int(wl.q_pos[0])
    picks = {0, 1, T - 2, T - 1}
    for period in (512, 4096):
        for p in range(p0 - p0 % period, p0 + T + 1, period):
            for q in (p - 2, p - 1, p, p + 1):
                if p0 <= q < p0 + T:
                    picks.add(q - p0)
    rng = np.random.default_rng(seed)
    picks.update(int(x) for x in rng.integers(0, T, n_random))
    return np.array(sorted(picks))


def test_named_prefill_sampled_tokens():
    """Prefill chunk (4096 new tokens on a 61440-token cache): the full GPU step, compared with
    the oracle on >= 64 sampled tokens (chunk boundaries of the indexer and the top-k, first,
    last and seeded random ones)."""
    wl = workloads.named(3)
    toks = prefill_sample(wl)
    assert len(toks) >= 64
    run_e2e(wl, token_subset=toks)


def test_topk_workspace_reuse_across_calls():
    """A workspace is zero-filled once: every call must leave its histograms cleared, so a call
    on a second workload through the same workspace selects exactly what a fresh one does (fused
    and standalone paths, rows of different lengths and batch sizes)."""
    a = Gpu(make(Spec("reuse_a", 7401, [9000, 70000, 3000], [2, 1, 1], k=2048, Hq=16)))
    b = Gpu(make(Spec("reuse_b", 7402, [66000, 5000], [1, 2], k=2048, Hq=16)))
    # sized with the largest token count and the longest row of the two calls
    need = dsa.dsa_topk_workspace_size(max(a.wl.T, b.wl.T),
                                       max(a.batch.max_kv_len, b.batch.max_kv_len), 2048)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    log("case topk workspace reuse")
    _, idx_a = a.indexer_topk(ws=ws)
    _, idx_b = b.indexer_topk(ws=ws)
    _, idx_b_fresh = b.indexer_topk()
    assert torch.equal(idx_b, idx_b_fresh)
    _, idx_a2 = a.indexer_topk(ws=ws)
    assert torch.equal(idx_a2, idx_a)
    sb = b.scores()
    assert torch.equal(dsa.dsa_topk(b.batch, sb, 2048, ws=ws), idx_b_fresh)
    assert torch.equal(dsa.dsa_topk(b.batch, sb, 2048, ws=ws), idx_b_fresh)
    assert not ws[: 4 * 2048 * 4 * max(a.wl.T, b.wl.T)].any(), "histograms left non-zero"
