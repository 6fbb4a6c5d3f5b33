"""The fused indexer half of a decode step (dsa_indexer_prolog_topk: the prolog inside the indexer
kernel) against the separate calls and the oracle.

[DIA] "Deepseek Indexer Attention" (jsqmd.com/news/787325): the indexer prolog, the Lightning
Indexer and its TopK run in that order; [PRO] Indexer Prolog: the query and the new key are
quantized per token-head after Hadamard(RoPE(.)).

Each case first runs the separate prolog over every cache row (codes checked against the oracle),
then overwrites the rows of the batch's new keys and the query outputs with junk, and runs the fused
call in each of its schedules (prolog inside the indexer kernel, prolog as its own launch; forced
through DSA_PROLOG_SCHEDULE where the in-kernel form is legal): it must restore exactly the same
query codes and scales, the same key cache (every row), the same scores on every visible column and
the same selection as dsa_indexer_topk on the separate prolog's operands.
"""
import os
import numpy as np
import pytest
import torch

import workloads
from workloads import make
from sparse_attention_14_amd import dsa

from gpu_common import Gpu, check_prolog, log, oracle_quant
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fused(g: Gpu, kc, ks, qc, qs, scores, ws):
    c, d = g.cfg, g.d
    k_new = d["idx_k_in"][d["new_rows"]].contiguous()
    return dsa.dsa_indexer_prolog_topk(
        g.batch, c.H, c.D, c.code, c.scale_dt, q_in=d["idx_q_in"], k_in=k_new, w=d["w"], q_codes=qc,
        q_scale=qs, k_cache=kc, k_scale=ks, k=c.k, q_cos=d["q_cos"], q_sin=d["q_sin"],
        rope_dim=c.rope_dim, rope_offset=c.rope_offset, rope_interleaved=c.rope_interleaved,
        hadamard=c.hadamard, scores=scores, ws=ws)


def run_fused_vs_separate(wl, with_oracle: bool, schedules=("fused", "separate", None)):
    for sched in schedules:
        if sched is None:
            os.environ.pop("DSA_PROLOG_SCHEDULE", None)
        else:
            os.environ["DSA_PROLOG_SCHEDULE"] = sched
        try:
            run_one(wl, with_oracle and sched is None, sched)
        finally:
            os.environ.pop("DSA_PROLOG_SCHEDULE", None)


def run_one(wl, with_oracle: bool, sched):
    log(f"case {wl.spec.name} (schedule {sched or 'auto'}): T={wl.T} B={wl.B} N={wl.N} code={wl.spec.code} "
        f"max_q_per_seq={int(np.max(np.diff(wl.q_start)))} full_prolog={wl.spec.full_prolog}")
    g = Gpu(wl)
    if with_oracle:
        check_prolog(g, oracle_quant(wl))
    T, L = wl.T, g.batch.max_kv_len
    ws = torch.zeros(max(1, dsa.dsa_topk_workspace_size(T, L, g.cfg.k)), dtype=torch.uint8, device="cuda")
    sc_ref, idx_ref = g.indexer_topk(ws)
    new = g.d["new_rows"]
    kc, ks = g.k_cache.clone(), g.k_scale.clone()
    kc[new] = 0x38                       # junk codes (e4m3 1.0 / int8 56) and scales on the new rows
    ks[new] = 3.0
    qc = torch.full_like(g.q_codes, 0x11)
    qs = torch.full_like(g.q_scale, 7.0)
    sc = torch.full_like(sc_ref, float("nan"))
    ws2 = torch.zeros_like(ws)
    idx = fused(g, kc, ks, qc, qs, sc, ws2)
    idx_again = fused(g, kc, ks, qc, qs, sc, ws2)   # the workspace is left zeroed: a second call matches
    torch.cuda.synchronize()
    log("  fused call done")
    assert torch.equal(qc, g.q_codes), "query codes"
    assert torch.equal(qs, g.q_scale), "query scales"
    assert torch.equal(kc, g.k_cache), "key cache (new rows restored, others untouched)"
    assert torch.equal(ks, g.k_scale), "key scales"
    cols = torch.arange(sc.shape[1], device="cuda")[None, :]
    vis = cols <= g.d["q_pos"][:, None].long()
    assert torch.equal(sc[vis], sc_ref[vis]), "scores on the visible columns"
    assert torch.equal(idx, idx_ref), "selection"
    assert torch.equal(idx_again, idx_ref), "selection on workspace reuse"
    log(f"  fused == separate: codes, cache, {int(vis.sum())} scores, selection")


FUSABLE_SMALL = ["short_rows", "fp8_prolog", "i8_prolog_interleaved", "no_sink", "many_seqs"]


@pytest.mark.parametrize("name", FUSABLE_SMALL)
def test_fused_prolog_small(name):
    run_fused_vs_separate(make(SMALL[name]), with_oracle=True)


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 4])
def test_fused_prolog_named(cfg_id):
    run_fused_vs_separate(workloads.named(cfg_id), with_oracle=cfg_id in (0, 1))


def test_fused_prolog_round_scale_f32_scales():
    """Power-of-two scales (round_scale) and fp32 scales through the fused path, against the
    separate prolog with the same settings."""
    wl = make(SMALL["fp8_prolog"])
    g = Gpu(wl)
    c, d = g.cfg, g.d
    qc_ref = torch.empty_like(g.q_codes)
    qs_ref = torch.empty(g.q_scale.shape, dtype=torch.float32, device="cuda")
    kc_ref = torch.empty_like(g.k_cache)
    ks_ref = torch.empty(g.k_scale.shape, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_prolog(c.H, c.D, c.code, "f32", q_in=d["idx_q_in"], q_cos=d["q_cos"], q_sin=d["q_sin"],
                           q_codes=qc_ref, q_scale=qs_ref, k_in=d["idx_k_in"], k_cos=d["k_cos"],
                           k_sin=d["k_sin"], k_slot=d["all_rows"], k_cache=kc_ref, k_scale=ks_ref,
                           rope_dim=c.rope_dim, rope_offset=c.rope_offset, hadamard=True, round_scale=True)
    ws = torch.zeros(dsa.dsa_topk_workspace_size(wl.T, g.batch.max_kv_len, c.k), dtype=torch.uint8, device="cuda")
    idx_ref = dsa.dsa_indexer_topk(g.batch, c.H, c.D, c.code, "f32", qc_ref, qs_ref, d["w"], kc_ref, ks_ref,
                                   c.k, ws=ws)
    kc, ks = kc_ref.clone(), ks_ref.clone()
    kc[d["new_rows"]] = 0
    ks[d["new_rows"]] = 0.5
    qc, qs = torch.zeros_like(qc_ref), torch.zeros_like(qs_ref)
    idx = dsa.dsa_indexer_prolog_topk(
        g.batch, c.H, c.D, c.code, "f32", q_in=d["idx_q_in"], k_in=d["idx_k_in"][d["new_rows"]].contiguous(),
        w=d["w"], q_codes=qc, q_scale=qs, k_cache=kc, k_scale=ks, k=c.k, q_cos=d["q_cos"], q_sin=d["q_sin"],
        rope_dim=c.rope_dim, rope_offset=c.rope_offset, hadamard=True, round_scale=True,
        ws=torch.zeros_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(qc, qc_ref) and torch.equal(qs, qs_ref)
    assert torch.equal(kc, kc_ref) and torch.equal(ks, ks_ref)
    assert torch.equal(idx, idx_ref)
    s = qs_ref[qs_ref > 0]
    assert torch.all(torch.log2(s) == torch.round(torch.log2(s))), "round_scale gives powers of two"


@pytest.mark.parametrize("name", ["ragged_i8", "many_tokens"])
def test_fused_prolog_shapes_outside_the_in_kernel_form(name):
    """Groups of 3-4 fp32 query rows at D = 128 exceed the in-kernel staging, and prefill-sized
    groups take the tiled indexer: the call runs the prolog as its own launch, with the same
    results."""
    run_fused_vs_separate(make(SMALL[name]), with_oracle=True, schedules=(None,))
