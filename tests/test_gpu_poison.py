"""Race-detection debug mode: DSA_DEBUG_POISON=1 makes every kernel fill its LDS with all-one
bytes before use and the library fill its written-before-read workspace regions the same way
(NaN as fp32/bf16, -1 as int, every bit set in a bitmap).  A read of LDS or workspace data before
the kernel's own write then changes the results.  Each case runs the indexer + top-k (fused and
separate), the attention, the fused prolog entry and the one-call path (both schedules) three
times -- normal, poisoned, normal -- and requires bit-identical outputs (determinism and no
read-before-write).  Selections are range-checked on the host before the attention consumes them.
"""
import os

import numpy as np
import pytest
import torch

import workloads
from workloads import make
from sparse_attention_14_amd import dsa

from gpu_common import Gpu, log
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def valid_idx(idx: torch.Tensor, q_pos: np.ndarray, k: int) -> None:
    g = idx.cpu().numpy()
    for t in range(g.shape[0]):
        keff = min(k, int(q_pos[t]) + 1)
        assert np.all(g[t, keff:] == -1) and g[t, :keff].min() >= 0 and g[t, :keff].max() <= q_pos[t], \
            f"token {t}: selection out of range"


def run_once(wl):
    g = Gpu(wl)
    T, L, k = wl.T, g.batch.max_kv_len, g.cfg.k
    ws = torch.zeros(max(1, dsa.dsa_topk_workspace_size(T, L, k)), dtype=torch.uint8, device="cuda")
    sc, idx = g.indexer_topk(ws)
    torch.cuda.synchronize()
    valid_idx(idx, wl.q_pos, k)
    out = g.sfa(idx)
    sc2 = g.scores()
    idx2 = g.topk(sc2)
    torch.cuda.synchronize()
    valid_idx(idx2, wl.q_pos, k)
    # the fused prolog entry on fresh copies, both schedules where the in-kernel form is legal
    c, d = g.cfg, g.d
    fused = []
    for sched in ("fused", "separate"):
        os.environ["DSA_PROLOG_SCHEDULE"] = sched
        try:
            kc, ks = g.k_cache.clone(), g.k_scale.clone()
            qc, qs = torch.zeros_like(g.q_codes), torch.zeros_like(g.q_scale)
            idx3 = dsa.dsa_indexer_prolog_topk(
                g.batch, c.H, c.D, c.code, c.scale_dt, q_in=d["idx_q_in"],
                k_in=d["idx_k_in"][d["new_rows"]].contiguous(), w=d["w"], q_codes=qc, q_scale=qs,
                k_cache=kc, k_scale=ks, k=k, q_cos=d["q_cos"], q_sin=d["q_sin"], rope_dim=c.rope_dim,
                rope_offset=c.rope_offset, rope_interleaved=c.rope_interleaved, hadamard=c.hadamard,
                ws=torch.zeros_like(ws))
        finally:
            os.environ.pop("DSA_PROLOG_SCHEDULE", None)
        torch.cuda.synchronize()
        fused.append((qc, qs, idx3))
    # the one-call path in both schedules
    dia = []
    for sched in ("slice", "finalize"):
        os.environ["DSA_DIA_SCHEDULE"] = sched
        try:
            i4, o4 = dsa.dsa_indexer_attention(
                g.batch, c.H, c.D, c.code, c.scale_dt, q_codes=g.q_codes, q_scale=g.q_scale, w=d["w"],
                k_cache=g.k_cache, k_scale=g.k_scale, k=k, q=d["q"], kv=d["kv"],
                sink=d["sink"] if g.wl.spec.sink else None, scale=g.wl.scale)
        finally:
            os.environ.pop("DSA_DIA_SCHEDULE", None)
        torch.cuda.synchronize()
        valid_idx(i4, wl.q_pos, k)
        dia += [i4, o4]
    vis = torch.arange(sc.shape[1], device="cuda")[None, :] <= g.d["q_pos"][:, None].long()
    return {**{f"dia_{i}": v for i, v in enumerate(dia)},"q_codes": g.q_codes, "q_scale": g.q_scale, "scores": sc[vis], "idx": idx, "out": out,
            "scores_sep": sc2[vis], "idx_sep": idx2,
            **{f"{n}_{i}": v for i, f in enumerate(fused) for n, v in zip(("qc", "qs", "idx_fused"), f)}}


def same(a: dict, b: dict, what: str) -> None:
    for n in a:
        assert torch.equal(a[n], b[n]), f"{what}: {n} differs"


@pytest.mark.parametrize("case", ["ragged_i8", "short_rows", "fp8_prolog", "many_tokens", "no_sink",
                                  "many_seqs", "named1"])
def test_poisoned_runs_are_bit_identical(case):
    wl = workloads.named(1) if case == "named1" else make(SMALL[case])
    log(f"case {case}: T={wl.T} B={wl.B}")
    os.environ.pop("DSA_DEBUG_POISON", None)
    ref = run_once(wl)
    os.environ["DSA_DEBUG_POISON"] = "1"
    try:
        pois = run_once(wl)
    finally:
        os.environ.pop("DSA_DEBUG_POISON", None)
    again = run_once(wl)
    same(ref, again, "second normal run")
    same(ref, pois, "poisoned run")
    assert torch.equal(ref["dia_0"], ref["idx"]) and torch.equal(ref["dia_2"], ref["idx"])
    assert torch.equal(ref["dia_1"], ref["out"]) and torch.equal(ref["dia_3"], ref["out"])
    log(f"  {len(ref)} outputs bit-identical across normal, poisoned, normal")
