"""Why the fp8 indexer contracts on the bf16 matrix core ([PRO] "NPU DeepSeek-V3.2-Exp PyPTO
融合算子开发优化实践", Indexer Prolog, quantization strategy: fp8 query and fp8 key cache).

e4m3 codes of the long fp8 workload's recipe (64 heads x 128 dims, RoPE + Hadamard + per-row
quantization by the oracle, eight sequences of 4096 rows instead of 131072) are contracted on the
GPU three ways -- widened to bf16 on v_mfma_f32_32x32x16_bf16 (the indexer's path), and on the two
fp8 matrix-core instructions -- and compared with the exact float64 dot products (every product of
two e4m3 values and every sum of 128 of them is exact in float64).

The budget: the top-k may differ from the oracle only at scores within 1e-5 of the k-th score, and
a score sums 64 weighted head dots, so a dot may carry at most 1e-6 of its row's largest |dot|.
The bf16 path must meet it; the fp8 instructions, whose internal adder is narrower, are recorded
and must exceed it (if they ever meet it, the indexer could contract on them instead).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import e4m3_decode
from sparse_attention_14_amd import dsa
from gpu_common import log

BUDGET = 1e-6


@pytest.mark.gpu
def test_fp8_indexer_contraction_choice():
    wl = workloads.make(workloads.NAMED[4], lens=[4096] * 8)
    q = oracle.step.quantize_workload(wl)
    A = q["q_codes"].reshape(-1, 128).view(np.uint8)            # 8 tokens x 64 heads
    B = q["k_codes"][:8192].view(np.uint8)
    exact = e4m3_decode(A) @ e4m3_decode(B).T
    rowmax = np.maximum(np.abs(exact).max(axis=1, keepdims=True), 1e-300)
    ga, gb = torch.from_numpy(A.copy()).cuda(), torch.from_numpy(B.copy()).cuda()
    rel = {}
    for path in ("bf16", "fp8_k64", "fp8_k16"):
        c = dsa.dsa_e4m3_dots(ga, gb, path).cpu().numpy().astype(np.float64)
        rel[path] = float((np.abs(c - exact) / rowmax).max())
        log(f"  {path}: max |dot - exact| / max_row |dot| = {rel[path]:.3e}")
    assert rel["bf16"] <= BUDGET, "the indexer's bf16 contraction exceeds the score budget"
    for path in ("fp8_k64", "fp8_k16"):
        assert rel[path] > BUDGET, f"{path} now meets the budget: the fp8 indexer could use it"
