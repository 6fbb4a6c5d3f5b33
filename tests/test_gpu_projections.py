"""GPU parity of dsa_indexer_projections (the Indexer Prolog's upstream linears) against the
oracle, then the prolog on the GPU's projections against the oracle prolog on the same values.

Bars: the W8A8 query dequant is an exact int32 contraction followed by three fp32 roundings
(|delta| <= 4 * 2^-24 * |ref|); the key linear's fp32 sums (at most ~130 terms deep per chain)
stay within 1e-5 * sum|x w| of the exact sums, which bounds the LayerNorm output; the FP16 head
weights may differ by one FP16 unit where the fp32 value rounds the other way.  The prolog on the
same fp32 inputs is bit-exact (codes and scales).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import bf16_decode
from sparse_attention_14_amd import dsa

from gpu_common import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(seed, T, R, H, D, hidden):
    rng = np.random.default_rng(seed)
    qa = rng.integers(-127, 128, (T, R)).astype(np.int8)
    qa_s = (rng.random(T) * 0.02 + 1e-3).astype(np.float16)
    wqb = rng.integers(-127, 128, (H * D, R)).astype(np.int8)
    wqb_s = (rng.random(H * D) * 0.002 + 1e-4).astype(np.float16)
    x = workloads.bf16_bits(rng.standard_normal((T, hidden)).astype(np.float32))
    wk = workloads.bf16_bits((rng.standard_normal((D, hidden)) / np.sqrt(hidden)).astype(np.float32))
    wp = workloads.bf16_bits((rng.standard_normal((H, hidden)) / np.sqrt(hidden)).astype(np.float32))
    g = rng.standard_normal(D).astype(np.float32)
    b = rng.standard_normal(D).astype(np.float32)
    return dict(qa=qa, qa_s=qa_s, wqb=wqb, wqb_s=wqb_s, x=x, wk=wk, wp=wp, g=g, b=b,
                eps=1e-6, wscale=float(H) ** -0.5)


def _gpu(c):
    dev = "cuda"
    bf = lambda a: torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    return dsa.dsa_indexer_projections(
        torch.from_numpy(c["qa"]).to(dev), torch.from_numpy(c["qa_s"]).to(dev),
        torch.from_numpy(c["wqb"]).to(dev), torch.from_numpy(c["wqb_s"]).to(dev),
        bf(c["x"]), bf(c["wk"]), torch.from_numpy(c["g"]).to(dev), torch.from_numpy(c["b"]).to(dev),
        c["eps"], bf(c["wp"]), c["wscale"])


def _check(c, q_pre, k_pre, weight):
    x, wk, wp = bf16_decode(c["x"]), bf16_decode(c["wk"]), bf16_decode(c["wp"])
    ref_q, ref_k, ref_w = oracle.indexer_projections(
        c["qa"], c["qa_s"].astype(np.float64), c["wqb"], c["wqb_s"].astype(np.float64), x, wk,
        c["g"], c["b"], c["eps"], wp, c["wscale"])
    gq = q_pre.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gq - ref_q) <= 4 * 2.0 ** -24 * np.abs(ref_q)), "W8A8 dequant"
    # key: the fp32 sums' error bound carried through the LayerNorm (the value, the mean and
    # the standard deviation each move by at most ev, i.e. (2 + |z|) ev / sigma in units of
    # gamma) plus the LayerNorm's own fp32 roundings
    lin = oracle.linear(x, wk)
    ev = 1e-5 * (np.abs(x) @ np.abs(wk).T).max(axis=1, keepdims=True)
    sigma = lin.std(axis=1, keepdims=True)
    z = (ref_k - c["b"]) / np.where(c["g"] == 0, 1, c["g"])
    tol = (2 + np.abs(z)) * ev / sigma * np.abs(c["g"]) + 1e-5 * (np.abs(c["g"]) * np.abs(z) + np.abs(c["b"])) + 1e-6
    gk = k_pre.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gk - ref_k) <= tol), f"key LayerNorm, max excess {np.max(np.abs(gk - ref_k) - tol)}"
    gw = weight.float().cpu().numpy().astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref_w), 2.0 ** -14))) - 10)
    assert np.all(np.abs(gw - ref_w) <= ulp), "fp16 head weights"
    return gq, gk


@pytest.mark.parametrize("shape", [(3, 256, 8, 64, 1024), (8, 1536, 64, 128, 7168),
                                   (1, 256, 64, 128, 512)])
def test_projections_match_oracle(shape):
    T, R, H, D, hidden = shape
    log(f"case projections T={T} R={R} H={H} D={D} hidden={hidden}")
    c = _case(9100 + T, T, R, H, D, hidden)
    q_pre, k_pre, weight = _gpu(c)
    torch.cuda.synchronize()
    _check(c, q_pre, k_pre, weight)


def test_prolog_on_gpu_projections_is_bit_exact():
    """Projections -> RoPE -> Hadamard -> e4m3 quant, the prolog fed the GPU's fp32 projections;
    the oracle prolog on the same values gives the same codes and scales."""
    T, R, H, D, hidden = 8, 1536, 64, 128, 7168
    c = _case(9200, T, R, H, D, hidden)
    q_pre, k_pre, weight = _gpu(c)
    gq, gk = _check(c, q_pre, k_pre, weight)
    pos = np.arange(1000, 1000 + T)
    cos, sin = workloads.rotary_tables(pos, 64)
    dev = "cuda"
    qc = torch.empty((T, H, D), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, H), dtype=torch.float16, device=dev)
    kc = torch.empty((T, D), dtype=torch.uint8, device=dev)
    ks = torch.empty((T,), dtype=torch.float16, device=dev)
    cos_t, sin_t = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    dsa.dsa_indexer_prolog(H, D, "e4m3", "f16", q_in=q_pre.view(T, H, D), q_cos=cos_t, q_sin=sin_t,
                           q_codes=qc, q_scale=qs, k_in=k_pre, k_cos=cos_t, k_sin=sin_t,
                           k_slot=torch.arange(T, device=dev), k_cache=kc, k_scale=ks,
                           rope_dim=64, rope_offset=64, hadamard=True)
    ref = oracle.indexer_prolog(gq.astype(np.float32).reshape(T, H, D), gk.astype(np.float32),
                                cos, sin, cos, sin, 64, 64, False, True, "e4m3", "f16")
    assert np.array_equal(qc.cpu().numpy(), ref["q_codes"])
    assert np.array_equal(qs.float().cpu().numpy().astype(np.float64), ref["q_scale"])
    assert np.array_equal(kc.cpu().numpy(), ref["k_codes"])
    assert np.array_equal(ks.float().cpu().numpy().astype(np.float64), ref["k_scale"])
