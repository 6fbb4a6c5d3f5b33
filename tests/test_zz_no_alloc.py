"""The attention entry point that allocates nothing (split partials in the library's fixed per-GPU
scratch) against the workspace entry point: same results, on two calls in a row with the second
one smaller, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads
from workloads import Spec, make
from sparse_attention_14_amd import dsa

pytestmark = pytest.mark.gpu


def _case(seed, lens, Hq, pad, rng):
    sp = Spec(f"noalloc_{seed}", seed, lens, [1] * len(lens), H=8, D=64, k=2048, Hq=Hq)
    wl = make(sp)
    idx = torch.from_numpy(workloads.random_topk_idx(rng, wl.q_pos, 2048, pad_frac=pad)).cuda()
    d = workloads.device_arrays(wl)
    batch = dsa.make_batch(wl.q_start, wl.q_seq, wl.q_pos, wl.kv_start)
    return wl, d, batch, idx


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_matches_workspace_entry_on_two_calls():
    rng = np.random.default_rng(4242)
    # first call: 8 tokens x 128 heads (split partials in the scratch); second: 3 tokens x 16 heads
    cases = [_case(7501, list(rng.integers(3000, 9000, size=8)), 128, 0.1, rng),
             _case(7502, list(rng.integers(2500, 5000, size=3)), 16, 0.3, rng)]
    outs = []
    for wl, d, batch, idx in cases:
        assert dsa.dsa_sparse_attn_workspace_size(wl.T, wl.spec.Hq, 2048) > 0
        out = torch.empty((wl.T, wl.spec.Hq, 512), dtype=torch.bfloat16, device="cuda")
        dsa.dsa_sparse_attn_decode_noalloc(batch, d["q"], d["kv"], idx, d["sink"], wl.scale, out=out)
        outs.append(out)
    torch.cuda.synchronize()
    for (wl, d, batch, idx), out in zip(cases, outs):
        ref = dsa.dsa_sparse_attn_decode(batch, d["q"], d["kv"], idx, d["sink"], wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_noalloc_rejects_partials_beyond_the_scratch():
    """63 tokens at 128 heads and k = 2048 split into partials of about 16.6 MB, beyond the 12 MiB
    scratch: the call must fail before launching anything."""
    T = 63
    need = dsa.dsa_sparse_attn_workspace_size(T, 128, 2048)
    assert need > 12 << 20
    b = dsa.make_batch(np.arange(T + 1), np.arange(T), np.full(T, 4999), np.arange(T) * 5000)
    q = torch.zeros((T, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((T * 5000, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, 2048), dtype=torch.int32, device="cuda")
    out = torch.full((T, 128, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        dsa.dsa_sparse_attn_decode_noalloc(b, q, kv, idx, None, 0.04, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote its output"
