#!/usr/bin/env python3
"""Benchmark of the DSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 256] [--warmup 32] [--workload 1]

A step is one pass of the whole path over one batch with every input resident in HBM:
  indexer prolog (the batch's new query tokens and their key rows) -> Lightning Indexer
  scores with the top-k's first radix pass fused -> top-k -> sparse attention (+ split
  combine).
The default workload is 4 sequences x 2 query tokens (MTP1) on 64K-token caches, indexer
64 heads x 128 int8 with fp16 scales, top-k 2048, 128 attention heads over 576-wide bf16
latent rows.  Inputs are seeded synthetic data of that shape.

Cache honesty: the 256 MiB Infinity Cache (MALL) would hold one step's ~55 MB working set.
The bench therefore keeps R copies of every input and output at distinct addresses and steps
round-robin through them (R * per-step bytes >= 4x the MALL), so each step reads HBM.  The R
steps are captured in one HIP graph that is replayed; the timed region is exactly `--steps`
steps between two device synchronizations.

Kernel timing: each kernel is also launched R times back to back (rotating copies) inside a
graph bracketed by HIP events on the stream it runs on; the average per launch is reported
per kernel, and the dominant one carries the roofline entry.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # dense int8 MFMA
BF16_PEAK_TFLOPS = 2500.0       # dense bf16 MFMA
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", type=int, default=1, help="named workload id (workloads.NAMED)")
    ap.add_argument("--sets", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="copy a buffer of this many MiB 4 times first (calibrates HBM counters)")
    return ap.parse_args()


def counter_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"step_kernels_{workload}_counters.md")


def kernel_source_hash() -> str:
    """sha256 of the kernel sources: counter-derived traffic is reported only while it still
    describes the kernels being timed."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(f for f in os.listdir(os.path.join(ROOT, "sparse_attention_14_amd", "csrc"))
                    if f.endswith((".hip", ".h"))):
        with open(os.path.join(ROOT, "sparse_attention_14_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it was taken on
    the current sources (line: `traffic_bytes_per_launch <kernel> <bytes> <source sha256>`)."""
    try:
        with open(counter_file(workload)) as fh:
            for line in fh:
                f = line.strip().strip("`").split()
                if len(f) == 4 and f[0] == "traffic_bytes_per_launch" and f[1] == kernel:
                    return int(f[2]) if f[3] == kernel_source_hash() else None
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    from sparse_attention_14_amd import dsa
    from sparse_attention_14_amd.step import IndexerCfg, StepBuffers, decode_step

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = workloads.named(args.workload)
    sp = wl.spec
    cfg = IndexerCfg(H=sp.H, D=sp.D, code=sp.code, scale_dt=sp.scale_dt,
                     rope_dim=sp.rope_dim if sp.full_prolog else 0, rope_offset=sp.rope_offset,
                     rope_interleaved=sp.rope_interleaved, hadamard=sp.full_prolog, k=sp.k)
    d0 = workloads.device_arrays(wl, dev)
    batch = dsa.make_batch(wl.q_start, wl.q_seq, wl.q_pos, wl.kv_start, dev)
    T, N, H, D, Hq, k = wl.T, wl.N, sp.H, sp.D, sp.Hq, sp.k
    ct = torch.int8 if cfg.code == "i8" else torch.uint8
    st = torch.float16 if cfg.scale_dt == "f16" else torch.float32
    sbytes = 2 if cfg.scale_dt == "f16" else 4

    # the quantized indexer key cache: every row through the prolog once (set-up, untimed)
    k_cache = torch.empty((N, D), dtype=ct, device=dev)
    k_scale = torch.empty((N,), dtype=st, device=dev)
    dsa.dsa_indexer_prolog(H, D, cfg.code, cfg.scale_dt, k_in=d0["idx_k_in"], k_cos=d0["k_cos"],
                           k_sin=d0["k_sin"], k_slot=d0["all_rows"], k_cache=k_cache,
                           k_scale=k_scale, rope_dim=cfg.rope_dim, rope_offset=cfg.rope_offset,
                           rope_interleaved=cfg.rope_interleaved, hadamard=cfg.hadamard)
    new_q_in = d0["idx_q_in"]
    new_k_in = d0["idx_k_in"][d0["new_rows"]].contiguous()
    new_cos = d0["k_cos"][d0["new_rows"]].contiguous() if d0["k_cos"] is not None else None
    new_sin = d0["k_sin"][d0["new_rows"]].contiguous() if d0["k_sin"] is not None else None

    # per-step compulsory HBM bytes (strict roofline): K codes+scales scanned, new-token inputs,
    # prolog outputs, scores written and read, gathered rows, attention q/out, indices
    n_keys = int(np.sum(wl.q_pos[wl.q_start[1:] - 1] + 1))          # keys scanned per sequence
    keff = np.minimum(k, wl.q_pos + 1)
    n_sel = int(keff.sum())
    score_cols = int(np.sum(wl.q_pos + 1))
    in_b = 2 if wl.in_dtype == "bf16" else 4
    b_prolog = T * H * D * in_b + T * D * in_b + T * H * (D + sbytes) + T * (D + sbytes)
    b_indexer = n_keys * (D + sbytes) + T * H * (D + sbytes + 2) + score_cols * 4
    b_topk = score_cols * 4 + T * k * 4
    b_sfa = n_sel * 1152 + T * Hq * 576 * 2 + T * Hq * 512 * 2 + T * k * 4 + Hq * 4
    step_bytes = b_prolog + b_indexer + b_topk + b_sfa
    idx_ops = float(np.sum((wl.q_pos + 1).astype(np.float64))) * H * D * 2
    sfa_flops = float(n_sel) * Hq * (576 + 512) * 2

    R = args.sets or max(4, int(np.ceil(4 * MALL_BYTES / step_bytes)))
    R = min(R, 32)

    class Set:
        pass

    sets = []
    for r in range(R):
        s = Set()
        s.k_cache = k_cache if r == 0 else k_cache.clone()
        s.k_scale = k_scale if r == 0 else k_scale.clone()
        s.kv = d0["kv"] if r == 0 else d0["kv"].clone()
        s.q = d0["q"] if r == 0 else d0["q"].clone()
        s.w = d0["w"] if r == 0 else d0["w"].clone()
        s.q_in = new_q_in if r == 0 else new_q_in.clone()
        s.k_in = new_k_in if r == 0 else new_k_in.clone()
        s.buf = StepBuffers.alloc(batch, cfg, Hq, dev)
        sets.append(s)
    sink = d0["sink"]
    new_slots = d0["new_rows"]

    def step(s):
        return decode_step(batch, cfg, q_in=s.q_in, k_in=s.k_in, new_slots=new_slots, w=s.w,
                           k_cache=s.k_cache, k_scale=s.k_scale, q_attn=s.q, kv=s.kv, sink=sink,
                           scale=wl.scale, buf=s.buf, q_cos=d0["q_cos"], q_sin=d0["q_sin"],
                           k_cos=new_cos, k_sin=new_sin)

    def step_separate(s):
        return decode_step(batch, cfg, q_in=s.q_in, k_in=s.k_in, new_slots=new_slots, w=s.w,
                           k_cache=s.k_cache, k_scale=s.k_scale, q_attn=s.q, kv=s.kv, sink=sink,
                           scale=wl.scale, buf=s.buf, q_cos=d0["q_cos"], q_sin=d0["q_sin"],
                           k_cos=new_cos, k_sin=new_sin, fused=False)

    # stage launchers (for per-kernel timing)
    def st_prolog(s):
        dsa.dsa_indexer_prolog(H, D, cfg.code, cfg.scale_dt, q_in=s.q_in, q_cos=d0["q_cos"],
                               q_sin=d0["q_sin"], q_codes=s.buf.q_codes, q_scale=s.buf.q_scale,
                               k_in=s.k_in, k_cos=new_cos, k_sin=new_sin, k_slot=new_slots,
                               k_cache=s.k_cache, k_scale=s.k_scale, rope_dim=cfg.rope_dim,
                               rope_offset=cfg.rope_offset, rope_interleaved=cfg.rope_interleaved,
                               hadamard=cfg.hadamard)

    def st_prolog_indexer_topk(s):
        dsa.dsa_indexer_prolog_topk(batch, H, D, cfg.code, cfg.scale_dt, q_in=s.q_in, k_in=s.k_in,
                                    w=s.w, q_codes=s.buf.q_codes, q_scale=s.buf.q_scale,
                                    k_cache=s.k_cache, k_scale=s.k_scale, k=k, q_cos=d0["q_cos"],
                                    q_sin=d0["q_sin"], rope_dim=cfg.rope_dim,
                                    rope_offset=cfg.rope_offset,
                                    rope_interleaved=cfg.rope_interleaved, hadamard=cfg.hadamard,
                                    scores=s.buf.scores, idx=s.buf.idx, ws=s.buf.ws_topk)

    def st_indexer(s):
        dsa.dsa_indexer_scores(batch, H, D, cfg.code, cfg.scale_dt, s.buf.q_codes, s.buf.q_scale,
                               s.w, s.k_cache, s.k_scale, scores=s.buf.scores)

    def st_indexer_topk(s):
        dsa.dsa_indexer_topk(batch, H, D, cfg.code, cfg.scale_dt, s.buf.q_codes, s.buf.q_scale,
                             s.w, s.k_cache, s.k_scale, k, scores=s.buf.scores, idx=s.buf.idx,
                             ws=s.buf.ws_topk)

    def st_indexer_attention(s):
        dsa.dsa_indexer_attention(batch, H, D, cfg.code, cfg.scale_dt, q_codes=s.buf.q_codes,
                                  q_scale=s.buf.q_scale, w=s.w, k_cache=s.k_cache,
                                  k_scale=s.k_scale, k=k, q=s.q, kv=s.kv, sink=sink,
                                  scale=wl.scale, scores=s.buf.scores, idx=s.buf.idx,
                                  out=s.buf.out, ws=s.buf.ws_dia)

    def st_sfa(s):
        dsa.dsa_sparse_attn_decode(batch, s.q, s.kv, s.buf.idx, sink, wl.scale, out=s.buf.out,
                                   ws=s.buf.ws_sfa)

    def st_sfa_split(s):
        dsa.dsa_sparse_attn_split(batch, s.q, s.kv, s.buf.idx, sink, wl.scale, out=s.buf.out,
                                  ws=s.buf.ws_sfa)

    def st_sfa_merge(s):
        dsa.dsa_sparse_attn_merge(batch, Hq, k, sink, s.buf.out, s.buf.ws_sfa)

    if args.copy_probe_mib:
        # a plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ref = step(sets[0]).clone()
        for s in sets[1:]:
            step(s)
    torch.cuda.synchronize()
    for s in sets:
        assert torch.equal(s.buf.out, ref), "rotating copies disagree"

    def capture(fn_per_set):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in sets:
                fn_per_set(s)
        return g

    def replay(g, n):
        # CUDAGraph.replay() launches on torch's current stream: make it the timed stream
        with torch.cuda.stream(stream):
            for _ in range(n):
                g.replay()

    g_step = capture(step)
    # replay check: several replays with eager work and syncs between, all equal to eager
    for rep in range(3):
        for s in sets:
            s.buf.out.zero_()
        torch.cuda.synchronize()
        replay(g_step, 1)
        torch.cuda.synchronize()
        for s in sets:
            assert torch.equal(s.buf.out, ref), f"graph replay {rep} differs from eager"

    # warm-up and timed region: whole replays of the R-step graph, at least 8 of them, each
    # bracketed by its own pair of events (per-replay samples for the median and spread); the
    # value is the mean over every timed step
    reps_w = max(1, int(np.ceil(args.warmup / R)))
    reps = max(8, int(np.ceil(args.steps / R)))
    K = reps * R
    replay(g_step, reps_w)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(reps):
        replay(g_step, 1)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us_step = evs[0].elapsed_time(evs[-1]) * 1000.0 / K
    per_rep = np.array([evs[i].elapsed_time(evs[i + 1]) * 1000.0 / R for i in range(reps)])

    # warm: the same step R times on one input set (everything it touches may sit in the MALL)
    g_warm = capture(lambda s: step(sets[0]))
    replay(g_warm, 2)
    torch.cuda.synchronize()
    a_w, b_w = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_w.record(stream)
    replay(g_warm, 4)
    b_w.record(stream)
    torch.cuda.synchronize()
    warm_us = a_w.elapsed_time(b_w) * 1000.0 / (4 * R)

    # paged caches (Page Attention blocks of 128 rows, shuffled): copies of every set's K and
    # KV caches, for the paged calls' stage timing; they must select and attend exactly as the
    # flat calls do
    lay = workloads.block_layout(wl, 128, seed=1)
    rm = torch.as_tensor(lay.row_map, device=dev)
    rows_p = lay.num_blocks * 128
    paging = dsa.Paging(torch.as_tensor(lay.table, device=dev), 128, lay.num_blocks)

    def paged_copy(t):
        out = torch.zeros((rows_p,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
        out[rm] = t
        return out

    for s in sets:
        s.k_cache_p, s.k_scale_p, s.kv_p = paged_copy(s.k_cache), paged_copy(s.k_scale), paged_copy(s.kv)

    def st_indexer_topk_paged(s):
        dsa.dsa_indexer_topk_paged(batch, paging, H, D, cfg.code, cfg.scale_dt, s.buf.q_codes,
                                   s.buf.q_scale, s.w, s.k_cache_p, s.k_scale_p, k,
                                   scores=s.buf.scores, idx=s.buf.idx, ws=s.buf.ws_topk)

    def st_sfa_paged(s):
        dsa.dsa_sparse_attn_decode_paged(batch, paging, s.q, s.kv_p, s.buf.idx, sink, wl.scale,
                                         out=s.buf.out, ws=s.buf.ws_sfa)

    with torch.cuda.stream(stream):
        st_indexer_topk(sets[0])
        idx_flat = sets[0].buf.idx.clone()
        st_sfa(sets[0])
        out_flat = sets[0].buf.out.clone()
        st_indexer_topk_paged(sets[0])
        st_sfa_paged(sets[0])
    torch.cuda.synchronize()
    assert torch.equal(sets[0].buf.idx, idx_flat) and torch.equal(sets[0].buf.out, out_flat), \
        "paged calls differ from flat"

    # per-stage / per-kernel timing: R launches of one stage per graph replay
    from sparse_attention_14_amd._lib import DSA_ERR_UNSUPPORTED, DsaError
    try:                                   # the fused prolog serves decode-shaped batches only
        st_prolog_indexer_topk(sets[0])
        fused_stage = {"prolog_indexer_topk": st_prolog_indexer_topk}
    except DsaError as e:
        if e.status != DSA_ERR_UNSUPPORTED:
            raise
        fused_stage = {}
    stages = {"step_separate_calls": step_separate,
              "prolog": st_prolog, "indexer": st_indexer, "indexer_topk": st_indexer_topk,
              **fused_stage, "indexer_attention": st_indexer_attention,
              "sfa": st_sfa, "sfa_split": st_sfa_split, "sfa_merge": st_sfa_merge,
              "indexer_topk_paged": st_indexer_topk_paged, "sfa_paged": st_sfa_paged}
    stage_us = {}
    for name, fn in stages.items():
        g = capture(fn)
        replay(g, 3)
        torch.cuda.synchronize()
        n = max(4, 64 // R)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        replay(g, n)
        b.record(stream)
        torch.cuda.synchronize()
        stage_us[name] = a.elapsed_time(b) * 1000.0 / (n * R)
    # the graphs of the stages replaced the step's results; restore and re-check once
    replay(g_step, 1)
    torch.cuda.synchronize()
    assert torch.equal(sets[0].buf.out, ref)

    proj = projections_stage(stream, dev)

    idx_tops = idx_ops / (stage_us["indexer"] * 1e-6) / 1e12
    sfa_gbps = n_sel * 1152 / (stage_us["sfa"] * 1e-6) / 1e9
    # roofline of the dominant kernel: among the single-kernel calls, the longest per launch.
    # Decode shapes are bound by HBM (algorithmic bytes per launch: the indexer's keys, scales,
    # q/w and scores; the attention split's gathered rows, q and indices); the prefill chunk
    # (many query tokens per sequence) by the matrix cores (int8 indexer ops, bf16 attention
    # flops), where the keys and gathered rows come from the caches
    prefill = wl.max_q_per_seq > 4
    idx_peak = INT8_PEAK_TOPS if cfg.code == "i8" else BF16_PEAK_TFLOPS
    # decode batches (at most 4 query tokens per sequence) take the streaming indexer kernel,
    # int8 prefill of the 64 x 128 shape the prefill kernel; batches with one attention split
    # per token and at least 256 workgroups of 64 heads the 64-head attention kernel
    if wl.max_q_per_seq <= 4:
        idx_kernel = "dsa::indexer_stream_kernel"
    elif cfg.code == "i8" and cfg.H == 64 and cfg.D == 128:
        idx_kernel = "dsa::indexer_prefill_kernel"
    else:
        idx_kernel = "dsa::indexer_kernel"
    sfa_kernel = "dsa::sfa_kernel64" if Hq % 64 == 0 and T * (Hq // 64) >= 256 else "dsa::sfa_kernel"
    single = {"indexer": (idx_kernel, b_indexer, idx_ops, idx_peak),
              "sfa_split": (sfa_kernel, n_sel * 1152 + T * Hq * 576 * 2 + T * k * 4,
                            sfa_flops, BF16_PEAK_TFLOPS)}
    dominant = max(single, key=lambda n: stage_us[n])
    kernel_name, dom_bytes, dom_ops, dom_peak = single[dominant]
    dom_sec = stage_us[dominant] * 1e-6
    if prefill:
        roof = {"kernel": kernel_name, "call": dominant, "bound": "mfma",
                "achieved": round(dom_ops / dom_sec / 1e12, 1), "peak": dom_peak,
                "unit": "TOP/s" if dominant == "indexer" and cfg.code == "i8" else "TFLOP/s",
                "frac": round(dom_ops / dom_sec / 1e12 / dom_peak, 4), "traffic": None,
                "ops_per_launch": dom_ops, "avg_launch_us": round(stage_us[dominant], 3)}
    else:
        dom_gbps = dom_bytes / dom_sec / 1e9
        roof = {"kernel": kernel_name, "call": dominant, "bound": "hbm", "achieved": round(dom_gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                "traffic": recorded_traffic(kernel_name, sp.name), "bytes_per_launch": dom_bytes,
                "avg_launch_us": round(stage_us[dominant], 3)}

    result = {
        "metric": "DSA decode us/step at B=4,64K ctx; indexer int8 TOPS; SFA gathered-KV GB/s",
        "value": round(us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": reps_w * R,
        "ms_per_step": round(us_step / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if cfg.code == "i8" else "fp8(e4m3)->bf16",
        "data": "synthetic",
        "config": {"workload": sp.name, "B": wl.B, "query_tokens": T, "kv_len_max": wl.max_kv_len,
                   "indexer": f"{H}x{D} {cfg.code} codes, {cfg.scale_dt} scales",
                   "topk": k, "attn_heads": Hq, "d_qk": 576, "d_v": 512,
                   "prolog": "rope+hadamard+quant" if sp.full_prolog else "quant",
                   "rotating_input_sets": R, "per_step_hbm_bytes": step_bytes},
        "timing": {"replays": reps, "steps_per_replay": R,
                   "median_us": round(float(np.median(per_rep)), 3),
                   "p10_us": round(float(np.percentile(per_rep, 10)), 3),
                   "p90_us": round(float(np.percentile(per_rep, 90)), 3),
                   "warm_us": round(warm_us, 3),
                   "note": "value = mean over every timed step; median/p10/p90 over the per-replay "
                           "means of R rotating-input steps; warm = R steps on one input set"},
        "step_roofline_frac": round(step_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "stage_us": {n: round(v, 3) for n, v in stage_us.items()},
        # indexer ops (2 H D per visible (token, key)) per second of the indexer call, against the
        # dense int8 (or, for e4m3 codes contracted on bf16, the bf16) MFMA peak
        ("indexer_tops_prefill_shape" if prefill else "indexer_tops_decode_shape"): round(idx_tops, 2),
        "indexer_tops_frac": round(idx_tops / idx_peak, 4),
        "sfa_gathered_GBps": round(sfa_gbps, 1),
        "sfa_gathered_frac": round(sfa_gbps / HBM_PEAK_GBPS, 4),
        "sfa_tflops": round(sfa_flops / (stage_us["sfa"] * 1e-6) / 1e12, 1),
        "roofline": roof,
        "wall_s_timed": round(wall, 4),
        "projections": proj,
    }

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def projections_stage(stream, dev) -> dict:
    """The Indexer Prolog's upstream linears at the pages' decode shape (8 tokens; W8A8
    1536 -> 64 x 128, key and weight linears from a 7168-wide hidden state), timed alone on
    rotating weight copies (past the MALL); HBM-bound on the weights."""
    import torch
    from sparse_attention_14_amd import dsa
    T, R, H, D, hidden = 8, 1536, 64, 128, 7168
    g = torch.Generator(device=dev).manual_seed(77)
    wbytes = H * D * R + H * D * 2 + (D + H) * hidden * 2
    n_sets = min(32, max(4, int(np.ceil(4 * MALL_BYTES / wbytes))))
    rint = lambda shape: torch.randint(-127, 128, shape, generator=g, device=dev, dtype=torch.int8)
    rn = lambda *shape: torch.randn(*shape, generator=g, device=dev)
    qa = rint((T, R))
    qa_s = (torch.rand(T, generator=g, device=dev) * 0.02 + 1e-3).half()
    x = rn(T, hidden).bfloat16()
    gam, bet = rn(D), rn(D)
    sets = [(rint((H * D, R)), (torch.rand(H * D, generator=g, device=dev) * 0.002 + 1e-4).half(),
             (rn(D, hidden) / hidden ** 0.5).bfloat16(), (rn(H, hidden) / hidden ** 0.5).bfloat16())
            for _ in range(n_sets)]
    q_pre = torch.empty((T, H * D), dtype=torch.float32, device=dev)
    k_pre = torch.empty((T, D), dtype=torch.float32, device=dev)
    wt = torch.empty((T, H), dtype=torch.float16, device=dev)
    ws = torch.empty(int(dsa.lib.dsa_indexer_projections_workspace_size(T, H, D)), dtype=torch.uint8,
                     device=dev)

    def run(sw):
        dsa.dsa_indexer_projections(qa, qa_s, sw[0], sw[1], x, sw[2], gam, bet, 1e-6, sw[3],
                                    H ** -0.5, q_pre=q_pre, k_pre=k_pre, weight=wt, ws=ws)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        run(sets[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for sw in sets:
            run(sw)
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(2, 64 // n_sets)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / (reps * n_sets)
    alg = wbytes + T * (R + hidden * 2) + T * (H * D + D) * 4 + T * H * 2
    return {"shape": {"tokens": T, "q_rank": R, "heads": H, "head_dim": D, "hidden": hidden},
            "us": round(us, 3), "algorithmic_bytes": alg,
            "GBps": round(alg / (us * 1e-6) / 1e9, 1),
            "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "rotating_weight_sets": n_sets}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, budget_s: float, max_tokens: int = 32) -> dict:
    """The oracle's decode step on the host cores (prolog of the new tokens and rows, indexer
    over every visible key, top-k, attention), repeated while within the time budget.  A batch
    of more than `max_tokens` query tokens is sampled: the oracle runs on a seeded subset of its
    tokens and the time is scaled by T / subset (every token's work is independent)."""
    import oracle
    from oracle.step import prolog_inputs_f64
    from threadpoolctl import threadpool_info
    sp = wl.spec
    oq = oracle.step.quantize_workload(wl)          # cache state from earlier steps (untimed)
    q_in, k_in = prolog_inputs_f64(wl)
    toks = np.arange(wl.T)
    if wl.T > max_tokens:
        toks = np.sort(np.random.default_rng(5).choice(wl.T, max_tokens, replace=False))
    rows = wl.new_rows()[toks]
    rope = sp.rope_dim if sp.full_prolog else 0
    sub = lambda a: None if a is None else a[toks]
    n, t_tot = 0, 0.0
    while (t_tot < budget_s and n < 50) or n == 0:
        t0 = time.perf_counter()
        nq = oracle.indexer_prolog(q_in[toks], k_in[rows], sub(wl.q_cos), sub(wl.q_sin),
                                   None if wl.k_cos is None else wl.k_cos[rows],
                                   None if wl.k_sin is None else wl.k_sin[rows], rope,
                                   sp.rope_offset, sp.rope_interleaved, sp.full_prolog, sp.code,
                                   sp.scale_dt)
        oq["k_codes"][rows] = nq["k_codes"]
        oq["k_scale"][rows] = nq["k_scale"]
        sc = oracle.indexer_scores(nq["q_codes"], nq["q_scale"], wl.w[toks], oq["k_codes"],
                                   oq["k_scale"], sp.code, wl.q_seq[toks], wl.q_pos[toks], wl.kv_start)
        idx = oracle.topk_select(sc, sp.k)
        oracle.sparse_attention(wl.q[toks], wl.kv, idx, wl.q_seq[toks], wl.kv_start, wl.sink, wl.scale)
        t_tot += time.perf_counter() - t0
        n += 1
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] + [1])
    blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer')})"
                     for p in info if p.get("user_api") == "blas") or "unknown"
    scale = wl.T / len(toks)
    what = (f"{n} full decode steps of the same workload ({wl.T} query tokens)" if scale == 1 else
            f"{n} steps over a seeded sample of {len(toks)} of the {wl.T} query tokens, time x {scale:g}")
    return {"value": round(t_tot / n * scale * 1e6, 1), "unit": "us/step", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(), "blas": blas,
            "sample": f"{what}, float64 numpy oracle, cache quantization excluded"}


if __name__ == "__main__":
    main()
