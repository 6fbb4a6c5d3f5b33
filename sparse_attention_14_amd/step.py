"""One DSA decode step through the C ABI: prolog -> indexer scores + top-k -> sparse attention,
in one call (dsa_indexer_attention: the prolog inside the indexer kernel where the library
supports that form, the attention resolving its own slices of the selection) or as separate calls.

[DIA] "Deepseek Indexer Attention" (jsqmd.com/news/787325): the decode layer runs the indexer
prolog, the Lightning Indexer with its TopK and Sparse Flash Attention in that order (the MLA
prolog that makes the attention query and the latent KV rows is upstream of this path).
The step allocates nothing when the caller passes preallocated buffers.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import DSA_ERR_UNSUPPORTED, DsaError
from .dsa import (Batch, _scores_ld, dsa_indexer_attention, dsa_indexer_attention_workspace_size,
                  dsa_indexer_prolog, dsa_indexer_topk, dsa_sparse_attn_decode,
                  dsa_sparse_attn_workspace_size, dsa_topk_workspace_size)


@dataclass
class IndexerCfg:
    H: int = 64
    D: int = 128
    code: str = "i8"            # "i8" | "e4m3"
    scale_dt: str = "f16"       # "f16" | "f32"
    rope_dim: int = 0           # 0 = no RoPE (already-rotated inputs)
    rope_offset: int = 64
    rope_interleaved: bool = False
    hadamard: bool = False
    k: int = 2048               # top-k


@dataclass
class StepBuffers:
    q_codes: torch.Tensor
    q_scale: torch.Tensor
    scores: torch.Tensor
    idx: torch.Tensor
    out: torch.Tensor
    ws_topk: torch.Tensor
    ws_sfa: Optional[torch.Tensor]
    ws_dia: torch.Tensor            # the one-call path's workspace (zero-filled once)

    @staticmethod
    def alloc(batch: Batch, cfg: IndexerCfg, Hq: int, device="cuda") -> "StepBuffers":
        T = batch.num_q
        ct = torch.int8 if cfg.code == "i8" else torch.uint8
        st = torch.float16 if cfg.scale_dt == "f16" else torch.float32
        nws = dsa_sparse_attn_workspace_size(T, Hq, cfg.k)
        return StepBuffers(
            q_codes=torch.empty((T, cfg.H, cfg.D), dtype=ct, device=device),
            q_scale=torch.empty((T, cfg.H), dtype=st, device=device),
            scores=torch.empty((T, _scores_ld(batch.max_kv_len)), dtype=torch.float32, device=device),
            idx=torch.empty((T, cfg.k), dtype=torch.int32, device=device),
            out=torch.empty((T, Hq, 512), dtype=torch.bfloat16, device=device),
            ws_topk=torch.zeros(max(1, dsa_topk_workspace_size(T, batch.max_kv_len, cfg.k)),
                                dtype=torch.uint8, device=device),
            ws_sfa=torch.empty(nws, dtype=torch.uint8, device=device) if nws else None,
            ws_dia=torch.zeros(max(1, dsa_indexer_attention_workspace_size(T, batch.max_kv_len, cfg.k, Hq)),
                               dtype=torch.uint8, device=device))


def decode_step(batch: Batch, cfg: IndexerCfg, *, q_in, k_in, new_slots, w, k_cache, k_scale,
                q_attn, kv, sink, scale: float, buf: StepBuffers, q_cos=None, q_sin=None,
                k_cos=None, k_sin=None, fused: bool = True) -> torch.Tensor:
    """Run the four stages for the batch's query tokens.

    q_in [T, H, D] / k_in [T, D]: raw indexer query / key activations of the new tokens
    (bf16 or fp32); new_slots [T] int64: cache rows of the new tokens' keys (row
    kv_start[q_seq[t]] + q_pos[t] of the batch layout); k_cache/k_scale: the quantized indexer
    key cache; q_attn [T, Hq, 576] bf16, kv [N, 576] bf16, sink [Hq].
    With `fused` the whole step is one call (dsa_indexer_attention; the keys' rotary tables are
    the tokens' own, q_cos/q_sin), else the separate calls dsa_indexer_prolog,
    dsa_indexer_topk and dsa_sparse_attn_decode.  Returns buf.out [T, Hq, 512] bf16 (buf.idx
    holds the selection, buf.scores the indexer scores).
    """
    if fused:
        try:
            dsa_indexer_attention(batch, cfg.H, cfg.D, cfg.code, cfg.scale_dt, q_codes=buf.q_codes,
                                  q_scale=buf.q_scale, w=w, k_cache=k_cache, k_scale=k_scale,
                                  k=cfg.k, q=q_attn, kv=kv, sink=sink, scale=scale, q_in=q_in,
                                  k_in=k_in, q_cos=q_cos, q_sin=q_sin, rope_dim=cfg.rope_dim,
                                  rope_offset=cfg.rope_offset,
                                  rope_interleaved=cfg.rope_interleaved, hadamard=cfg.hadamard,
                                  scores=buf.scores, idx=buf.idx, out=buf.out, ws=buf.ws_dia)
            return buf.out
        except DsaError as e:
            if e.status != DSA_ERR_UNSUPPORTED:
                raise
    dsa_indexer_prolog(cfg.H, cfg.D, cfg.code, cfg.scale_dt, q_in=q_in, q_cos=q_cos, q_sin=q_sin,
                       q_codes=buf.q_codes, q_scale=buf.q_scale, k_in=k_in, k_cos=k_cos, k_sin=k_sin,
                       k_slot=new_slots, k_cache=k_cache, k_scale=k_scale, rope_dim=cfg.rope_dim,
                       rope_offset=cfg.rope_offset, rope_interleaved=cfg.rope_interleaved,
                       hadamard=cfg.hadamard)
    dsa_indexer_topk(batch, cfg.H, cfg.D, cfg.code, cfg.scale_dt, buf.q_codes, buf.q_scale, w,
                     k_cache, k_scale, cfg.k, scores=buf.scores, idx=buf.idx, ws=buf.ws_topk)
    return dsa_sparse_attn_decode(batch, q_attn, kv, buf.idx, sink, scale, out=buf.out,
                                  ws=buf.ws_sfa)
