"""Python binding of the C ABI (include/dsa.h): same names, argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks device, dtype,
shape and contiguity, allocates missing outputs/workspaces with torch (device memory is
torch's business), and enqueues the HIP kernels on torch's current stream through
libdsa.so.  No step of the path runs in Python or in torch.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (DSA_BF16, DSA_F16, DSA_F32, DSA_FP8_E4M3, DSA_I8, DsaBatch, DsaDia, DsaPaging,
                   DsaPrologCfg, DsaProjections, check, lib)

D_QK, D_V = 576, 512

_CODE = {"i8": DSA_I8, "e4m3": DSA_FP8_E4M3}
_SCALE = {"f16": DSA_F16, "f32": DSA_F32}
_SCALE_TORCH = {"f16": torch.float16, "f32": torch.float32}
_CODE_TORCH = {"i8": torch.int8, "e4m3": torch.uint8}


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@dataclass
class Batch:
    """A ragged batch (mirrors dsa_batch).  Device arrays plus host-side sizes."""
    q_start: torch.Tensor   # [B+1] int32
    q_seq: torch.Tensor     # [T] int32
    q_pos: torch.Tensor     # [T] int32
    kv_start: torch.Tensor  # [B] int64
    num_seqs: int
    num_q: int
    max_q_per_seq: int
    max_kv_len: int

    def c(self) -> DsaBatch:
        return DsaBatch(self.num_seqs, self.num_q, self.max_q_per_seq, self.max_kv_len,
                        self.q_start.data_ptr(), self.q_seq.data_ptr(), self.q_pos.data_ptr(),
                        self.kv_start.data_ptr())


def make_batch(q_start, q_seq, q_pos, kv_start, device="cuda") -> Batch:
    """Build a Batch from host sequences/arrays (host sizes are derived from them)."""
    import numpy as np
    qs = np.asarray(q_start, dtype=np.int32)
    qq = np.asarray(q_seq, dtype=np.int32)
    qp = np.asarray(q_pos, dtype=np.int32)
    ks = np.asarray(kv_start, dtype=np.int64)
    B, T = ks.shape[0], qq.shape[0]
    if qs.shape != (B + 1,) or qp.shape != (T,) or (B and qs[-1] != T):
        raise ValueError("inconsistent batch arrays")
    mq = int(np.diff(qs).max()) if B and T else 0
    ml = int(qp.max()) + 1 if T else 0
    dev = lambda a: torch.from_numpy(a.copy()).to(device)
    return Batch(dev(qs), dev(qq), dev(qp), dev(ks), B, T, mq, ml)


def dsa_indexer_prolog(H: int, D: int, code: str, scale_dt: str, *, q_in=None, q_cos=None,
                       q_sin=None, q_codes=None, q_scale=None, k_in=None, k_cos=None,
                       k_sin=None, k_slot=None, k_cache=None, k_scale=None, rope_dim=0,
                       rope_offset=0, rope_interleaved=False, hadamard=False,
                       round_scale=False) -> None:
    """RoPE -> Hadamard -> per-row quant; writes q_codes/q_scale and k_cache/k_scale rows."""
    if code not in _CODE or scale_dt not in _SCALE:
        raise ValueError("code must be 'i8'|'e4m3', scale_dt 'f16'|'f32'")
    ct, st = _CODE_TORCH[code], _SCALE_TORCH[scale_dt]
    in_dt = None
    nq = nk = 0
    if q_in is not None:
        in_dt = q_in.dtype
        nq = q_in.shape[0]
        _need(q_in, "q_in", None, (nq, H, D))
        _need(q_codes, "q_codes", ct, (nq, H, D))
        _need(q_scale, "q_scale", st, (nq, H))
        if rope_dim:
            _need(q_cos, "q_cos", torch.float32, (nq, rope_dim // 2))
            _need(q_sin, "q_sin", torch.float32, (nq, rope_dim // 2))
    if k_in is not None:
        in_dt = in_dt or k_in.dtype
        nk = k_in.shape[0]
        _need(k_in, "k_in", in_dt, (nk, D))
        _need(k_slot, "k_slot", torch.int64, (nk,))
        _need(k_cache, "k_cache", ct)
        _need(k_scale, "k_scale", st)
        if k_cache.dim() != 2 or k_cache.shape[1] != D or k_scale.shape != (k_cache.shape[0],):
            raise ValueError("k_cache must be [N, D] and k_scale [N]")
        if rope_dim:
            _need(k_cos, "k_cos", torch.float32, (nk, rope_dim // 2))
            _need(k_sin, "k_sin", torch.float32, (nk, rope_dim // 2))
    if in_dt not in (None, torch.bfloat16, torch.float32):
        raise ValueError("inputs must be bf16 or fp32")
    cfg = DsaPrologCfg(H, D, rope_dim, rope_offset, int(rope_interleaved), int(hadamard),
                       int(round_scale), DSA_BF16 if in_dt == torch.bfloat16 else DSA_F32,
                       _CODE[code], _SCALE[scale_dt])
    check("dsa_indexer_prolog", lib.dsa_indexer_prolog(
        ctypes.byref(cfg), nq, _ptr(q_in), _ptr(q_cos), _ptr(q_sin), _ptr(q_codes), _ptr(q_scale),
        nk, _ptr(k_in), _ptr(k_cos), _ptr(k_sin), _ptr(k_slot), _ptr(k_cache), _ptr(k_scale),
        _stream()))


@dataclass
class Paging:
    """A paged cache layout (mirrors dsa_paging): position p of sequence b is cache row
    block_table[b, p // block_size] * block_size + p % block_size."""
    block_table: torch.Tensor  # [B, blocks_per_seq] int32
    block_size: int
    num_blocks: int

    def c(self) -> DsaPaging:
        _need(self.block_table, "block_table", torch.int32)
        if self.block_table.dim() != 2:
            raise ValueError("block_table must be [B, blocks_per_seq]")
        return DsaPaging(self.block_table.data_ptr(), self.block_table.shape[1], self.block_size,
                         self.num_blocks)


def _scores_ld(max_kv_len: int) -> int:
    return max(4, (max_kv_len + 63) // 64 * 64)


def dsa_indexer_scores(batch: Batch, H: int, D: int, code: str, scale_dt: str, q_codes, q_scale,
                       w, k_cache, k_scale, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Lightning Indexer scores -> fp32 [T, ld] (row t valid on columns 0..p_t)."""
    T = batch.num_q
    ct, st = _CODE_TORCH[code], _SCALE_TORCH[scale_dt]
    _need(q_codes, "q_codes", ct, (T, H, D))
    _need(q_scale, "q_scale", st, (T, H))
    _need(w, "w", torch.float16, (T, H))
    _need(k_cache, "k_cache", ct)
    _need(k_scale, "k_scale", st)
    if scores is None:
        scores = torch.empty((T, _scores_ld(batch.max_kv_len)), dtype=torch.float32,
                             device=q_codes.device)
    _need(scores, "scores", torch.float32)
    b = batch.c()
    check("dsa_indexer_scores", lib.dsa_indexer_scores(
        ctypes.byref(b), H, D, _CODE[code], _SCALE[scale_dt], _ptr(q_codes), _ptr(q_scale), _ptr(w),
        _ptr(k_cache), _ptr(k_scale), _ptr(scores), scores.shape[1] if scores.dim() == 2 else 0,
        _stream()))
    return scores


def dsa_indexer_dots_i32(batch: Batch, H: int, D: int, q_codes, k_cache,
                         dots: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Raw int32 dot products [T, H, ld] of the int8 indexer MFMA path (test hook)."""
    T = batch.num_q
    _need(q_codes, "q_codes", torch.int8, (T, H, D))
    _need(k_cache, "k_cache", torch.int8)
    if dots is None:
        dots = torch.zeros((T, H, _scores_ld(batch.max_kv_len)), dtype=torch.int32,
                           device=q_codes.device)
    _need(dots, "dots", torch.int32)
    b = batch.c()
    check("dsa_indexer_dots_i32", lib.dsa_indexer_dots_i32(
        ctypes.byref(b), H, D, _ptr(q_codes), _ptr(k_cache), _ptr(dots), dots.shape[-1], _stream()))
    return dots


CONTRACTIONS = {"bf16": 0, "fp8_k64": 1, "fp8_k16": 2}


def dsa_e4m3_dots(a, b, contraction: str) -> torch.Tensor:
    """fp32 C = A B^T over e4m3 codes (uint8 [m, d] and [n, d]) on one matrix-core path:
    "bf16" (the fp8 indexer's widening), "fp8_k64" or "fp8_k16" (test hook)."""
    _need(a, "a", torch.uint8)
    _need(b, "b", torch.uint8)
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("a and b must be [m, d] and [n, d]")
    c = torch.empty((a.shape[0], b.shape[0]), dtype=torch.float32, device=a.device)
    check("dsa_e4m3_dots", lib.dsa_e4m3_dots(_ptr(a), a.shape[0], _ptr(b), b.shape[0], a.shape[1],
                                             CONTRACTIONS[contraction], _ptr(c), _stream()))
    return c


def dsa_topk_workspace_size(num_q: int, max_kv_len: int, k: int) -> int:
    return int(lib.dsa_topk_workspace_size(num_q, max_kv_len, k))


def dsa_sparse_attn_workspace_size(num_q: int, Hq: int, k: int) -> int:
    return int(lib.dsa_sparse_attn_workspace_size(num_q, Hq, k))


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes; zero-filled
    # because the top-k workspace must start (and is left) zeroed
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)


def dsa_topk(batch: Batch, scores: torch.Tensor, k: int, idx: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k positions per token -> int32 [T, k], ascending, -1 padded."""
    T = batch.num_q
    _need(scores, "scores", torch.float32)
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32, (T, k))
    need = dsa_topk_workspace_size(T, batch.max_kv_len, k)
    if ws is None:
        ws = _workspace(need, scores.device)
    _need(ws, "ws", torch.uint8)
    b = batch.c()
    check("dsa_topk", lib.dsa_topk(ctypes.byref(b), _ptr(scores), scores.shape[1], k, _ptr(idx),
                                   _ptr(ws), ws.numel(), _stream()))
    return idx


def dsa_indexer_topk(batch: Batch, H: int, D: int, code: str, scale_dt: str, q_codes, q_scale,
                     w, k_cache, k_scale, k: int, scores: Optional[torch.Tensor] = None,
                     idx: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer scores then top-k in one call (the top-k's first radix pass fused into the
    indexer) -> idx int32 [T, k]; `scores` is written as by dsa_indexer_scores."""
    T = batch.num_q
    ct, st = _CODE_TORCH[code], _SCALE_TORCH[scale_dt]
    _need(q_codes, "q_codes", ct, (T, H, D))
    _need(q_scale, "q_scale", st, (T, H))
    _need(w, "w", torch.float16, (T, H))
    _need(k_cache, "k_cache", ct)
    _need(k_scale, "k_scale", st)
    if scores is None:
        scores = torch.empty((T, _scores_ld(batch.max_kv_len)), dtype=torch.float32,
                             device=q_codes.device)
    _need(scores, "scores", torch.float32)
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=q_codes.device)
    _need(idx, "idx", torch.int32, (T, k))
    if ws is None:
        ws = _workspace(dsa_topk_workspace_size(T, batch.max_kv_len, k), q_codes.device)
    _need(ws, "ws", torch.uint8)
    b = batch.c()
    check("dsa_indexer_topk", lib.dsa_indexer_topk(
        ctypes.byref(b), H, D, _CODE[code], _SCALE[scale_dt], _ptr(q_codes), _ptr(q_scale), _ptr(w),
        _ptr(k_cache), _ptr(k_scale), _ptr(scores), scores.shape[1] if scores.dim() == 2 else 0,
        k, _ptr(idx), _ptr(ws), ws.numel(), _stream()))
    return idx


def dsa_indexer_prolog_topk(batch: Batch, H: int, D: int, code: str, scale_dt: str, *, q_in, k_in,
                            w, q_codes, q_scale, k_cache, k_scale, k: int, q_cos=None, q_sin=None,
                            rope_dim=0, rope_offset=0, rope_interleaved=False, hadamard=False,
                            round_scale=False, scores: Optional[torch.Tensor] = None,
                            idx: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prolog of the batch's query rows and of each token's own key row (written at cache row
    kv_start[q_seq[t]] + q_pos[t]), indexer scores and top-k in one call -> idx int32 [T, k].
    q_codes/q_scale receive the quantized query; `scores` is written as by dsa_indexer_scores."""
    if code not in _CODE or scale_dt not in _SCALE:
        raise ValueError("code must be 'i8'|'e4m3', scale_dt 'f16'|'f32'")
    T = batch.num_q
    ct, st = _CODE_TORCH[code], _SCALE_TORCH[scale_dt]
    in_dt = q_in.dtype
    if in_dt not in (torch.bfloat16, torch.float32):
        raise ValueError("inputs must be bf16 or fp32")
    _need(q_in, "q_in", in_dt, (T, H, D))
    _need(k_in, "k_in", in_dt, (T, D))
    _need(w, "w", torch.float16, (T, H))
    _need(q_codes, "q_codes", ct, (T, H, D))
    _need(q_scale, "q_scale", st, (T, H))
    _need(k_cache, "k_cache", ct)
    _need(k_scale, "k_scale", st)
    if rope_dim:
        _need(q_cos, "q_cos", torch.float32, (T, rope_dim // 2))
        _need(q_sin, "q_sin", torch.float32, (T, rope_dim // 2))
    if scores is None:
        scores = torch.empty((T, _scores_ld(batch.max_kv_len)), dtype=torch.float32, device=q_in.device)
    _need(scores, "scores", torch.float32)
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=q_in.device)
    _need(idx, "idx", torch.int32, (T, k))
    if ws is None:
        ws = _workspace(dsa_topk_workspace_size(T, batch.max_kv_len, k), q_in.device)
    _need(ws, "ws", torch.uint8)
    cfg = DsaPrologCfg(H, D, rope_dim, rope_offset, int(rope_interleaved), int(hadamard),
                       int(round_scale), DSA_BF16 if in_dt == torch.bfloat16 else DSA_F32,
                       _CODE[code], _SCALE[scale_dt])
    b = batch.c()
    check("dsa_indexer_prolog_topk", lib.dsa_indexer_prolog_topk(
        ctypes.byref(cfg), ctypes.byref(b), _ptr(q_in), _ptr(q_cos), _ptr(q_sin), _ptr(k_in), _ptr(w),
        _ptr(q_codes), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale), k, _ptr(scores),
        scores.shape[1] if scores.dim() == 2 else 0, _ptr(idx), _ptr(ws), ws.numel(), _stream()))
    return idx


def dsa_sparse_attn_decode(batch: Batch, q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor,
                           sink: Optional[torch.Tensor], scale: float,
                           out: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse attention over the selected latent rows -> bf16 [T, Hq, 512]."""
    Hq, k, out, ws = _sfa_args(batch, q, kv, idx, sink, out, ws)
    b = batch.c()
    check("dsa_sparse_attn_decode", lib.dsa_sparse_attn_decode(
        ctypes.byref(b), Hq, _ptr(q), _ptr(kv), kv.stride(0), _ptr(idx), k, _ptr(sink),
        ctypes.c_float(scale), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return out


def dsa_sparse_attn_decode_noalloc(batch: Batch, q: torch.Tensor, kv: torch.Tensor,
                                   idx: torch.Tensor, sink: Optional[torch.Tensor], scale: float,
                                   out: torch.Tensor) -> torch.Tensor:
    """dsa_sparse_attn_decode with the split partials in the library's fixed per-GPU scratch
    (no workspace; `out` must be given, so nothing is allocated)."""
    _need(out, "out", torch.bfloat16)
    Hq, k, out, _ = _sfa_args(batch, q, kv, idx, sink, out, None, want_ws=False)
    b = batch.c()
    check("dsa_sparse_attn_decode_noalloc", lib.dsa_sparse_attn_decode_noalloc(
        ctypes.byref(b), Hq, _ptr(q), _ptr(kv), kv.stride(0), _ptr(idx), k, _ptr(sink),
        ctypes.c_float(scale), _ptr(out), _stream()))
    return out


def _sfa_args(batch: Batch, q, kv, idx, sink, out, ws, want_ws: bool = True):
    T = batch.num_q
    if q.dim() != 3:
        raise ValueError("q must be [T, Hq, 576]")
    Hq = q.shape[1]
    _need(q, "q", torch.bfloat16, (T, Hq, D_QK))
    if kv.dim() != 2 or kv.shape[1] < D_QK or kv.stride(1) != 1:
        raise ValueError("kv must be [N, >=576] bf16 with unit column stride")
    _need(kv, "kv", torch.bfloat16, contiguous=False)
    k = idx.shape[1]
    _need(idx, "idx", torch.int32, (T, k))
    if sink is not None:
        _need(sink, "sink", torch.float32, (Hq,))
    if out is None:
        out = torch.empty((T, Hq, D_V), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (T, Hq, D_V))
    need = dsa_sparse_attn_workspace_size(T, Hq, k)
    if want_ws and ws is None and need:
        ws = _workspace(need, q.device)
    return Hq, k, out, ws


def dsa_sparse_attn_split(batch: Batch, q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor,
                          sink: Optional[torch.Tensor], scale: float,
                          out: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None):
    """First stage of dsa_sparse_attn_decode: per-split partials into ws (or, when no
    workspace is needed, the final output).  Returns (out, ws) for dsa_sparse_attn_merge."""
    Hq, k, out, ws = _sfa_args(batch, q, kv, idx, sink, out, ws)
    b = batch.c()
    check("dsa_sparse_attn_split", lib.dsa_sparse_attn_split(
        ctypes.byref(b), Hq, _ptr(q), _ptr(kv), kv.stride(0), _ptr(idx), k, _ptr(sink),
        ctypes.c_float(scale), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return out, ws


def dsa_sparse_attn_merge(batch: Batch, Hq: int, k: int, sink: Optional[torch.Tensor],
                          out: torch.Tensor, ws: Optional[torch.Tensor]) -> torch.Tensor:
    """Second stage: merge the split partials in ws, apply the sink, write bf16 out."""
    _need(out, "out", torch.bfloat16, (batch.num_q, Hq, D_V))
    if sink is not None:
        _need(sink, "sink", torch.float32, (Hq,))
    b = batch.c()
    check("dsa_sparse_attn_merge", lib.dsa_sparse_attn_merge(
        ctypes.byref(b), Hq, k, _ptr(sink), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream()))
    return out


def dsa_indexer_attention_workspace_size(num_q: int, max_kv_len: int, k: int, Hq: int) -> int:
    return int(lib.dsa_indexer_attention_workspace_size(num_q, max_kv_len, k, Hq))


def dsa_indexer_attention(batch: Batch, H: int, D: int, code: str, scale_dt: str, *, q_codes,
                          q_scale, w, k_cache, k_scale, k: int, q: torch.Tensor, kv: torch.Tensor,
                          sink: Optional[torch.Tensor], scale: float, q_in=None, k_in=None,
                          q_cos=None, q_sin=None, rope_dim=0, rope_offset=0,
                          rope_interleaved=False, hadamard=False, round_scale=False,
                          scores: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Indexer (with the prolog when q_in is given), top-k and sparse attention of a decode step
    in one call -> (idx int32 [T, k], out bf16 [T, Hq, 512]).  With q_in, q_codes/q_scale
    receive the quantized query and token t's new key row (k_in row t) is written at cache row
    kv_start[q_seq[t]] + q_pos[t]; `scores` is written as by dsa_indexer_scores."""
    if code not in _CODE or scale_dt not in _SCALE:
        raise ValueError("code must be 'i8'|'e4m3', scale_dt 'f16'|'f32'")
    T = batch.num_q
    scores = _indexer_operands(batch, H, D, code, scale_dt, q_codes, q_scale, w, k_cache, k_scale,
                               scores)
    cfg = None
    if q_in is not None:
        in_dt = q_in.dtype
        if in_dt not in (torch.bfloat16, torch.float32):
            raise ValueError("inputs must be bf16 or fp32")
        _need(q_in, "q_in", in_dt, (T, H, D))
        _need(k_in, "k_in", in_dt, (T, D))
        if rope_dim:
            _need(q_cos, "q_cos", torch.float32, (T, rope_dim // 2))
            _need(q_sin, "q_sin", torch.float32, (T, rope_dim // 2))
        cfg = DsaPrologCfg(H, D, rope_dim, rope_offset, int(rope_interleaved), int(hadamard),
                           int(round_scale), DSA_BF16 if in_dt == torch.bfloat16 else DSA_F32,
                           _CODE[code], _SCALE[scale_dt])
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=q_codes.device)
    _need(idx, "idx", torch.int32, (T, k))
    Hq, _, out, _ = _sfa_args(batch, q, kv, idx, sink, out, None, want_ws=False)
    if ws is None:
        ws = _workspace(dsa_indexer_attention_workspace_size(T, batch.max_kv_len, k, Hq), q.device)
    _need(ws, "ws", torch.uint8)
    d = DsaDia(ctypes.pointer(cfg) if cfg is not None else None, _ptr(q_in), _ptr(q_cos),
               _ptr(q_sin), _ptr(k_in), H, D, _CODE[code], _SCALE[scale_dt], _ptr(q_codes),
               _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(scores),
               scores.shape[1] if scores.dim() == 2 else 0, k, _ptr(idx), Hq, _ptr(q), _ptr(kv),
               kv.stride(0), _ptr(sink), ctypes.c_float(scale), _ptr(out))
    b = batch.c()
    check("dsa_indexer_attention", lib.dsa_indexer_attention(
        ctypes.byref(b), ctypes.byref(d), _ptr(ws), ws.numel(), _stream()))
    return idx, out


def _indexer_operands(batch, H, D, code, scale_dt, q_codes, q_scale, w, k_cache, k_scale, scores):
    T = batch.num_q
    ct, st = _CODE_TORCH[code], _SCALE_TORCH[scale_dt]
    _need(q_codes, "q_codes", ct, (T, H, D))
    _need(q_scale, "q_scale", st, (T, H))
    _need(w, "w", torch.float16, (T, H))
    _need(k_cache, "k_cache", ct)
    _need(k_scale, "k_scale", st)
    if scores is None:
        scores = torch.empty((T, _scores_ld(batch.max_kv_len)), dtype=torch.float32,
                             device=q_codes.device)
    _need(scores, "scores", torch.float32)
    return scores


def dsa_indexer_scores_paged(batch: Batch, paging: Paging, H: int, D: int, code: str,
                             scale_dt: str, q_codes, q_scale, w, k_cache, k_scale,
                             scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dsa_indexer_scores with k_cache / k_scale rows addressed through the block table."""
    scores = _indexer_operands(batch, H, D, code, scale_dt, q_codes, q_scale, w, k_cache, k_scale,
                               scores)
    b, pg = batch.c(), paging.c()
    check("dsa_indexer_scores_paged", lib.dsa_indexer_scores_paged(
        ctypes.byref(b), ctypes.byref(pg), H, D, _CODE[code], _SCALE[scale_dt], _ptr(q_codes),
        _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(scores),
        scores.shape[1] if scores.dim() == 2 else 0, _stream()))
    return scores


def dsa_indexer_topk_paged(batch: Batch, paging: Paging, H: int, D: int, code: str,
                           scale_dt: str, q_codes, q_scale, w, k_cache, k_scale, k: int,
                           scores: Optional[torch.Tensor] = None,
                           idx: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dsa_indexer_topk with k_cache / k_scale rows addressed through the block table."""
    T = batch.num_q
    scores = _indexer_operands(batch, H, D, code, scale_dt, q_codes, q_scale, w, k_cache, k_scale,
                               scores)
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=q_codes.device)
    _need(idx, "idx", torch.int32, (T, k))
    if ws is None:
        ws = _workspace(dsa_topk_workspace_size(T, batch.max_kv_len, k), q_codes.device)
    _need(ws, "ws", torch.uint8)
    b, pg = batch.c(), paging.c()
    check("dsa_indexer_topk_paged", lib.dsa_indexer_topk_paged(
        ctypes.byref(b), ctypes.byref(pg), H, D, _CODE[code], _SCALE[scale_dt], _ptr(q_codes),
        _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(scores),
        scores.shape[1] if scores.dim() == 2 else 0, k, _ptr(idx), _ptr(ws), ws.numel(),
        _stream()))
    return idx


def dsa_sparse_attn_decode_paged(batch: Batch, paging: Paging, q: torch.Tensor, kv: torch.Tensor,
                                 idx: torch.Tensor, sink: Optional[torch.Tensor], scale: float,
                                 out: Optional[torch.Tensor] = None,
                                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dsa_sparse_attn_decode with kv rows addressed through the block table."""
    Hq, k, out, ws = _sfa_args(batch, q, kv, idx, sink, out, ws)
    b, pg = batch.c(), paging.c()
    check("dsa_sparse_attn_decode_paged", lib.dsa_sparse_attn_decode_paged(
        ctypes.byref(b), ctypes.byref(pg), Hq, _ptr(q), _ptr(kv), kv.stride(0), _ptr(idx), k,
        _ptr(sink), ctypes.c_float(scale), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream()))
    return out


def dsa_indexer_projections(q_a, q_a_scale, w_qb, w_qb_scale, x, w_k, ln_gamma, ln_beta,
                            ln_eps: float, w_proj, weight_scale: float, q_pre=None, k_pre=None,
                            weight=None, ws=None):
    """The Indexer Prolog's upstream projections -> (q_pre fp32 [T, H*D], k_pre fp32 [T, D],
    weight fp16 [T, H]).  q_a int8 [T, R], q_a_scale fp16 [T], w_qb int8 [H*D, R],
    w_qb_scale fp16 [H*D], x bf16 [T, hidden], w_k bf16 [D, hidden], ln_gamma/ln_beta fp32 [D],
    w_proj bf16 [H, hidden]."""
    T, R = q_a.shape
    D, hidden = w_k.shape
    H = w_proj.shape[0]
    _need(q_a, "q_a", torch.int8, (T, R))
    _need(q_a_scale, "q_a_scale", torch.float16, (T,))
    _need(w_qb, "w_qb", torch.int8, (H * D, R))
    _need(w_qb_scale, "w_qb_scale", torch.float16, (H * D,))
    _need(x, "x", torch.bfloat16, (T, hidden))
    _need(w_k, "w_k", torch.bfloat16, (D, hidden))
    _need(ln_gamma, "ln_gamma", torch.float32, (D,))
    _need(ln_beta, "ln_beta", torch.float32, (D,))
    _need(w_proj, "w_proj", torch.bfloat16, (H, hidden))
    dev = q_a.device
    if q_pre is None:
        q_pre = torch.empty((T, H * D), dtype=torch.float32, device=dev)
    if k_pre is None:
        k_pre = torch.empty((T, D), dtype=torch.float32, device=dev)
    if weight is None:
        weight = torch.empty((T, H), dtype=torch.float16, device=dev)
    _need(q_pre, "q_pre", torch.float32, (T, H * D))
    _need(k_pre, "k_pre", torch.float32, (T, D))
    _need(weight, "weight", torch.float16, (T, H))
    if ws is None:
        ws = torch.empty(max(int(lib.dsa_indexer_projections_workspace_size(T, H, D)), 1),
                         dtype=torch.uint8, device=dev)
    _need(ws, "ws", torch.uint8)
    args = DsaProjections(T, R, hidden, H, D, q_a.data_ptr(), q_a_scale.data_ptr(), w_qb.data_ptr(),
                          w_qb_scale.data_ptr(), x.data_ptr(), w_k.data_ptr(), ln_gamma.data_ptr(),
                          ln_beta.data_ptr(), ln_eps, w_proj.data_ptr(), weight_scale,
                          q_pre.data_ptr(), k_pre.data_ptr(), weight.data_ptr())
    check("dsa_indexer_projections", lib.dsa_indexer_projections(ctypes.byref(args), _ptr(ws),
                                                                 ws.numel(), _stream()))
    return q_pre, k_pre, weight


def dsa_last_error() -> str:
    return lib.dsa_last_error().decode(errors="replace")


def dsa_version() -> str:
    return lib.dsa_version().decode()
