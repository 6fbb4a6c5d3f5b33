"""Seeded synthetic workloads for the DeepSeek sparse-attention (DSA) decode path.

This module computes no step of the method.  It only
  * draws random values (numpy PCG64, seed = 1000 + workload id for the five
    named workloads),
  * casts drawn values to their storage dtype (bf16 / fp16, round-to-nearest-even),
  * lays out ragged batches (sequence starts, query-token positions),
  * builds rotary cos/sin tables, which the indexer prolog takes as caller inputs.

Both the HIP path and the CPU oracle consume what it returns; neither is imported here.

Shapes follow the workloads described on the pages: an indexer of 64 heads x 128
dims with int8 (or fp8) codes and fp16 per-token-head scales, top-k 2048, and MLA
latent KV rows of 576 = 512 (nope) + 64 (rope) bf16 values with d_v = 512 for
128 query heads ("DeepSeek-V3.2-Exp Indexer Prolog / Lightning Indexer" page, typical
shape 4 batch, MTP1, 64K cache; "TileLang-Ascend SFA" page, tensor shapes).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

D_QK = 576        # 512 nope + 64 rope, one latent KV head shared by all query heads
D_V = 512         # value = first 512 columns of the same row
ROPE_BASE = 10000.0


@dataclasses.dataclass
class Spec:
    """Shape/recipe of one workload (no arrays)."""
    name: str
    seed: int
    seq_lens: Sequence[int]          # L_b: cache rows of sequence b, counting its new tokens
    q_per_seq: Sequence[int]         # S_b: query tokens of sequence b (at positions L_b-S_b .. L_b-1)
    H: int = 64                      # indexer heads
    D: int = 128                     # indexer head dim
    code: str = "i8"                 # "i8" or "e4m3"
    scale_dt: str = "f16"            # "f16" or "f32"
    w_std: float = 1.0 / 8.0         # indexer head weights ~ N(0,1) * w_std, stored fp16
    k: int = 2048                    # top-k
    Hq: int = 128                    # SFA query heads
    full_prolog: bool = False        # True: RoPE + Hadamard + quant on device (bf16 inputs)
    rope_dim: int = 64
    rope_offset: int = 64            # rope dims are the last 64 of 128 (nope || rope)
    rope_interleaved: bool = False
    sink: bool = True


NAMED = {
    0: Spec("tiny_decode_b1_L2048", 1000, [2048], [1], H=8, D=64, code="i8",
            scale_dt="f32", w_std=1.0 / math.sqrt(8.0), k=256, Hq=16),
    1: Spec("decode_b4_mtp1_L65536", 1001, [65536] * 4, [2] * 4),
    2: Spec("ragged_decode_b32_L4096-65536", 1002, [], [1] * 32),   # lengths drawn
    3: Spec("prefill_4096_on_61440", 1003, [65536], [4096]),
    4: Spec("long_fp8_prolog_b8_L131072", 1004, [131072] * 8, [1] * 8, code="e4m3",
            full_prolog=True),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    # ragged batch layout (host copies; the device gets the same arrays)
    q_start: np.ndarray      # [B+1] int32
    q_seq: np.ndarray        # [T] int32
    q_pos: np.ndarray        # [T] int32, keys 0..q_pos[t] of its sequence are visible
    kv_start: np.ndarray     # [B] int64 first row of sequence b in the flat caches
    seq_lens: np.ndarray     # [B] int64
    # indexer prolog inputs (raw activations); bf16 inputs are given as uint16 bit patterns
    in_dtype: str            # "f32" or "bf16"
    idx_q_in: np.ndarray     # [T, H, D]
    idx_k_in: np.ndarray     # [N, D] one raw key row per cache row (new rows included)
    q_cos: Optional[np.ndarray]   # [T, rope_dim/2] float32 (None: no rope)
    q_sin: Optional[np.ndarray]
    k_cos: Optional[np.ndarray]   # [N, rope_dim/2] float32
    k_sin: Optional[np.ndarray]
    w: np.ndarray            # [T, H] float16 head weights
    # sparse attention inputs
    kv: np.ndarray           # [N, 576] uint16 bf16 bits
    q: np.ndarray            # [T, Hq, 576] uint16 bf16 bits
    sink: Optional[np.ndarray]    # [Hq] float32 or None
    scale: float             # softmax scale 1/sqrt(576)

    @property
    def T(self) -> int:
        return int(self.q_seq.shape[0])

    @property
    def B(self) -> int:
        return int(self.kv_start.shape[0])

    @property
    def N(self) -> int:
        return int(self.idx_k_in.shape[0])

    @property
    def max_kv_len(self) -> int:
        return int(self.q_pos.max()) + 1 if self.T else 0

    @property
    def max_q_per_seq(self) -> int:
        return int(np.diff(self.q_start).max()) if self.B else 0

    def new_rows(self) -> np.ndarray:
        """Flat cache row of each query token's own key (its prolog writes it)."""
        return (self.kv_start[self.q_seq] + self.q_pos).astype(np.int64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Cast float32 values to bf16 (round-to-nearest-even) and return the uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def rotary_tables(pos: np.ndarray, rope_dim: int, base: float = ROPE_BASE):
    """cos/sin of pos * base^(-2i/rope_dim), i < rope_dim/2, as float32 [len(pos), rope_dim/2]."""
    half = rope_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / rope_dim)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make(spec: Spec, seed: Optional[int] = None, lens: Optional[Sequence[int]] = None) -> Workload:
    """Draw a workload.  Draw order: lengths -> indexer k -> indexer q -> w -> kv -> SFA q -> sink."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    B = len(spec.q_per_seq)
    if lens is not None:
        seq_lens = np.asarray(lens, dtype=np.int64)
    elif len(spec.seq_lens) == 0:
        seq_lens = rng.integers(4096, 65536, size=B, endpoint=True).astype(np.int64)
    else:
        seq_lens = np.asarray(spec.seq_lens, dtype=np.int64)
    S = np.asarray(spec.q_per_seq, dtype=np.int64)
    assert seq_lens.shape == (B,) and np.all(S >= 0) and np.all(S <= seq_lens)
    kv_start = np.zeros(B, dtype=np.int64)
    if B:
        kv_start[1:] = np.cumsum(seq_lens)[:-1]
    N = int(seq_lens.sum())
    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(S)
    T = int(q_start[-1])
    q_seq = np.repeat(np.arange(B, dtype=np.int32), S)
    q_pos = np.concatenate([np.arange(L - s, L, dtype=np.int32) for L, s in zip(seq_lens, S)]) \
        if T else np.zeros(0, dtype=np.int32)

    H, D = spec.H, spec.D
    k_raw = rng.standard_normal((N, D), dtype=np.float32)
    q_raw = rng.standard_normal((T, H, D), dtype=np.float32)
    w = (rng.standard_normal((T, H), dtype=np.float32) * np.float32(spec.w_std)).astype(np.float16)
    kv = bf16_bits(rng.standard_normal((N, D_QK), dtype=np.float32))
    q = bf16_bits(rng.standard_normal((T, spec.Hq, D_QK), dtype=np.float32))
    sink = rng.standard_normal(spec.Hq, dtype=np.float32) if spec.sink else None

    if spec.full_prolog:
        in_dtype = "bf16"
        idx_k_in, idx_q_in = bf16_bits(k_raw), bf16_bits(q_raw)
        row_pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seq_lens]) if N else \
            np.zeros(0, dtype=np.int64)
        k_cos, k_sin = rotary_tables(row_pos, spec.rope_dim)
        q_cos, q_sin = rotary_tables(q_pos, spec.rope_dim)
    else:
        in_dtype = "f32"
        idx_k_in, idx_q_in = k_raw, q_raw
        k_cos = k_sin = q_cos = q_sin = None
    return Workload(spec=spec, q_start=q_start, q_seq=q_seq, q_pos=q_pos, kv_start=kv_start,
                    seq_lens=seq_lens, in_dtype=in_dtype, idx_q_in=idx_q_in, idx_k_in=idx_k_in,
                    q_cos=q_cos, q_sin=q_sin, k_cos=k_cos, k_sin=k_sin, w=w, kv=kv, q=q,
                    sink=sink, scale=1.0 / math.sqrt(D_QK))


def named(cfg_id: int) -> Workload:
    return make(NAMED[cfg_id])


def random_topk_idx(rng: np.random.Generator, q_pos: np.ndarray, k: int,
                    pad_frac: float = 0.0) -> np.ndarray:
    """Random selections for isolated attention tests: per token, min(k, p+1) distinct
    positions in [0, p] (ascending), then -1 padding; pad_frac of the slots are
    additionally replaced by -1 at random places."""
    T = q_pos.shape[0]
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = min(k, int(q_pos[t]) + 1)
        sel = np.sort(rng.choice(int(q_pos[t]) + 1, size=n, replace=False)).astype(np.int32)
        out[t, :n] = sel
        if pad_frac > 0:
            drop = rng.random(k) < pad_frac
            out[t, drop] = -1
    return out


@dataclasses.dataclass
class BlockLayout:
    """A paged placement of a workload's flat caches (rows of sequence b at kv_start[b] + p):
    sequence b's logical block j sits in physical block table[b, j]; row_map[r] is the paged
    row of flat row r.  Pure data layout: blocks of `block_size` rows in a random order, with
    `spare` unused blocks mixed in."""
    block_size: int
    table: np.ndarray        # [B, blocks_per_seq] int32 (-1 past a sequence's last block)
    row_map: np.ndarray      # [N] int64
    num_blocks: int


def block_layout(wl: Workload, block_size: int, seed: int = 0, spare: int = 3) -> BlockLayout:
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in wl.seq_lens]
    nblk = [-(-n // block_size) for n in lengths]
    total = sum(nblk) + spare
    perm = rng.permutation(total)
    table = np.full((len(lengths), max(nblk)), -1, dtype=np.int32)
    row_map = np.empty(wl.N, dtype=np.int64)
    k = 0
    for b, n in enumerate(lengths):
        for j in range(nblk[b]):
            table[b, j] = perm[k]
            k += 1
        p = np.arange(n)
        row_map[int(wl.kv_start[b]) + p] = table[b, p // block_size].astype(np.int64) * block_size + p % block_size
    return BlockLayout(block_size, table, row_map, total)


def device_arrays(wl: Workload, device="cuda") -> dict:
    """The same workload as torch tensors on `device` (no arithmetic: copies and dtype views)."""
    import torch

    def dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            t = t.view(dtype)
        return t.to(device)

    in_t = torch.bfloat16 if wl.in_dtype == "bf16" else None
    out = {
        "q_start": dev(wl.q_start), "q_seq": dev(wl.q_seq), "q_pos": dev(wl.q_pos),
        "kv_start": dev(wl.kv_start),
        "idx_q_in": dev(wl.idx_q_in, in_t), "idx_k_in": dev(wl.idx_k_in, in_t),
        "w": dev(wl.w), "kv": dev(wl.kv, torch.bfloat16), "q": dev(wl.q, torch.bfloat16),
        "sink": None if wl.sink is None else dev(wl.sink),
        "new_rows": dev(wl.new_rows()), "all_rows": torch.arange(wl.N, dtype=torch.int64, device=device),
    }
    for name in ("q_cos", "q_sin", "k_cos", "k_sin"):
        v = getattr(wl, name)
        out[name] = None if v is None else dev(v)
    return out
