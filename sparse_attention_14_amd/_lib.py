"""ctypes loader for libdsa.so and the C structs of include/dsa.h.

The library must exist (build it with `python -m sparse_attention_14_amd.build`); there is
no fallback of any kind -- importing this module without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

# dsa_status
DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}
# dsa_dtype
DSA_I8, DSA_FP8_E4M3, DSA_F16, DSA_BF16, DSA_F32 = 1, 2, 3, 4, 5


class DsaBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q", ctypes.c_int32),
                ("max_q_per_seq", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("q_start", ctypes.c_void_p), ("q_seq", ctypes.c_void_p),
                ("q_pos", ctypes.c_void_p), ("kv_start", ctypes.c_void_p)]


class DsaPaging(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("blocks_per_seq", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32)]


class DsaPrologCfg(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("D", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("rope_offset", ctypes.c_int32), ("rope_interleaved", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("round_scale", ctypes.c_int32),
                ("in_dtype", ctypes.c_int), ("code_dtype", ctypes.c_int),
                ("scale_dtype", ctypes.c_int)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_BP = ctypes.POINTER(DsaBatch)
_PP = ctypes.POINTER(DsaPaging)

# name -> (restype, argtypes); mirrors include/dsa.h
class DsaProjections(ctypes.Structure):
    _fields_ = [("num_q", ctypes.c_int32), ("q_rank", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("q_a", ctypes.c_void_p), ("q_a_scale", ctypes.c_void_p), ("w_qb", ctypes.c_void_p),
                ("w_qb_scale", ctypes.c_void_p), ("x", ctypes.c_void_p), ("w_k", ctypes.c_void_p),
                ("ln_gamma", ctypes.c_void_p), ("ln_beta", ctypes.c_void_p), ("ln_eps", ctypes.c_float),
                ("w_proj", ctypes.c_void_p), ("weight_scale", ctypes.c_float),
                ("q_pre", ctypes.c_void_p), ("k_pre", ctypes.c_void_p), ("weight", ctypes.c_void_p)]


class DsaDia(ctypes.Structure):
    _fields_ = [("prolog", ctypes.POINTER(DsaPrologCfg)), ("q_in", ctypes.c_void_p),
                ("q_cos", ctypes.c_void_p), ("q_sin", ctypes.c_void_p), ("k_in", ctypes.c_void_p),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("code_dtype", ctypes.c_int),
                ("scale_dtype", ctypes.c_int), ("q_codes", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p), ("w", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("k", ctypes.c_int32), ("idx", ctypes.c_void_p), ("Hq", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_row_stride", ctypes.c_int64),
                ("sink", ctypes.c_void_p), ("scale", ctypes.c_float), ("out", ctypes.c_void_p)]


SIGNATURES = {
    "dsa_indexer_prolog": (ctypes.c_int, [ctypes.POINTER(DsaPrologCfg), _I32, _P, _P, _P, _P, _P,
                                          _I32, _P, _P, _P, _P, _P, _P, _P]),
    "dsa_indexer_scores": (ctypes.c_int, [_BP, _I32, _I32, ctypes.c_int, ctypes.c_int, _P, _P, _P,
                                          _P, _P, _P, _I64, _P]),
    "dsa_indexer_dots_i32": (ctypes.c_int, [_BP, _I32, _I32, _P, _P, _P, _I64, _P]),
    "dsa_e4m3_dots": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _I32, _P, _P]),
    "dsa_indexer_prolog_topk": (ctypes.c_int, [ctypes.POINTER(DsaPrologCfg), _BP, _P, _P, _P, _P, _P,
                                               _P, _P, _P, _P, _I32, _P, _I64, _P, _P, _SZ, _P]),
    "dsa_topk_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "dsa_topk": (ctypes.c_int, [_BP, _P, _I64, _I32, _P, _P, _SZ, _P]),
    "dsa_indexer_topk": (ctypes.c_int, [_BP, _I32, _I32, ctypes.c_int, ctypes.c_int, _P, _P, _P,
                                        _P, _P, _P, _I64, _I32, _P, _P, _SZ, _P]),
    "dsa_sparse_attn_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "dsa_sparse_attn_decode": (ctypes.c_int, [_BP, _I32, _P, _P, _I64, _P, _I32, _P,
                                              ctypes.c_float, _P, _P, _SZ, _P]),
    "dsa_sparse_attn_split": (ctypes.c_int, [_BP, _I32, _P, _P, _I64, _P, _I32, _P,
                                             ctypes.c_float, _P, _P, _SZ, _P]),
    "dsa_sparse_attn_merge": (ctypes.c_int, [_BP, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "dsa_sparse_attn_decode_noalloc": (ctypes.c_int, [_BP, _I32, _P, _P, _I64, _P, _I32, _P,
                                                      ctypes.c_float, _P, _P]),
    "dsa_indexer_scores_paged": (ctypes.c_int, [_BP, _PP, _I32, _I32, ctypes.c_int, ctypes.c_int,
                                                _P, _P, _P, _P, _P, _P, _I64, _P]),
    "dsa_indexer_topk_paged": (ctypes.c_int, [_BP, _PP, _I32, _I32, ctypes.c_int, ctypes.c_int,
                                              _P, _P, _P, _P, _P, _P, _I64, _I32, _P, _P, _SZ, _P]),
    "dsa_sparse_attn_decode_paged": (ctypes.c_int, [_BP, _PP, _I32, _P, _P, _I64, _P, _I32, _P,
                                                    ctypes.c_float, _P, _P, _SZ, _P]),
    "dsa_indexer_attention_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
    "dsa_indexer_attention": (ctypes.c_int, [_BP, ctypes.POINTER(DsaDia), _P, _SZ, _P]),
    "dsa_indexer_projections_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "dsa_indexer_projections": (ctypes.c_int, [ctypes.POINTER(DsaProjections), _P, _SZ, _P]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_version": (ctypes.c_char_p, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          f"(python -m sparse_attention_14_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib.dsa_last_error().decode(errors="replace")
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")


def check(fn: str, status: int) -> None:
    if status != DSA_OK:
        raise DsaError(fn, status)
