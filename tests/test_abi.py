"""CPU checks of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments (or no-ops on empty batches) before making any HIP call -- no GPU needed."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _lib():
    from sparse_attention_14_amd import _lib
    return _lib


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return {m.group(1): m.group(2) for m in re.finditer(r"\b(dsa_\w+)\s*\(([^;{]*)\)\s*;", txt)}


def test_library_exports_every_declared_symbol():
    L = _lib()
    decl = _declared()
    assert {"dsa_indexer_prolog", "dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn_decode"} <= set(decl)
    for name in decl:
        assert hasattr(L.lib, name), name
    out = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    for name in decl:
        assert re.search(rf"\bT {name}\b", out), f"{name} not exported"


def test_ctypes_signatures_match_header_arity():
    L = _lib()
    decl = _declared()
    assert set(decl) == set(L.SIGNATURES)
    for name, args in decl.items():
        n = 0 if args.strip() in ("", "void") else args.count(",") + 1
        assert n == len(L.SIGNATURES[name][1]), name


def test_version_and_error_text():
    L = _lib()
    assert b"gfx950" in L.lib.dsa_version()
    assert isinstance(L.lib.dsa_last_error(), bytes)


def _batch(T=8, B=4, mq=2, ml=65536):
    L = _lib()
    p = ctypes.c_void_p(0x1000)          # never dereferenced: validation returns first
    return L.DsaBatch(B, T, mq, ml, p, p, p, p)


def test_validation_errors_before_any_device_call():
    L = _lib()
    lib = L.lib
    b = _batch()
    P = ctypes.c_void_p(0x1000)
    # NULL batch
    assert lib.dsa_indexer_scores(None, 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, None) == L.DSA_ERR_INVALID_ARG
    assert b"batch is NULL" in lib.dsa_last_error()
    # unsupported head shape
    assert lib.dsa_indexer_scores(ctypes.byref(b), 32, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, None) == L.DSA_ERR_UNSUPPORTED
    # ld too small
    assert lib.dsa_indexer_scores(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 100, None) == L.DSA_ERR_INVALID_ARG
    # null data pointer
    assert lib.dsa_indexer_scores(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, None, P, P, P, P, P, 65536, None) == L.DSA_ERR_INVALID_ARG
    # misaligned q_scale / w rows (an odd storage offset of a torch view)
    Q2 = ctypes.c_void_p(0x1002)
    assert lib.dsa_indexer_scores(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, P, Q2, P, P, P, P, 65536, None) == L.DSA_ERR_INVALID_ARG
    assert b"aligned" in lib.dsa_last_error()
    assert lib.dsa_indexer_scores(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, P, P, Q2, P, P, P, 65536, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_topk(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, P, P, Q2, P, P, P, 65536, 2048, P, P, 1 << 30, None) == L.DSA_ERR_INVALID_ARG
    # top-k: k out of range, workspace too small
    assert lib.dsa_topk(ctypes.byref(b), P, 65536, 4096, P, P, 1 << 30, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(ctypes.byref(b), P, 65536, 2048, P, P, 16, None) == L.DSA_ERR_WORKSPACE
    # fused indexer + top-k: the top-k checks run first, then the indexer's
    assert lib.dsa_indexer_topk(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, 2048, P, P, 16, None) == L.DSA_ERR_WORKSPACE
    assert lib.dsa_indexer_topk(ctypes.byref(b), 32, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, 2048, P, P, 1 << 30, None) == L.DSA_ERR_UNSUPPORTED
    # sparse attention: unsupported heads, bad stride, missing workspace
    assert lib.dsa_sparse_attn_decode(ctypes.byref(b), 64, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, None, 0, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_sparse_attn_decode(ctypes.byref(b), 128, P, P, 500, P, 2048, None, ctypes.c_float(0.04), P, None, 0, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_attn_decode(ctypes.byref(b), 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, None, 0, None) == L.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_attn_decode(ctypes.byref(b), 128, P, P, 576, P, 2048, None, ctypes.c_float(-1.0), P, None, 0, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_attn_split(ctypes.byref(b), 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, None, 0, None) == L.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_attn_merge(ctypes.byref(b), 64, 2048, None, P, P, 1 << 30, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_sparse_attn_merge(ctypes.byref(b), 128, 2048, None, P, None, 0, None) == L.DSA_ERR_WORKSPACE
    # prolog: bad D, bad rope range, missing pointers
    cfg = L.DsaPrologCfg(64, 96, 0, 0, 0, 0, 0, L.DSA_BF16, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog(ctypes.byref(cfg), 8, P, None, None, P, P, 0, None, None, None, None, None, None, None) == L.DSA_ERR_UNSUPPORTED
    cfg = L.DsaPrologCfg(64, 128, 64, 96, 0, 1, 0, L.DSA_BF16, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog(ctypes.byref(cfg), 8, P, P, P, P, P, 0, None, None, None, None, None, None, None) == L.DSA_ERR_INVALID_ARG
    cfg = L.DsaPrologCfg(64, 128, 64, 64, 0, 1, 0, L.DSA_BF16, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog(ctypes.byref(cfg), 8, P, None, None, P, P, 0, None, None, None, None, None, None, None) == L.DSA_ERR_INVALID_ARG
    # fused prolog + indexer + top-k: cfg checks first, then the fused form's own limits, then top-k
    assert lib.dsa_indexer_prolog_topk(None, ctypes.byref(b), P, P, P, P, P, P, P, P, P, 2048, P, 65536, P, P, 1 << 30, None) == L.DSA_ERR_INVALID_ARG
    cfg = L.DsaPrologCfg(32, 128, 64, 64, 0, 1, 0, L.DSA_BF16, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog_topk(ctypes.byref(cfg), ctypes.byref(b), P, P, P, P, P, P, P, P, P, 2048, P, 65536, P, P, 1 << 30, None) == L.DSA_ERR_UNSUPPORTED
    assert b"not compiled" in lib.dsa_last_error()
    cfg = L.DsaPrologCfg(64, 128, 64, 64, 0, 1, 0, 99, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog_topk(ctypes.byref(cfg), ctypes.byref(b), P, P, P, P, P, P, P, P, P, 2048, P, 65536, P, P, 1 << 30, None) == L.DSA_ERR_UNSUPPORTED
    cfg = L.DsaPrologCfg(64, 128, 64, 64, 0, 1, 0, L.DSA_BF16, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog_topk(ctypes.byref(cfg), ctypes.byref(b), P, P, P, P, P, P, P, P, P, 2048, P, 65536, P, P, 16, None) == L.DSA_ERR_WORKSPACE
    assert lib.dsa_indexer_prolog_topk(ctypes.byref(cfg), ctypes.byref(b), None, P, P, P, P, P, P, P, P, 2048, P, 65536, P, P, 1 << 30, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_prolog_topk(ctypes.byref(cfg), ctypes.byref(b), ctypes.c_void_p(0x1008), P, P, P, P, P, P, P, P, 2048, P, 65536, P, P, 1 << 30, None) == L.DSA_ERR_INVALID_ARG
    # fp8 contraction hook: unknown path, ragged sizes, bad depth, misaligned operand; empty is a no-op
    assert lib.dsa_e4m3_dots(P, 32, P, 32, 128, 3, P, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_e4m3_dots(P, 33, P, 32, 128, 0, P, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_e4m3_dots(P, 32, P, 32, 96, 1, P, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_e4m3_dots(ctypes.c_void_p(0x1008), 32, P, 32, 128, 2, P, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_e4m3_dots(None, 0, None, 32, 128, 0, None, None) == L.DSA_OK


def test_empty_batches_are_noops_without_device():
    L = _lib()
    lib = L.lib
    b = _batch(T=0, B=0, mq=0, ml=0)
    assert lib.dsa_indexer_scores(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, None, None, None, None, None, None, 0, None) == L.DSA_OK
    assert lib.dsa_topk(ctypes.byref(b), None, 0, 2048, None, None, 0, None) == L.DSA_OK
    assert lib.dsa_indexer_topk(ctypes.byref(b), 64, 128, L.DSA_I8, L.DSA_F16, None, None, None, None, None, None, 0, 2048, None, None, 0, None) == L.DSA_OK
    pcfg = L.DsaPrologCfg(64, 128, 0, 0, 0, 0, 0, L.DSA_F32, L.DSA_I8, L.DSA_F16)
    assert lib.dsa_indexer_prolog_topk(ctypes.byref(pcfg), ctypes.byref(b), None, None, None, None, None, None, None, None, None, 2048, None, 0, None, None, 0, None) == L.DSA_OK
    assert lib.dsa_sparse_attn_decode(ctypes.byref(b), 128, None, None, 576, None, 2048, None, ctypes.c_float(0.04), None, None, 0, None) == L.DSA_OK
    cfg = L.DsaPrologCfg(64, 128, 64, 64, 0, 1, 0, L.DSA_BF16, L.DSA_FP8_E4M3, L.DSA_F16)
    assert lib.dsa_indexer_prolog(ctypes.byref(cfg), 0, None, None, None, None, None, 0, None, None, None, None, None, None, None) == L.DSA_OK
    assert lib.dsa_topk_workspace_size(0, 10, 5) == 0 and lib.dsa_sparse_attn_workspace_size(0, 128, 5) == 0


def test_workspace_sizes():
    L = _lib()
    # decode at 8 tokens spreads each token's 2048 keys over several workgroups
    assert L.lib.dsa_sparse_attn_workspace_size(8, 128, 2048) > 0
    # a large batch needs no split partials
    assert L.lib.dsa_sparse_attn_workspace_size(4096, 128, 2048) == 0
    # top-k: at least the per-row histograms (4 shards of 2048 bins); grows with the batch and
    # the row length; 256-byte multiples; nothing for an empty batch
    sz = L.lib.dsa_topk_workspace_size
    assert sz(8, 65536, 2048) >= 8 * 4 * 2048 * 4
    assert sz(16, 65536, 2048) > sz(8, 65536, 2048) and sz(8, 131072, 2048) > sz(8, 65536, 2048)
    assert sz(3, 65536, 2048) % 256 == 0 and sz(0, 65536, 2048) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    from sparse_attention_14_amd import dsa
    with pytest.raises(ValueError):
        dsa._need(torch.zeros(3), "x", torch.float32)


def test_paged_validation_before_any_device_call():
    L = _lib()
    lib = L.lib
    b = _batch()
    P = ctypes.c_void_p(0x1000)
    PP = lambda bs=128, bps=512, nb=2048, tab=P: L.DsaPaging(tab, bps, bs, nb)
    big = 1 << 30
    # NULL paging
    assert lib.dsa_sparse_attn_decode_paged(ctypes.byref(b), None, 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, P, big, None) == L.DSA_ERR_INVALID_ARG
    assert b"paging is NULL" in lib.dsa_last_error()
    assert lib.dsa_indexer_topk_paged(ctypes.byref(b), None, 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, 2048, P, P, big, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores_paged(ctypes.byref(b), None, 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, None) == L.DSA_ERR_INVALID_ARG
    # block size not a power of two / out of range
    for bs in (100, 8, 2048):
        pg = PP(bs=bs)
        assert lib.dsa_sparse_attn_decode_paged(ctypes.byref(b), ctypes.byref(pg), 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, P, big, None) == L.DSA_ERR_INVALID_ARG
        assert lib.dsa_indexer_scores_paged(ctypes.byref(b), ctypes.byref(pg), 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, None) == L.DSA_ERR_INVALID_ARG
    # too few blocks per sequence for max_kv_len (65536), NULL table, no blocks
    for pg in (PP(bps=100), PP(tab=None), PP(nb=0)):
        assert lib.dsa_indexer_topk_paged(ctypes.byref(b), ctypes.byref(pg), 64, 128, L.DSA_I8, L.DSA_F16, P, P, P, P, P, P, 65536, 2048, P, P, big, None) == L.DSA_ERR_INVALID_ARG
    # the attention stages at most 2048 table entries per sequence; caches must span < 4 GiB
    pg = PP(bs=16, bps=4096)
    assert lib.dsa_sparse_attn_decode_paged(ctypes.byref(b), ctypes.byref(pg), 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, P, big, None) == L.DSA_ERR_UNSUPPORTED
    pg = PP(nb=1 << 20)
    assert lib.dsa_sparse_attn_decode_paged(ctypes.byref(b), ctypes.byref(pg), 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, P, big, None) == L.DSA_ERR_UNSUPPORTED
    # a paged batch may leave kv_start NULL; an empty one is a no-op
    nb = _batch()
    nb.kv_start = None
    pg = PP(bps=100)
    assert lib.dsa_sparse_attn_decode_paged(ctypes.byref(nb), ctypes.byref(pg), 128, P, P, 576, P, 2048, None, ctypes.c_float(0.04), P, P, big, None) == L.DSA_ERR_INVALID_ARG
    assert b"blocks_per_seq" in lib.dsa_last_error()
    e = _batch(T=0, B=0, mq=0, ml=0)
    pg = PP()
    assert lib.dsa_indexer_topk_paged(ctypes.byref(e), ctypes.byref(pg), 64, 128, L.DSA_I8, L.DSA_F16, None, None, None, None, None, None, 0, 2048, None, None, 0, None) == L.DSA_OK
    assert lib.dsa_sparse_attn_decode_paged(ctypes.byref(e), ctypes.byref(pg), 128, None, None, 576, None, 2048, None, ctypes.c_float(0.04), None, None, 0, None) == L.DSA_OK


def test_projections_validation_before_any_device_call():
    L = _lib()
    lib = L.lib
    P = 0x1000
    def args(T=8, R=1536, hidden=7168, H=64, D=128, null=False):
        return L.DsaProjections(T, R, hidden, H, D, P, P, P, P, P, P, None if null else P, P, 1e-6,
                                P, 0.125, P, P, P)
    big = 1 << 30
    assert lib.dsa_indexer_projections(None, ctypes.c_void_p(P), big, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_projections(ctypes.byref(args(T=9)), ctypes.c_void_p(P), big, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_indexer_projections(ctypes.byref(args(R=1000)), ctypes.c_void_p(P), big, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_indexer_projections(ctypes.byref(args(hidden=7000)), ctypes.c_void_p(P), big, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_indexer_projections(ctypes.byref(args(H=200)), ctypes.c_void_p(P), big, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_indexer_projections(ctypes.byref(args(null=True)), ctypes.c_void_p(P), big, None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_projections(ctypes.byref(args()), ctypes.c_void_p(P), 16, None) == L.DSA_ERR_WORKSPACE
    assert lib.dsa_indexer_projections(ctypes.byref(args(T=0)), None, 0, None) == L.DSA_OK
    assert lib.dsa_indexer_projections_workspace_size(8, 64, 128) >= 8 * 8 * 192 * 4
    assert lib.dsa_indexer_projections_workspace_size(0, 64, 128) == 0


def _dia(L, **kw):
    P = ctypes.c_void_p(0x1000)
    f = dict(prolog=None, q_in=None, q_cos=None, q_sin=None, k_in=None, H=64, D=128,
             code_dtype=L.DSA_I8, scale_dtype=L.DSA_F16, q_codes=P, q_scale=P, w=P, k_cache=P,
             k_scale=P, scores=P, ld=65536, k=2048, idx=P, Hq=128, q=P, kv=P, kv_row_stride=576,
             sink=P, scale=0.04, out=P)
    f.update(kw)
    return L.DsaDia(**f)


def test_indexer_attention_validation_before_any_device_call():
    L = _lib()
    lib = L.lib
    b = _batch()
    ws = ctypes.c_void_p(0x100000)
    need = lib.dsa_indexer_attention_workspace_size(8, 65536, 2048, 128)
    # the workspace holds the top-k's part and at least the attention's partials
    assert need >= lib.dsa_topk_workspace_size(8, 65536, 2048) + lib.dsa_sparse_attn_workspace_size(8, 128, 2048)
    # its bound on the partials grows with the batch (a buffer sized for the largest batch serves
    # every smaller one), though the attention's own partials do not
    for T in range(1, 64):
        assert lib.dsa_indexer_attention_workspace_size(T + 1, 65536, 2048, 128) >= \
            lib.dsa_indexer_attention_workspace_size(T, 65536, 2048, 128)
        assert lib.dsa_indexer_attention_workspace_size(T, 65536, 2048, 128) >= \
            lib.dsa_topk_workspace_size(T, 65536, 2048) + lib.dsa_sparse_attn_workspace_size(T, 128, 2048)
    call = lambda d, nbytes=need, w=ws, batch=b: lib.dsa_indexer_attention(ctypes.byref(batch), ctypes.byref(d), w, nbytes, None)
    assert lib.dsa_indexer_attention(ctypes.byref(b), None, ws, need, None) == L.DSA_ERR_INVALID_ARG
    assert call(_dia(L), need - 256) == L.DSA_ERR_WORKSPACE
    assert call(_dia(L), need, None) == L.DSA_ERR_WORKSPACE
    assert call(_dia(L), need, ctypes.c_void_p(0x100080)) == L.DSA_ERR_INVALID_ARG      # misaligned
    assert call(_dia(L, k=0)) == L.DSA_ERR_UNSUPPORTED                                      # top-k
    assert call(_dia(L, H=32)) == L.DSA_ERR_UNSUPPORTED                                     # indexer
    assert call(_dia(L, q_codes=None)) == L.DSA_ERR_INVALID_ARG
    assert call(_dia(L, Hq=64)) == L.DSA_ERR_UNSUPPORTED                                    # attention
    assert call(_dia(L, out=None)) == L.DSA_ERR_INVALID_ARG
    assert call(_dia(L, kv=ctypes.c_void_p(0x1008))) == L.DSA_ERR_INVALID_ARG
    # with a prolog: its dims and dtypes must match the indexer's
    cfg = L.DsaPrologCfg(64, 128, 64, 64, 0, 1, 0, L.DSA_BF16, L.DSA_I8, L.DSA_F16)
    assert call(_dia(L, prolog=ctypes.pointer(cfg), q_in=ctypes.c_void_p(0x1000), k_in=ctypes.c_void_p(0x1000),
                     q_cos=ctypes.c_void_p(0x1000), q_sin=ctypes.c_void_p(0x1000), scale_dtype=L.DSA_F32)) == L.DSA_ERR_INVALID_ARG
    assert b"must equal the prolog" in lib.dsa_last_error()
    assert call(_dia(L, prolog=ctypes.pointer(cfg), q_in=None, k_in=ctypes.c_void_p(0x1000),
                     q_cos=ctypes.c_void_p(0x1000), q_sin=ctypes.c_void_p(0x1000))) == L.DSA_ERR_INVALID_ARG
    # an empty batch is a no-op that needs no workspace
    e = _batch(T=0, B=0, mq=0, ml=0)
    assert call(_dia(L), 0, None, e) == L.DSA_OK
    assert lib.dsa_indexer_attention_workspace_size(0, 65536, 2048, 128) == 0
