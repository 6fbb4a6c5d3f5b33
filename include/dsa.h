/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek sparse-attention (DSA) decode path.
 *
 * The path (one decode step of a DSA layer):
 *   dsa_indexer_prolog      RoPE -> Hadamard -> per-token-head dynamic int8/fp8 quant of the
 *                           indexer query and of the new key rows (written into the key cache)
 *   dsa_indexer_scores      Lightning Indexer: int8/fp8 dot products of every query head against
 *                           every visible cached key, ReLU, head-weighted sum
 *   dsa_topk                per query token, the k highest-scoring visible positions
 *   dsa_sparse_attn_decode  attention of 128 (or 16) query heads over the selected 576-wide MLA
 *                           latent rows, online softmax in fp32, per-head attention sink
 *
 * Sources, cited by page title and section:
 *   [SFA] "NPU DeepSeek-V4 TileLang算子开发实践" (mooersco.com/news/996258), 1 Sparse Flash
 *         Attention: I/O tensors and algorithm steps 1-8.
 *   [AQ]  same page, 4 Activation Quantization, steps 1-3.
 *   [PRO] "NPU DeepSeek-V3.2-Exp PyPTO 融合算子开发优化实践" (jsqmd.com/news/787325), Indexer
 *         Prolog: formulas and quantization strategy.
 *   [LI]  same page, Lightning Indexer.   [DIA] same page, Deepseek Indexer Attention.
 *   [ARCH] ops-tilelang docs/architecture.md: public-API duties (validate every argument,
 *         compute launch parameters on the host, empty inputs are defined no-ops).
 *
 * Conventions for every call:
 *  - Pointers marked "device" are device (HBM) pointers; everything else is host memory.
 *  - The caller owns and allocates every buffer and keeps it alive until the stream has
 *    passed the work.  The library never allocates, frees or synchronizes, keeps no pointer
 *    after returning, and only enqueues kernels on `stream` (a hipStream_t; NULL = default).
 *  - Arrays are dense row-major.  Row pointers and row strides must be 16-byte aligned.
 *  - Validation failures return before any HIP call, write nothing, and leave a message in
 *    dsa_last_error().  A HIP launch error returns DSA_ERR_HIP with hipGetErrorString text.
 *    Values inside device arrays (indices, positions) are not checked: out-of-range values
 *    there are undefined behaviour, as for any kernel input.
 *  - A call with zero query tokens (or zero rows) is a successful no-op.
 *  - Calls on the same stream are ordered; calls that share a workspace buffer must not run
 *    concurrently on different streams.
 *  - Debug mode for read-before-write races: with the environment variable DSA_DEBUG_POISON=1
 *    (read at each call) the indexer, top-k and attention kernels fill their LDS with all-one
 *    bytes (NaN as a float, -1 as an integer) before use, and the calls fill the workspace
 *    regions their kernels write before reading (top-k candidate slots, attention split
 *    partials) the same way with an extra fill kernel on `stream`.  Results must not change;
 *    a read of data that was never written shows up as NaN, -1 or a wrong selection.  Slower;
 *    never for production.  The projection kernels (dynamic LDS) are not covered.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, inconsistent sizes   */
  DSA_ERR_UNSUPPORTED = 2,   /* a valid request outside the compiled set (head counts...)  */
  DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than *_workspace_size()       */
  DSA_ERR_HIP = 4            /* a HIP runtime error while enqueuing                        */
} dsa_status;

typedef enum dsa_dtype {
  DSA_I8 = 1,                /* int8 code                                                  */
  DSA_FP8_E4M3 = 2,          /* OCP fp8 E4M3FN code (max 448)                              */
  DSA_F16 = 3,
  DSA_BF16 = 4,
  DSA_F32 = 5
} dsa_dtype;

/*
 * A ragged decode batch over flat per-sequence caches.
 * Sequence b owns cache rows kv_start[b] .. kv_start[b] + L_b - 1 of the key cache and of the
 * latent KV cache; its query tokens are t = q_start[b] .. q_start[b+1]-1 (contiguous), and
 * token t sees its sequence's positions 0 .. q_pos[t] (causal; its own row included, since
 * the prolog writes a token's key row before the indexer runs -- [DIA] order).
 */
typedef struct dsa_batch {
  int32_t num_seqs;          /* B >= 0 (host)                                              */
  int32_t num_q;             /* T >= 0 (host), = q_start[B]                                */
  int32_t max_q_per_seq;     /* host: max_b (q_start[b+1] - q_start[b]), >= 1 if T > 0    */
  int32_t max_kv_len;        /* host: max_t q_pos[t] + 1 (score columns used, grid sizing) */
  const int32_t* q_start;    /* device [B+1], q_start[0] = 0, non-decreasing               */
  const int32_t* q_seq;      /* device [T]: the sequence of token t                        */
  const int32_t* q_pos;      /* device [T]: position p_t of token t, 0 <= p_t < max_kv_len */
  const int64_t* kv_start;   /* device [B]: first cache row of sequence b                  */
} dsa_batch;

/* ---------------------------------------------------------------- indexer prolog ---------- */
/*
 * [PRO] Indexer Prolog, from RoPE on:  codes, scale = DynamicQuant(Hadamard(RoPE(x)))
 * per (token, head) for the indexer query and per token for the indexer key ("C8" cache).
 * [AQ] steps 1-3 define the quantizer: fp32, amax over the row, scale = amax / 127 (int8) or
 * amax / 448 (e4m3), optional power-of-two rounding of the scale, codes = round-half-even(
 * clamp(x / scale, -max, max)); an all-zero row gets scale 0 and zero codes.
 * RoPE and the Hadamard are evaluated in fp64 and rounded once to fp32 before the quantizer.
 * The stored scale is the fp32 scale rounded to scale_dtype (fp16 per [PRO], or fp32).
 */
typedef struct dsa_prolog_cfg {
  int32_t H;                 /* query heads (key rows have one head)                      */
  int32_t D;                 /* head dim: 64 or 128                                       */
  int32_t rope_dim;          /* 0 = no RoPE, else even, rope_offset + rope_dim <= D       */
  int32_t rope_offset;       /* first rotated dim (64 = the last 64 dims of 128)          */
  int32_t rope_interleaved;  /* 0: pairs (i, i + rope_dim/2);  1: pairs (2i, 2i + 1)      */
  int32_t hadamard;          /* 1: right-multiply by the orthonormal Sylvester Hadamard_D */
  int32_t round_scale;       /* 1: scale rounded up to a power of two                    */
  dsa_dtype in_dtype;        /* DSA_BF16 or DSA_F32 activations                           */
  dsa_dtype code_dtype;      /* DSA_I8 or DSA_FP8_E4M3                                    */
  dsa_dtype scale_dtype;     /* DSA_F16 or DSA_F32                                        */
} dsa_prolog_cfg;

/*
 * Query part (num_q > 0): q_in device [num_q, H, D] in_dtype -> q_codes device [num_q, H, D]
 *   (1 byte each), q_scale device [num_q, H] scale_dtype.  q_cos/q_sin device
 *   [num_q, rope_dim/2] fp32 (ignored when rope_dim == 0).
 * Key part (num_k > 0): k_in device [num_k, D] in_dtype; row r is written to cache row
 *   k_slot[r] (device int64) of k_cache device [*, D] and k_scale device [*].  k_cos/k_sin
 *   device [num_k, rope_dim/2] fp32.
 * Either part may be empty (its pointers are then ignored).
 */
dsa_status dsa_indexer_prolog(const dsa_prolog_cfg* cfg,
                              int32_t num_q, const void* q_in, const float* q_cos,
                              const float* q_sin, void* q_codes, void* q_scale,
                              int32_t num_k, const void* k_in, const float* k_cos,
                              const float* k_sin, const int64_t* k_slot, void* k_cache,
                              void* k_scale, void* stream);

/* ---------------------------------------------------------------- lightning indexer ------- */
/*
 * [LI] (scores before TopK), operands from [PRO]:
 *   D[t,h,s] = sum_d q[t,h,d] k[s,d]                       (int32-exact for int8 codes)
 *   I[t,s]   = sum_h w[t,h] * ReLU(q_scale[t,h] * k_scale[s] * D[t,h,s]),   s = 0 .. p_t
 * evaluated as k_scale[s] * sum_h (w*q_scale)[t,h] * max(D[t,h,s], 0) in fp32 (the scales are
 * positive).  Supported: (H, D) in {(64,128), (8,64)}; codes DSA_I8 (int8 MFMA) or
 * DSA_FP8_E4M3 (codes widened exactly to bf16, bf16 MFMA, fp32 sums); scales DSA_F16 or
 * DSA_F32; w is fp16.
 *   q_codes  device [T, H, D]          q_scale device [T, H]        w device [T, H] fp16
 *   k_cache  device [N, D] (rows of every sequence, see dsa_batch)  k_scale device [N]
 *   scores   device [T, ld] fp32, ld >= max_kv_len, ld % 4 == 0.  Row t gets columns 0 .. p_t;
 *            columns past p_t are not written.
 */
dsa_status dsa_indexer_scores(const dsa_batch* batch, int32_t H, int32_t D,
                              dsa_dtype code_dtype, dsa_dtype scale_dtype,
                              const void* q_codes, const void* q_scale, const void* w,
                              const void* k_cache, const void* k_scale,
                              float* scores, int64_t ld, void* stream);

/*
 * The indexer half of a step in one call ([DIA] "Deepseek Indexer Attention": the indexer
 * prolog, the Lightning Indexer and its TopK run back to back).  The result equals
 *   dsa_indexer_prolog(cfg, T, q_in, q_cos, q_sin, q_codes, q_scale,
 *                      T, k_in, q_cos, q_sin, k_slot, k_cache, k_scale)
 *   dsa_indexer_topk(batch, cfg->H, cfg->D, cfg->code_dtype, cfg->scale_dtype, q_codes,
 *                    q_scale, w, k_cache, k_scale, k, scores, ld, idx, ws, ws_bytes)
 * with k_slot[t] = kv_start[q_seq[t]] + q_pos[t]: row t of k_in (device [T, D] in_dtype) is the
 * key of token t at its own position, rotated with the token's own table (q_cos/q_sin row t).
 * q_codes / q_scale are outputs here (the quantized query, as dsa_indexer_prolog writes it).
 * Schedule (chosen from the shapes; the results are identical): for decode batches with few
 * key spans per sequence (at most 4 query tokens per sequence, at most 16 spans of the
 * streaming indexer, rope_dim 0 or rope_offset % 8 == 0 and rope_dim % 16 == 0, the group's
 * raw query rows within 64 KiB at D = 128 / 80 KiB at D = 64) the prolog runs inside the
 * indexer kernel -- one launch fewer; otherwise as a launch of its own before it.  The
 * environment variable DSA_PROLOG_SCHEDULE=fused|separate overrides the choice where the form
 * is legal (testing).  (H, D) as for dsa_indexer_scores; flat caches only; q_in, k_in,
 * q_codes, q_scale and w 16-byte aligned.
 */
dsa_status dsa_indexer_prolog_topk(const dsa_prolog_cfg* cfg, const dsa_batch* batch,
                                   const void* q_in, const float* q_cos, const float* q_sin,
                                   const void* k_in, const void* w, void* q_codes, void* q_scale,
                                   void* k_cache, void* k_scale, int32_t k, float* scores,
                                   int64_t ld, int32_t* idx, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Test hook for the bit-exactness rule: the same int8 MFMA contraction as
 * dsa_indexer_scores, writing the raw int32 dot products dots[t, h, s] (device
 * [T, H, ld] int32, s = 0 .. p_t) instead of the weighted scores.  int8 codes only.
 */
dsa_status dsa_indexer_dots_i32(const dsa_batch* batch, int32_t H, int32_t D,
                                const int8_t* q_codes, const int8_t* k_cache,
                                int32_t* dots, int64_t ld, void* stream);

/*
 * Test hook for the choice of the fp8 indexer contraction ([PRO] quantization strategy: fp8
 * query and fp8 key cache).  c[i, j] = sum_d a[i, d] * b[j, d] over e4m3 codes, in fp32, on:
 *   DSA_CONTRACT_BF16     codes widened to bf16 (exact), v_mfma_f32_32x32x16_bf16 -- the
 *                         contraction dsa_indexer_scores uses for e4m3 codes;
 *   DSA_CONTRACT_FP8_K64  v_mfma_scale_f32_32x32x64_f8f6f4 on the codes, unit scales;
 *   DSA_CONTRACT_FP8_K16  v_mfma_f32_32x32x16_fp8_fp8 on the codes.
 *   a  device [m, d] e4m3 codes    b  device [n, d] e4m3 codes    c  device [m, n] fp32
 * m and n multiples of 32 (m < 2^21), d a multiple of 64 in [64, 4096]; a and b 16-byte
 * aligned.  Every path forms the same exact products and differs only in how it sums them.
 */
typedef enum dsa_contraction {
  DSA_CONTRACT_BF16 = 0,
  DSA_CONTRACT_FP8_K64 = 1,
  DSA_CONTRACT_FP8_K16 = 2
} dsa_contraction;
dsa_status dsa_e4m3_dots(const uint8_t* a, int32_t m, const uint8_t* b, int32_t n, int32_t d,
                         int32_t contraction, float* c, void* stream);

/* ---------------------------------------------------------------- upstream projections ---- */
/*
 * [PRO] Indexer Prolog formulas, the parts before RoPE: the indexer query's W8A8 linear
 * q_pre = DeQuant(q_a . w_qb) (q_a and w_qb int8, dequant factors FP16 per token and per output
 * channel: ((float)acc * q_a_scale[t]) * w_qb_scale[n], the int32 contraction exact, as in the
 * [AQ] page's Int8 GEMM), the indexer key's k_pre = LayerNorm(x . w_k) (over the D key values,
 * population variance, gamma, beta and eps given), and the head weights
 * weight = (x . w_proj) * weight_scale rounded to FP16.  q_pre and k_pre are fp32 and feed
 * dsa_indexer_prolog as its q_in ([T, H, D]) and k_in ([T, D]).
 * Decode shapes only: 1 <= num_q <= 8, H + D <= 256, q_rank a multiple of 256 with
 * num_q * q_rank <= 65536, hidden a multiple of 512 with num_q * hidden <= 131072.
 * Weights are stored as rows of their input dimension: w_qb [H*D, q_rank] int8, w_k [D, hidden]
 * and w_proj [H, hidden] bf16 (16-byte aligned).  The bf16 sums are fp32 in a fixed order.
 */
typedef struct dsa_projections {
  int32_t num_q;            /* T                                                          */
  int32_t q_rank;           /* contraction length of the query linear (e.g. 1536)         */
  int32_t hidden;           /* contraction length of the key and weight linears (7168)    */
  int32_t H, D;             /* indexer heads, head dim                                    */
  const int8_t* q_a;        /* device [T, q_rank] int8                                    */
  const void* q_a_scale;    /* device [T] fp16                                            */
  const int8_t* w_qb;       /* device [H*D, q_rank] int8                                  */
  const void* w_qb_scale;   /* device [H*D] fp16                                          */
  const void* x;            /* device [T, hidden] bf16                                    */
  const void* w_k;          /* device [D, hidden] bf16                                    */
  const float* ln_gamma;    /* device [D] fp32                                            */
  const float* ln_beta;     /* device [D] fp32                                            */
  float ln_eps;             /* >= 0                                                       */
  const void* w_proj;       /* device [H, hidden] bf16                                    */
  float weight_scale;
  float* q_pre;             /* device out [T, H*D] fp32                                   */
  float* k_pre;             /* device out [T, D] fp32                                     */
  void* weight;             /* device out [T, H] fp16                                     */
} dsa_projections;

/* Workspace bytes for dsa_indexer_projections (slice partial sums; no zero-fill needed). */
size_t dsa_indexer_projections_workspace_size(int32_t num_q, int32_t H, int32_t D);
/* Outside the decode shapes: DSA_ERR_UNSUPPORTED.  ws: device, 16-byte aligned. */
dsa_status dsa_indexer_projections(const dsa_projections* args, void* ws, size_t ws_bytes,
                                   void* stream);

/* ---------------------------------------------------------------- top-k ------------------- */
/*
 * [LI] TopK; [SFA] step 2 index convention.  For every token t: the k_eff = min(k, p_t + 1)
 * positions s in 0 .. p_t with the largest scores[t, s]; equal scores go to the lower
 * position; the set is written to idx[t, 0 .. k_eff) in ascending position order and
 * idx[t, k_eff .. k) = -1.  Selection is exact on the fp32 scores (radix select over
 * order-preserving keys; -0.0 equals +0.0).  1 <= k <= 2048.
 *   scores device [T, ld] fp32 (as written by dsa_indexer_scores), idx device [T, k] int32.
 *   ws: device workspace of at least dsa_topk_workspace_size(T, max_kv_len, k) bytes,
 *       256-byte aligned, ZERO-FILLED before its first use; every call leaves the part that
 *       must start at zero (the per-row histograms, at the start of the buffer) zeroed again,
 *       so a workspace is allocated and cleared once and then reused.  A workspace shared by
 *       calls of different shapes must be sized with the largest num_q and the largest
 *       max_kv_len among them (the other regions sit at the end of the buffer, past every
 *       call's histograms).  Calls sharing a workspace must not overlap.
 *       max_kv_len <= 262144.
 */
size_t dsa_topk_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k);
dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * [LI] the indexer followed by its TopK in one call: exactly dsa_indexer_scores (scores
 * written as documented there) and then dsa_topk on those scores, with the same arguments,
 * results, workspace contract and errors.  The top-k's first radix pass (a histogram of the
 * top 11 key bits per row) is accumulated by the indexer workgroups, which saves one pass
 * over the scores and one launch.  Batches of 256 or more query tokens (a prefill chunk) finish
 * each row's selection in one workgroup of their own (one launch after the indexer).
 */
dsa_status dsa_indexer_topk(const dsa_batch* batch, int32_t H, int32_t D,
                            dsa_dtype code_dtype, dsa_dtype scale_dtype,
                            const void* q_codes, const void* q_scale, const void* w,
                            const void* k_cache, const void* k_scale, float* scores,
                            int64_t ld, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------- sparse attention -------- */
/*
 * [SFA] steps 1-8 with the attention sink of step 7 read as a per-head logit that joins the
 * softmax denominator:  for J_t = { idx[t, j] != -1 },
 *   z_j = scale * q[t,h,:576] . kv[row_j, :576],   row_j = kv_start[seq(t)] + idx[t, j]
 *   o[t,h,:] = sum_j e^{z_j} kv[row_j, :512] / (sum_j e^{z_j} + e^{sink[h]})
 * (MLA absorbed form: one latent KV head of 576 = 512 nope + 64 rope columns shared by all
 * query heads; the value is the first 512 columns).  Empty J_t gives 0.  QK^T and PV run on
 * bf16 MFMA with fp32 accumulation; the softmax is online in fp32; probabilities enter PV
 * as bf16.
 *   q      device [T, Hq, 576] bf16         Hq in {16, 128}
 *   kv     device rows of 576 bf16, row r at kv + r * kv_row_stride elements
 *          (kv_row_stride >= 576, multiple of 8)
 *   idx    device [T, k] int32 (positions within the token's sequence, -1 = skip), 1 <= k <= 2048
 *   sink   device [Hq] fp32, or NULL for no sink
 *   out    device [T, Hq, 512] bf16
 *   ws:    device workspace of at least dsa_sparse_attn_workspace_size(T, Hq, k) bytes,
 *          256-byte aligned (split-K partials); may be NULL when that size is 0.
 * Schedule (shapes only): the selection is split over workgroups of 32 heads so that a batch
 * fills the GPU; batches that need no split (one per token) on flat caches with Hq a multiple
 * of 64 and at least 256 workgroups of 64 heads run a kernel with 64 heads per workgroup
 * instead, with bit-identical results.  DSA_SFA_H64=0 in the environment keeps the 32-head
 * kernel (tests).
 */
size_t dsa_sparse_attn_workspace_size(int32_t num_q, int32_t Hq, int32_t k);
dsa_status dsa_sparse_attn_decode(const dsa_batch* batch, int32_t Hq, const void* q,
                                  const void* kv, int64_t kv_row_stride, const int32_t* idx,
                                  int32_t k, const float* sink, float scale, void* out,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * The two stages of dsa_sparse_attn_decode, for callers that schedule them apart (same
 * arguments, validation and errors).  [SFA] steps 1-6 run per split of the selection:
 * dsa_sparse_attn_split writes each split's softmax-weighted average (bf16) with its running
 * max and sum (fp32) into ws -- or, when the call needs no workspace (dsa_sparse_attn_workspace_size == 0),
 * finishes steps 7-8 itself and writes out.  dsa_sparse_attn_merge then applies [SFA] steps
 * 7-8 over the splits (log-sum-exp merge, sink, bf16 store to out); it reads only ws and sink,
 * and is a no-op when the workspace size is 0.  Running split then merge on one stream gives
 * exactly the result of dsa_sparse_attn_decode.
 */
dsa_status dsa_sparse_attn_split(const dsa_batch* batch, int32_t Hq, const void* q,
                                 const void* kv, int64_t kv_row_stride, const int32_t* idx,
                                 int32_t k, const float* sink, float scale, void* out,
                                 void* ws, size_t ws_bytes, void* stream);
dsa_status dsa_sparse_attn_merge(const dsa_batch* batch, int32_t Hq, int32_t k,
                                 const float* sink, void* out, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc): dsa_sparse_attn_decode with the same arguments, results and errors except
 * the workspace, which is a fixed scratch array of 12 MiB that the library holds on every GPU it
 * runs on (from the first call on that GPU until the process ends).  Calls whose split partials
 * (dsa_sparse_attn_workspace_size) exceed 12 MiB return DSA_ERR_UNSUPPORTED before any launch;
 * decode batches of up to 32 query tokens at 128 heads and k <= 2048 fit.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (concurrent streams) race.  Nothing
 * in the scratch needs clearing between calls.
 */
dsa_status dsa_sparse_attn_decode_noalloc(const dsa_batch* batch, int32_t Hq, const void* q,
                                          const void* kv, int64_t kv_row_stride,
                                          const int32_t* idx, int32_t k, const float* sink,
                                          float scale, void* out, void* stream);

/* ---------------------------------------------------------------- indexer attention ------- */
/*
 * [DIA] "Deepseek Indexer Attention": the indexer prolog, the Lightning Indexer, its TopK and
 * the Sparse Flash Attention of a decode step back to back, in one call.  The results equal
 *   dsa_indexer_prolog_topk(prolog, batch, q_in, q_cos, q_sin, k_in, w, q_codes, q_scale,
 *                           k_cache, k_scale, k, scores, ld, idx, ...)      when prolog != NULL
 *   dsa_indexer_topk(batch, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
 *                    k_scale, scores, ld, k, idx, ...)                     when prolog == NULL
 * followed by
 *   dsa_sparse_attn_decode(batch, Hq, q, kv, kv_row_stride, idx, k, sink, scale, out, ...)
 * with the argument meanings, layouts and errors of those calls (flat caches only).  With a
 * prolog, H, D, code_dtype and scale_dtype must equal the prolog's.  Every argument is checked
 * before the first launch.
 * Schedule (chosen from the shapes; the results are identical): for at most 32 query tokens on
 * rows of at most 131072 positions the attention workgroups resolve their own slice of the
 * selection from the state the top-k's select pass leaves in the workspace (the k-th key of the
 * row by two more radix digits over the candidates, then their slots of the ascending
 * selection), which takes the top-k's separate finalize launch out of the step; idx is written
 * by those workgroups.  Other decode batches run the finalize pass before the attention, and
 * batches of 256 or more tokens the row top-k.  DSA_DIA_SCHEDULE=slice|finalize overrides the
 * choice below 256 tokens (testing).
 *   ws: device workspace of at least dsa_indexer_attention_workspace_size(T, max_kv_len, k, Hq)
 *       bytes, 256-byte aligned, with the contract of the top-k workspace (zero-filled before
 *       its first use, left so by every call; sized for the largest num_q and max_kv_len of the
 *       calls that share it; calls sharing it must not overlap).
 */
typedef struct dsa_dia {
  const dsa_prolog_cfg* prolog;  /* NULL: q_codes, q_scale and the batch's new key rows are   */
                                 /* already quantized inputs                                */
  const void* q_in;              /* prolog only: device [T, H, D] in_dtype                   */
  const float* q_cos;            /* prolog with rope_dim > 0: device [T, rope_dim / 2] fp32  */
  const float* q_sin;
  const void* k_in;              /* prolog only: device [T, D] in_dtype, token t's new key    */
                                 /* row (written at kv_start[seq(t)] + q_pos[t])              */
  int32_t H, D;                  /* indexer heads and head dim                               */
  dsa_dtype code_dtype, scale_dtype;
  void* q_codes;                 /* device [T, H, D] codes (written by the prolog)            */
  void* q_scale;                 /* device [T, H] (written by the prolog)                     */
  const void* w;                 /* device [T, H] fp16 head weights                           */
  void* k_cache;                 /* device [N, D] key codes                                   */
  void* k_scale;                 /* device [N] key scales                                     */
  float* scores;                 /* device [T, ld] fp32 indexer scores (output)               */
  int64_t ld;
  int32_t k;                     /* top-k size, 1 .. 2048                                     */
  int32_t* idx;                  /* device [T, k] int32 selection (output)                    */
  int32_t Hq;                    /* attention heads, 16 or 128                                */
  const void* q;                 /* device [T, Hq, 576] bf16                                  */
  const void* kv;                /* device latent rows of 576 bf16                            */
  int64_t kv_row_stride;
  const float* sink;             /* device [Hq] fp32, or NULL                                 */
  float scale;
  void* out;                     /* device [T, Hq, 512] bf16 (output)                         */
} dsa_dia;
size_t dsa_indexer_attention_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k, int32_t Hq);
dsa_status dsa_indexer_attention(const dsa_batch* batch, const dsa_dia* args, void* ws,
                                 size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- paged caches ----------- */
/*
 * [LI] the Page Attention layout of the caches: a sequence's rows are stored in fixed-size
 * blocks anywhere in the cache, listed by a block table.  Position p of sequence b lives in
 * cache row  block_table[b * blocks_per_seq + p / block_size] * block_size + p % block_size
 * (of k_cache / k_scale for the indexer, of kv for the attention).  The pages use blocks of
 * 128 rows.  The paged calls take every other argument of their flat counterparts with the
 * same meaning, results and errors; batch->kv_start is not read (may be NULL).
 *   block_table     device [num_seqs, blocks_per_seq] int32, entries in [0, num_blocks)
 *   blocks_per_seq  >= ceil(max_kv_len / block_size); <= 2048 for the attention call (its
 *                   workgroups stage a sequence's table in on-chip memory)
 *   block_size      a power of two in [16, 1024]
 *   num_blocks      physical blocks in the cache; num_blocks * block_size rows must span
 *                   < 4 GiB of k_cache codes and of kv rows (32-bit gather offsets)
 * The caller owns the table; entries past a sequence's last block are not read.
 */
typedef struct dsa_paging {
  const int32_t* block_table;
  int32_t blocks_per_seq;
  int32_t block_size;
  int32_t num_blocks;
} dsa_paging;

/* dsa_indexer_scores with k_cache / k_scale rows addressed through the block table. */
dsa_status dsa_indexer_scores_paged(const dsa_batch* batch, const dsa_paging* paging, int32_t H,
                                    int32_t D, dsa_dtype code_dtype, dsa_dtype scale_dtype,
                                    const void* q_codes, const void* q_scale, const void* w,
                                    const void* k_cache, const void* k_scale, float* scores,
                                    int64_t ld, void* stream);
/* dsa_indexer_topk with k_cache / k_scale rows addressed through the block table. */
dsa_status dsa_indexer_topk_paged(const dsa_batch* batch, const dsa_paging* paging, int32_t H,
                                  int32_t D, dsa_dtype code_dtype, dsa_dtype scale_dtype,
                                  const void* q_codes, const void* q_scale, const void* w,
                                  const void* k_cache, const void* k_scale, float* scores,
                                  int64_t ld, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                                  void* stream);
/* dsa_sparse_attn_decode with kv rows addressed through the block table (kv_row_stride and
 * the workspace as there). */
dsa_status dsa_sparse_attn_decode_paged(const dsa_batch* batch, const dsa_paging* paging,
                                        int32_t Hq, const void* q, const void* kv,
                                        int64_t kv_row_stride, const int32_t* idx, int32_t k,
                                        const float* sink, float scale, void* out, void* ws,
                                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- misc -------------------- */
/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* dsa_last_error(void);
/* Library version string. */
const char* dsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
