// Indexer prolog on gfx950: RoPE -> Sylvester Hadamard -> per-row dynamic int8 / e4m3 quant.
//
// [PRO] "Indexer Prolog" (jsqmd.com/news/787325): q and the cache key are quantized per
// token-head after Hadamard(RoPE(.)); dequant factors are FP16.  [AQ] "Activation
// Quantization" (mooersco.com/news/996258, section 4, steps 1-3): fp32, amax, scale =
// amax / 127, round(clamp(x / scale)).
//
// One wave per row (a (token, head) query row or a key row).  The prolog moves < 1 MB per
// decode step, so it is latency-bound: the kernel keeps every row in registers, does the
// RoPE pair exchange and the 7 Hadamard butterfly stages with cross-lane shuffles in fp64
// (cheap at this size, and it leaves a single rounding to fp32 before the fp32 quantizer),
// and writes codes with one coalesced store per lane.
#include "common.h"

namespace dsa {

struct PrologArgs {
  int H, D, rope_dim, rope_offset, rope_interleaved, hadamard, round_scale;
  int in_bf16, code_fp8, scale_f16;
  int num_q, num_k;
  const void* q_in; const float* q_cos; const float* q_sin; void* q_codes; void* q_scale;
  const void* k_in; const float* k_cos; const float* k_sin; const int64_t* k_slot;
  void* k_cache; void* k_scale;
  // k_slot == NULL: key row r is token r's own key, at row kv_start[q_seq[r]] + q_pos[r]
  const int32_t* q_seq; const int32_t* q_pos; const int64_t* kv_start;
};

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  return __shfl_xor(v, m, kWave);
}

// EPL = elements per lane (D / 64).  Lane l holds elements l*EPL .. l*EPL + EPL - 1.  BF16: the
// input rows are bf16 (else fp32).
template <int EPL, bool BF16>
__global__ void __launch_bounds__(256) prolog_kernel(PrologArgs a) {
  const int lane = threadIdx.x & 63;
  // the wave's row, in scalar registers (every branch on it below is wave-uniform)
  const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long nq_rows = (long)a.num_q * a.H;
  if (row >= nq_rows + a.num_k) return;
  const bool is_q = row < nq_rows;
  const long r_in = is_q ? row : row - nq_rows;           // input row
  const long tab = is_q ? row / a.H : r_in;               // cos/sin row (token or key row)
  const int D = EPL * 64;
  const void* src = is_q ? a.q_in : a.k_in;

  // Every load of the row is issued before the first wait: its elements (raw bf16 or fp32 bits,
  // one load per lane when the row is aligned for it), its rotary table entries and, for a key
  // row, where it goes.
  const long off = r_in * D + lane * EPL;
  const bool wide = EPL == 2 && ((uintptr_t)src & (BF16 ? 3u : 7u)) == 0;   // wave-uniform
  uint2 w = {0u, 0u};
  if constexpr (BF16) {                                   // w.x = both elements (element 0 low)
    if (wide) w.x = ((const uint32_t*)src)[off / 2];
    else w.x = (uint32_t)((const u16*)src)[off] | (EPL == 2 ? (uint32_t)((const u16*)src)[off + EPL - 1] << 16 : 0u);
  } else {
    if (wide) w = ((const uint2*)src)[off / 2];
    else {
      w.x = ((const uint32_t*)src)[off];
      if (EPL == 2) w.y = ((const uint32_t*)src)[off + EPL - 1];
    }
  }
  long drow = 0;                                          // destination row of a key row
  if (!is_q) drow = a.k_slot ? a.k_slot[r_in] : a.kv_start[a.q_seq[r_in]] + a.q_pos[r_in];

  // RoPE on [rope_offset, rope_offset + rope_dim): partner of element i is i +- rope_dim/2
  // (or i ^ 1 when interleaved).  Products of fp32 values are exact in fp64, so each output
  // is rounded once.
  const bool rope = a.rope_dim > 0;
  const int half = a.rope_dim >> 1;
  int plane[EPL], pe[EPL];
  bool first[EPL], in[EPL];
  float cv[EPL], sv[EPL];
  if (rope) {
    const float* cs = is_q ? a.q_cos : a.k_cos;
    const float* sn = is_q ? a.q_sin : a.k_sin;
    int pair[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane * EPL + e;
      const int rel = i - a.rope_offset;
      in[e] = rel >= 0 && rel < a.rope_dim;
      int partner;
      if (a.rope_interleaved) { partner = i ^ 1; pair[e] = rel >> 1; first[e] = (rel & 1) == 0; }
      else {
        first[e] = rel < half;
        partner = first[e] ? i + half : i - half;
        pair[e] = first[e] ? rel : rel - half;
      }
      if (!in[e]) { partner = i; pair[e] = 0; }
      plane[e] = partner / EPL; pe[e] = partner % EPL;
      cv[e] = cs[tab * half + pair[e]];                   // pair 0 for elements outside the range
      sv[e] = sn[tab * half + pair[e]];
    }
  }
  double x[EPL];
  if constexpr (BF16) {
    x[0] = (double)bf16_to_f32((u16)w.x);
    if (EPL == 2) x[EPL - 1] = (double)bf16_to_f32((u16)(w.x >> 16));
  } else {
    x[0] = (double)__uint_as_float(w.x);
    if (EPL == 2) x[EPL - 1] = (double)__uint_as_float(w.y);
  }
  if (rope) {
    double pv[EPL];
    // gather every partner value before any element is rotated
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      pv[e] = 0.0;
#pragma unroll
      for (int f = 0; f < EPL; ++f) {
        const double v = __shfl(x[f], plane[e], kWave);
        if (f == pe[e]) pv[e] = v;
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if (in[e]) {
        const double c = (double)cv[e];
        const double sng = (double)sv[e];
        // first of the pair: x1 c - x2 s ; second: x2 c + x1 s
        x[e] = first[e] ? x[e] * c - pv[e] * sng : x[e] * c + pv[e] * sng;
      }
    }
  }

  // Hadamard, natural (Sylvester) order: for stride h, (a, b) -> (a + b, a - b) where a is
  // the element whose index has bit h clear.  Then one multiplication by 1/sqrt(D).
  if (a.hadamard) {
#pragma unroll
    for (int h = 1; h < EPL; h <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if ((e & h) == 0) {
          const double u = x[e], v = x[e + h];
          x[e] = u + v; x[e + h] = u - v;
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool hi = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double o = shfl_xor_f64(x[e], m);
        x[e] = hi ? o - x[e] : x[e] + o;
      }
    }
    const double norm = EPL == 2 ? 0.088388347648318440550 : 0.125;   // 1/sqrt(128), 1/sqrt(64)
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] *= norm;
  }

  // fp32 quantizer ([AQ] steps 1-3): amax, scale = amax / qmax, codes = rne(clamp(x / scale)).
  float xf[EPL];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) { xf[e] = (float)x[e]; amax = fmaxf(amax, fabsf(xf[e])); }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  const float qmax = a.code_fp8 ? 448.0f : 127.0f;
  float s = amax / qmax;                                   // IEEE-rounded division
  if (a.round_scale && s > 0.f) {
    // smallest power of two >= s (s is a positive normal or subnormal fp32)
    int ex;
    const float m = frexpf(s, &ex);                        // s = m * 2^ex, m in [0.5, 1)
    s = m == 0.5f ? s : ldexpf(1.0f, ex);
  }
  uint8_t code[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float y = s > 0.f ? xf[e] / s : 0.f;                   // IEEE-rounded division
    y = fminf(fmaxf(y, -qmax), qmax);
    if (a.code_fp8) {
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false);
      code[e] = (uint8_t)(pk & 0xFF);
    } else {
      code[e] = (uint8_t)(int8_t)__float2int_rn(y);
    }
  }

  uint8_t* dst;
  void* sdst;
  if (is_q) { dst = (uint8_t*)a.q_codes; drow = r_in; sdst = a.q_scale; }
  else { dst = (uint8_t*)a.k_cache; sdst = a.k_scale; }
  if (EPL == 2) {
    const uint16_t v = (uint16_t)code[0] | ((uint16_t)code[EPL - 1] << 8);
    ((uint16_t*)(dst + drow * D))[lane] = v;
  } else {
    dst[drow * D + lane] = code[0];
  }
  if (lane == 0) {
    if (a.scale_f16) ((u16*)sdst)[drow] = f32_to_f16_bits(s);
    else ((float*)sdst)[drow] = s;
  }
}

template <int EPL>
static void launch_prolog_d(const PrologArgs& a, dim3 grid, hipStream_t st) {
  if (a.in_bf16) hipLaunchKernelGGL((prolog_kernel<EPL, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((prolog_kernel<EPL, false>), grid, dim3(256), 0, st, a);
}
static void launch_prolog(int D, const PrologArgs& a, dim3 grid, hipStream_t st) {
  if (D == 128) launch_prolog_d<2>(a, grid, st);
  else launch_prolog_d<1>(a, grid, st);
}

}  // namespace dsa

// Checks a prolog configuration (shared with dsa_indexer_prolog_topk).
dsa_status dsa_check_prolog_cfg(const dsa_prolog_cfg* cfg, const char* fn) {
  using dsa_host::fail;
  if (!cfg) return fail(DSA_ERR_INVALID_ARG, "%s: cfg is NULL", fn);
  const dsa_prolog_cfg c = *cfg;
  if (c.D != 64 && c.D != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, c.D);
  if (c.H < 1 || c.H > 1024) return fail(DSA_ERR_INVALID_ARG, "%s: H out of range (got %d)", fn, c.H);
  if (c.rope_dim < 0 || (c.rope_dim & 1) || c.rope_offset < 0 || c.rope_offset + c.rope_dim > c.D)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad rope_dim/rope_offset (%d, %d) for D=%d", fn,
                c.rope_dim, c.rope_offset, c.D);
  if (c.rope_interleaved != 0 && c.rope_interleaved != 1) return fail(DSA_ERR_INVALID_ARG, "%s: rope_interleaved must be 0/1", fn);
  if (c.hadamard != 0 && c.hadamard != 1) return fail(DSA_ERR_INVALID_ARG, "%s: hadamard must be 0/1", fn);
  if (c.round_scale != 0 && c.round_scale != 1) return fail(DSA_ERR_INVALID_ARG, "%s: round_scale must be 0/1", fn);
  if (c.in_dtype != DSA_BF16 && c.in_dtype != DSA_F32) return fail(DSA_ERR_UNSUPPORTED, "%s: in_dtype must be BF16 or F32", fn);
  if (c.code_dtype != DSA_I8 && c.code_dtype != DSA_FP8_E4M3) return fail(DSA_ERR_UNSUPPORTED, "%s: code_dtype must be I8 or FP8_E4M3", fn);
  if (c.scale_dtype != DSA_F16 && c.scale_dtype != DSA_F32) return fail(DSA_ERR_UNSUPPORTED, "%s: scale_dtype must be F16 or F32", fn);
  return DSA_OK;
}

extern "C" dsa_status dsa_indexer_prolog(const dsa_prolog_cfg* cfg, int32_t num_q,
                                         const void* q_in, const float* q_cos,
                                         const float* q_sin, void* q_codes, void* q_scale,
                                         int32_t num_k, const void* k_in, const float* k_cos,
                                         const float* k_sin, const int64_t* k_slot,
                                         void* k_cache, void* k_scale, void* stream) {
  using dsa_host::fail;
  if (!cfg) return fail(DSA_ERR_INVALID_ARG, "dsa_indexer_prolog: cfg is NULL");
  const dsa_prolog_cfg c = *cfg;
  if (num_q < 0 || num_k < 0) return fail(DSA_ERR_INVALID_ARG, "dsa_indexer_prolog: negative row count");
  const dsa_status cst = dsa_check_prolog_cfg(cfg, "dsa_indexer_prolog");
  if (cst != DSA_OK) return cst;
  if (num_q > 0 && (!q_in || !q_codes || !q_scale || (c.rope_dim && (!q_cos || !q_sin))))
    return fail(DSA_ERR_INVALID_ARG, "dsa_indexer_prolog: a query pointer is NULL");
  if (num_k > 0 && (!k_in || !k_slot || !k_cache || !k_scale || (c.rope_dim && (!k_cos || !k_sin))))
    return fail(DSA_ERR_INVALID_ARG, "dsa_indexer_prolog: a key pointer is NULL");
  const long rows = (long)num_q * c.H + num_k;
  if (rows == 0) return DSA_OK;
  if (rows > (long)INT32_MAX * 4) return fail(DSA_ERR_INVALID_ARG, "dsa_indexer_prolog: too many rows");

  dsa::PrologArgs a{};
  a.H = c.H; a.D = c.D; a.rope_dim = c.rope_dim; a.rope_offset = c.rope_offset;
  a.rope_interleaved = c.rope_interleaved; a.hadamard = c.hadamard; a.round_scale = c.round_scale;
  a.in_bf16 = c.in_dtype == DSA_BF16; a.code_fp8 = c.code_dtype == DSA_FP8_E4M3;
  a.scale_f16 = c.scale_dtype == DSA_F16; a.num_q = num_q; a.num_k = num_k;
  a.q_in = q_in; a.q_cos = q_cos; a.q_sin = q_sin; a.q_codes = q_codes; a.q_scale = q_scale;
  a.k_in = k_in; a.k_cos = k_cos; a.k_sin = k_sin; a.k_slot = k_slot; a.k_cache = k_cache;
  a.k_scale = k_scale;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipStream_t st = (hipStream_t)stream;
  dsa::launch_prolog(c.D, a, grid, st);
  return dsa_host::check_launch("dsa_indexer_prolog");
}

// The prolog of a decode batch's query rows and of each token's own key row (cache row
// kv_start[q_seq[t]] + q_pos[t], rotated with the token's table): the separate-launch schedule of
// dsa_indexer_prolog_topk.  cfg and the pointers have been validated by the caller.
dsa_status dsa_prolog_own_keys(const dsa_prolog_cfg* cfg, const dsa_batch* bt, const void* q_in,
                               const float* q_cos, const float* q_sin, void* q_codes, void* q_scale,
                               const void* k_in, void* k_cache, void* k_scale, void* stream) {
  const dsa_prolog_cfg c = *cfg;
  const long rows = (long)bt->num_q * (c.H + 1);
  if (rows == 0) return DSA_OK;
  dsa::PrologArgs a{};
  a.H = c.H; a.D = c.D; a.rope_dim = c.rope_dim; a.rope_offset = c.rope_offset;
  a.rope_interleaved = c.rope_interleaved; a.hadamard = c.hadamard; a.round_scale = c.round_scale;
  a.in_bf16 = c.in_dtype == DSA_BF16; a.code_fp8 = c.code_dtype == DSA_FP8_E4M3;
  a.scale_f16 = c.scale_dtype == DSA_F16; a.num_q = bt->num_q; a.num_k = bt->num_q;
  a.q_in = q_in; a.q_cos = q_cos; a.q_sin = q_sin; a.q_codes = q_codes; a.q_scale = q_scale;
  a.k_in = k_in; a.k_cos = q_cos; a.k_sin = q_sin; a.k_slot = nullptr; a.k_cache = k_cache;
  a.k_scale = k_scale; a.q_seq = bt->q_seq; a.q_pos = bt->q_pos; a.kv_start = bt->kv_start;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipStream_t st = (hipStream_t)stream;
  dsa::launch_prolog(c.D, a, grid, st);
  return DSA_OK;
}
