// Upstream projections of the Indexer Prolog on gfx950 (decode shapes: a few query tokens).
//
// [PRO] "Indexer Prolog" (jsqmd.com/news/787325), formulas and quantization strategy: the
// indexer query is DeQuant(q . w_qb) with q and w_qb int8 (the W8A8 linear), the indexer key is
// LayerNorm(x . w_k), the head weights are (x . w_proj) * scale cast to FP16; dequant factors
// are stored in FP16.  [AQ] page, "Int8 GEMM": int8 x int8 -> int32, cast to float, times the
// per-row scale of A and then the per-column scale of B.  What follows (RoPE -> Hadamard ->
// per-token-head quant) is dsa_indexer_prolog.
//
// At decode the token count T is tiny (8 at batch 4 with MTP1) and every linear is a stream over
// its weight matrix (w_qb: 8192 x 1536 int8 = 12 MiB; w_k and w_proj: 192 x 7168 bf16 = 2.6 MiB),
// so the kernels are built to spread the weight rows over every CU, not around a matrix core:
//   w8a8 part     workgroup = 16 output channels; lane (channel c = lane / 16, part kp = lane % 16)
//                 reads one sixteenth of the channel's int8 row in 16-byte pieces and contracts it
//                 with the T activation rows (LDS) on v_dot4_i32_i8, exact int32; four xor
//                 shuffles sum the parts; dequant (acc * a_scale) * b_scale in fp32
//   bf16 part     the key and weight linears as one: workgroup = (32 output rows, one of S = 16
//                 (or 8) slices of the hidden dim); same lane split, fp32 FMAs on bf16 widened
//                 exactly; the S slice sums go to a workspace (a fixed summation order:
//                 deterministic)
// Both parts run in one launch (proj_linears), the w8a8 workgroups first.
//   proj_finish   workgroup per token: sums the slices in order, LayerNorm over the D key values
//                 (fp32, two-pass mean / variance), and the weights times the scale, to FP16.
#include <algorithm>

#include "common.h"

namespace dsa {

constexpr int kPjMaxT = 8;          // query tokens per call
constexpr int kPjCols = 32;         // output channels per workgroup (8 per wave)
constexpr int kPjSlices = 16;       // slices of the hidden dim (bf16 linears), at most

struct PjArgs {
  int T, R, N, hidden, D, H, S;                  // S: hidden slices of the bf16 linears
  const int8_t* qa; const u16* qa_scale; const int8_t* wqb; const u16* wqb_scale;
  const u16* x; const u16* wk; const u16* wp;
  const float* gamma; const float* beta; float eps; float wscale;
  float* q_pre; float* k_pre; u16* weight; float* part;
};

// 16 output channels per workgroup (4 per wave), each row split in 16 parts: 512 workgroups
// for the 8192 channels of the pages' shape, so every CU streams a small share of w_qb.
constexpr int kQCols = 16;
__device__ __forceinline__ void w8a8_block(const PjArgs& a, int blk, unsigned char* qa_l) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, kp = lane & 15;
  const int n = blk * kQCols + wave * 4 + c;
  const int nc = min(n, a.N - 1);                                      // clamped row (no store)
  const int seg = a.R / 16;                                            // bytes per part (16k)
  const int8_t* brow = a.wqb + (long)nc * a.R + kp * seg;
  for (int i = tid * 16; i < a.T * a.R; i += 256 * 16)
    *reinterpret_cast<int4*>(qa_l + i) = *reinterpret_cast<const int4*>(a.qa + i);
  __syncthreads();
  int acc[kPjMaxT];
#pragma unroll
  for (int t = 0; t < kPjMaxT; ++t) acc[t] = 0;
  for (int o = 0; o < seg; o += 16) {
    const int4 b = *reinterpret_cast<const int4*>(brow + o);
#pragma unroll
    for (int t = 0; t < kPjMaxT; ++t) {
      if (t < a.T) {
        const int4 q = *reinterpret_cast<const int4*>(qa_l + t * a.R + kp * seg + o);
        int s = acc[t];
        s = __builtin_amdgcn_sdot4(q.x, b.x, s, false);
        s = __builtin_amdgcn_sdot4(q.y, b.y, s, false);
        s = __builtin_amdgcn_sdot4(q.z, b.z, s, false);
        s = __builtin_amdgcn_sdot4(q.w, b.w, s, false);
        acc[t] = s;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kPjMaxT; ++t) {
    acc[t] += __shfl_xor(acc[t], 1, kWave);
    acc[t] += __shfl_xor(acc[t], 2, kWave);
    acc[t] += __shfl_xor(acc[t], 4, kWave);
    acc[t] += __shfl_xor(acc[t], 8, kWave);
  }
  if (n >= a.N) return;
  const float sb = f16_bits_to_f32(a.wqb_scale[n]);
#pragma unroll
  for (int t = 0; t < kPjMaxT; ++t)
    if (t == kp && t < a.T)                                           // part kp stores token kp
      a.q_pre[(long)t * a.N + n] = ((float)acc[t] * f16_bits_to_f32(a.qa_scale[t])) * sb;
}

// Output row n of the stacked [w_k; w_proj] (D + H rows), hidden slice `sl`.
__device__ __forceinline__ void bf16_block(const PjArgs& a, int blk, int sl, float* x_l) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 3, kp = lane & 7;
  const int NT = a.D + a.H;
  const int n = blk * kPjCols + wave * 8 + c;
  const int nc = min(n, NT - 1);
  const int slice = a.hidden / a.S, k0 = sl * slice;
  const int seg = slice / 8;                                           // elements per part (8k)
  const u16* wrow = (nc < a.D ? a.wk + (long)nc * a.hidden : a.wp + (long)(nc - a.D) * a.hidden) + k0 + kp * seg;
  for (int i = tid * 8; i < a.T * slice; i += 256 * 8) {               // 8 activations per load
    const int t = i / slice, e = i % slice;
    const uint4 v = *reinterpret_cast<const uint4*>(a.x + (long)t * a.hidden + k0 + e);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x_l[i + 2 * q] = __uint_as_float(w[q] << 16);
      x_l[i + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  float acc[kPjMaxT];
#pragma unroll
  for (int t = 0; t < kPjMaxT; ++t) acc[t] = 0.f;
  for (int o = 0; o < seg; o += 8) {
    const uint4 b = *reinterpret_cast<const uint4*>(wrow + o);
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
    float wv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wv[2 * e] = __uint_as_float(bw[e] << 16);
      wv[2 * e + 1] = __uint_as_float(bw[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int t = 0; t < kPjMaxT; ++t) {
      if (t < a.T) {
        const float* xr = x_l + t * slice + kp * seg + o;
        const float4 x0 = *reinterpret_cast<const float4*>(xr);
        const float4 x1 = *reinterpret_cast<const float4*>(xr + 4);
        float s = acc[t];
        s = fmaf(x0.x, wv[0], s); s = fmaf(x0.y, wv[1], s); s = fmaf(x0.z, wv[2], s); s = fmaf(x0.w, wv[3], s);
        s = fmaf(x1.x, wv[4], s); s = fmaf(x1.y, wv[5], s); s = fmaf(x1.z, wv[6], s); s = fmaf(x1.w, wv[7], s);
        acc[t] = s;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kPjMaxT; ++t) {
    acc[t] += __shfl_xor(acc[t], 1, kWave);
    acc[t] += __shfl_xor(acc[t], 2, kWave);
    acc[t] += __shfl_xor(acc[t], 4, kWave);
  }
  if (n >= NT) return;
#pragma unroll
  for (int t = 0; t < kPjMaxT; ++t)
    if (t == kp && t < a.T) a.part[((long)sl * a.T + t) * NT + n] = acc[t];
}

// The query's W8A8 linear and the key/weight linears are independent: one launch runs both, the
// first nq workgroups on w_qb, the rest on the bf16 weights (so the two streams overlap).
__global__ void __launch_bounds__(256) proj_linears(PjArgs a, int nq, int ncb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char pj_lds[];
  const int b = blockIdx.x;
  if (b < nq) w8a8_block(a, b, pj_lds);
  else bf16_block(a, (b - nq) % ncb, (b - nq) / ncb, reinterpret_cast<float*>(pj_lds));
}

__global__ void __launch_bounds__(256) proj_finish(PjArgs a) {
  __shared__ float red[2][4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NT = a.D + a.H;
  // every slice's partial is loaded before the first add (one round trip), then summed in order
  float pv[kPjSlices];
  const int nn = min(tid, NT - 1);
#pragma unroll
  for (int s = 0; s < kPjSlices; ++s) pv[s] = a.part[((long)min(s, a.S - 1) * a.T + t) * NT + nn];
  float v = 0.f;
#pragma unroll
  for (int s = 0; s < kPjSlices; ++s) v += s < a.S ? pv[s] : 0.f;
  const bool key = tid < a.D;
  // LayerNorm over the key values (threads 0 .. D-1): two block sums
  auto block_sum = [&](float x, int slot) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
    if (lane == 0) red[slot][wave] = x;
    __syncthreads();
    return red[slot][0] + red[slot][1] + red[slot][2] + red[slot][3];
  };
  const float mean = block_sum(key ? v : 0.f, 0) / (float)a.D;
  const float dv = key ? v - mean : 0.f;
  const float var = block_sum(dv * dv, 1) / (float)a.D;
  if (key) {
    a.k_pre[(long)t * a.D + tid] = dv / sqrtf(var + a.eps) * a.gamma[tid] + a.beta[tid];
  } else if (tid < NT) {
    a.weight[(long)t * a.H + (tid - a.D)] = f32_to_f16_bits(v * a.wscale);
  }
}

}  // namespace dsa

using dsa_host::fail;

static size_t pj_part_bytes(int32_t T, int32_t H, int32_t D) {
  return (size_t)dsa::kPjSlices * T * (H + D) * 4;
}

extern "C" size_t dsa_indexer_projections_workspace_size(int32_t num_q, int32_t H, int32_t D) {
  if (num_q <= 0 || H <= 0 || D <= 0) return 0;
  return (pj_part_bytes(num_q, H, D) + 255) / 256 * 256;
}

extern "C" dsa_status dsa_indexer_projections(const dsa_projections* p, void* ws, size_t ws_bytes,
                                              void* stream) {
  const char* fn = "dsa_indexer_projections";
  if (!p) return fail(DSA_ERR_INVALID_ARG, "%s: args is NULL", fn);
  const int T = p->num_q;
  if (T < 0) return fail(DSA_ERR_INVALID_ARG, "%s: negative token count", fn);
  if (T == 0) return DSA_OK;
  if (T > dsa::kPjMaxT) return fail(DSA_ERR_UNSUPPORTED, "%s: at most %d query tokens (got %d)", fn, dsa::kPjMaxT, T);
  if (p->H < 1 || p->D < 1 || p->D + p->H > 256 || p->D > 256)
    return fail(DSA_ERR_UNSUPPORTED, "%s: need H + D <= 256 (got H=%d, D=%d)", fn, p->H, p->D);
  if (p->q_rank < 256 || p->q_rank % 256 || (long)T * p->q_rank > 65536)
    return fail(DSA_ERR_UNSUPPORTED, "%s: q_rank must be a multiple of 256 with T*q_rank <= 65536 (got %d)", fn, p->q_rank);
  if (p->hidden < 512 || p->hidden % 512 || (long)T * (p->hidden / 8) * 4 > 65536)
    return fail(DSA_ERR_UNSUPPORTED, "%s: hidden must be a multiple of 512 with T*hidden <= 131072 (got %d)", fn, p->hidden);
  if (!p->q_a || !p->q_a_scale || !p->w_qb || !p->w_qb_scale || !p->x || !p->w_k || !p->ln_gamma ||
      !p->ln_beta || !p->w_proj || !p->q_pre || !p->k_pre || !p->weight)
    return fail(DSA_ERR_INVALID_ARG, "%s: a data pointer is NULL", fn);
  if (((uintptr_t)p->q_a | (uintptr_t)p->w_qb | (uintptr_t)p->x | (uintptr_t)p->w_k | (uintptr_t)p->w_proj) & 15)
    return fail(DSA_ERR_INVALID_ARG, "%s: q_a, w_qb, x, w_k and w_proj must be 16-byte aligned", fn);
  if (!(p->ln_eps >= 0.f)) return fail(DSA_ERR_INVALID_ARG, "%s: ln_eps must be >= 0", fn);
  const size_t need = pj_part_bytes(T, p->H, p->D);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  if ((uintptr_t)ws & 15) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  dsa::PjArgs a{};
  a.S = p->hidden % (dsa::kPjSlices * 64) == 0 ? dsa::kPjSlices : dsa::kPjSlices / 2;   // parts of 8k
  a.T = T; a.R = p->q_rank; a.N = p->H * p->D; a.hidden = p->hidden; a.D = p->D; a.H = p->H;
  a.qa = p->q_a; a.qa_scale = (const dsa::u16*)p->q_a_scale; a.wqb = p->w_qb;
  a.wqb_scale = (const dsa::u16*)p->w_qb_scale; a.x = (const dsa::u16*)p->x;
  a.wk = (const dsa::u16*)p->w_k; a.wp = (const dsa::u16*)p->w_proj;
  a.gamma = p->ln_gamma; a.beta = p->ln_beta; a.eps = p->ln_eps; a.wscale = p->weight_scale;
  a.q_pre = p->q_pre; a.k_pre = p->k_pre; a.weight = (dsa::u16*)p->weight; a.part = (float*)ws;
  hipStream_t s = (hipStream_t)stream;
  const int nq = (a.N + dsa::kQCols - 1) / dsa::kQCols;
  const int ncb = (a.D + a.H + dsa::kPjCols - 1) / dsa::kPjCols;
  const unsigned lds = (unsigned)std::max(T * a.R, T * (a.hidden / a.S) * 4);
  hipLaunchKernelGGL(dsa::proj_linears, dim3((unsigned)(nq + ncb * a.S)), dim3(256), lds, s, a, nq, ncb);
  hipLaunchKernelGGL(dsa::proj_finish, dim3((unsigned)T), dim3(256), 0, s, a);
  return dsa_host::check_launch(fn);
}
