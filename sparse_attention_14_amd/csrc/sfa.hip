// Sparse Flash Attention decode on gfx950: gather -> bf16 MFMA QK^T -> fp32 online softmax
// -> bf16 MFMA PV -> attention sink.
//
// [SFA] "NPU DeepSeek-V4 TileLang算子开发实践" (mooersco.com/news/996258), section 1, steps 1-8:
// index list with -1 for unused slots (step 2), scores = q . k^T times the scale (step 3), an
// online softmax with running max and sum (step 4), score . value accumulated over key
// blocks and rescaled at the end (steps 5-6), then the per-head sink (step 7).  [DIA]
// "Deepseek Indexer Attention" (jsqmd.com/news/787325): the scattered read of the selected
// kv rows dominated until it went straight from global memory into the matrix unit's
// on-chip buffer -- here the selected rows are gathered straight into LDS.
//
// Decomposition.  The latent KV is one head shared by all query heads (MLA absorbed), so a
// workgroup handles one query token, NH = 16*NB query heads and a contiguous range (split)
// of its selected keys, in tiles of 64 keys:
//   gather : 64 rows x 1152 B into LDS (row pitch 1168 B: 16-B reads of 8 consecutive rows
//            hit distinct banks)
//   QK^T   : S^T = K . Q^T on v_mfma_f32_16x16x32_bf16; wave w owns keys 16w..16w+15 of the
//            tile, Q (NH heads x 576) stays in VGPRs as the B operand for the whole split
//   softmax: per-head tile max via LDS, exp2 in the log2 domain, P in bf16 through LDS
//   PV     : O^T = V^T . P^T; wave w owns value dims 128w..128w+127 for all NH heads, so the
//            accumulator of head h lives in the lanes with lane%16 == h%16 and the softmax
//            rescale is per lane
// A split writes (unnormalised O, running max, running sum) when the selection is spread over
// several workgroups; the combine kernel merges them with the sink.  With one split the main
// kernel applies the sink and writes bf16 directly.
#include "common.h"

namespace dsa {

constexpr int kDqk = 576, kDv = 512;
constexpr int kKT = 64;                              // keys per tile
constexpr int kPitch = kDqk * 2 + 16;                // LDS row pitch in bytes (1168)
constexpr int kChunks = kDqk * 2 / 16;               // 72 16-byte chunks per row
constexpr float kLog2e = 1.4426950408889634f;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

struct SfaArgs {
  const int32_t* q_seq; const int64_t* kv_start;
  const u16* q; const u16* kv; long kv_stride; const int32_t* idx; int k;
  const float* sink; float scale_log2;
  u16* out; float* ws_o; float* ws_ml;
  int T, Hq, n_hg, n_split, kps;
};

__device__ __forceinline__ float exp2_or_zero(float x) { return x == -INFINITY ? 0.f : exp2f(x); }

template <int NB, bool FINAL>
__global__ void __launch_bounds__(256) sfa_kernel(SfaArgs a) {
  constexpr int NH = 16 * NB;
  constexpr int PP = 144;                            // P row pitch in bytes (64 keys + 16 B pad)
  __shared__ __attribute__((aligned(16))) unsigned char kt[kKT * kPitch];
  __shared__ __attribute__((aligned(16))) unsigned char pt[NH * PP];
  __shared__ float red_max[4][NH];
  __shared__ float red_sum[4][NH];
  __shared__ long rows[kKT];
  lds_u8* const kt_lds = (lds_u8*)kt;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int nwg = a.T * a.n_hg * a.n_split;
  const int lid = xcd_remap(blockIdx.x, nwg);
  const int hg = lid % a.n_hg;
  const int ts = lid / a.n_hg;
  const int t = ts / a.n_split, split = ts % a.n_split;
  const int h0 = hg * NH;
  const int kbeg = split * a.kps;
  const int kend = min(a.k, kbeg + a.kps);
  const long kv0 = a.kv_start[a.q_seq[t]];

  // Q^T fragments: lane holds head h0 + 16 nb + c16, dims 32 ks + 8 g .. +7
  v8bf qf[NB][18];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const u16* qrow = a.q + ((long)t * a.Hq + h0 + 16 * nb + c16) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[nb][ks] = *reinterpret_cast<const v8bf*>(qrow + 32 * ks);
  }

  v4f acc_o[8][NB];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc_o[mb][nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { m_run[nb] = -INFINITY; l_run[nb] = 0.f; }

  for (int key0 = kbeg; key0 < kend; key0 += kKT) {
    // ---- selected rows of this tile
    if (tid < kKT) {
      const int j = key0 + tid;
      long r = -1;
      if (j < kend) {
        const int ix = a.idx[(long)t * a.k + j];
        if (ix >= 0) r = kv0 + ix;
      }
      rows[tid] = r;
    }
    __syncthreads();
    // ---- gather 64 x 1152 B into LDS; unused slots are zero-filled
#pragma unroll 6
    for (int it = 0; it < kKT * kChunks / 256; ++it) {
      const int f = tid + 256 * it;
      const int r = f / kChunks, c = f % kChunks;
      const long row = rows[r];
      uint4 v = {0u, 0u, 0u, 0u};
      if (row >= 0) v = *reinterpret_cast<const uint4*>(a.kv + row * a.kv_stride + c * 8);
      *reinterpret_cast<uint4*>(kt + r * kPitch + c * 16) = v;
    }
    __syncthreads();

    // ---- S^T = K . Q^T for keys 16 wave .. +15 of the tile
    v4f s[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = v4f{0.f, 0.f, 0.f, 0.f};
    const unsigned char* arow = kt + (16 * wave + c16) * kPitch + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const v8bf af = *reinterpret_cast<const v8bf*>(arow + 64 * ks);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[nb][ks], s[nb], 0, 0, 0);
    }
    // lane holds keys 16 wave + 4 g + i (i < 4) of head h0 + 16 nb + c16
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 16 * wave + 4 * g + i;
        const float z = rows[slot] >= 0 ? s[nb][i] * a.scale_log2 : -INFINITY;
        s[nb][i] = z;
        m = fmaxf(m, z);
      }
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      if (g == 0) red_max[wave][16 * nb + c16] = m;
    }
    __syncthreads();
    float alpha[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int hl = 16 * nb + c16;
      const float tm = fmaxf(fmaxf(red_max[0][hl], red_max[1][hl]), fmaxf(red_max[2][hl], red_max[3][hl]));
      const float mn = fmaxf(m_run[nb], tm);
      alpha[nb] = (m_run[nb] == -INFINITY) ? (mn == -INFINITY ? 1.f : 0.f) : exp2f(m_run[nb] - mn);
      float ps = 0.f;
      u16 pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = mn == -INFINITY ? 0.f : exp2_or_zero(s[nb][i] - mn);
        pb[i] = f32_to_bf16(pv);
        ps += bf16_to_f32(pb[i]);
      }
      ps += __shfl_xor(ps, 16, kWave);
      ps += __shfl_xor(ps, 32, kWave);
      if (g == 0) red_sum[wave][hl] = ps;
      uint2 pk;
      pk.x = (uint32_t)pb[0] | ((uint32_t)pb[1] << 16);
      pk.y = (uint32_t)pb[2] | ((uint32_t)pb[3] << 16);
      *reinterpret_cast<uint2*>(pt + hl * PP + (16 * wave + 4 * g) * 2) = pk;
      m_run[nb] = mn;
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int hl = 16 * nb + c16;
      l_run[nb] = alpha[nb] * l_run[nb] + (red_sum[0][hl] + red_sum[1][hl] + red_sum[2][hl] + red_sum[3][hl]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc_o[mb][nb] *= alpha[nb];
    }

    // ---- O^T += V^T . P^T for value dims 128 wave .. +127
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8bf pf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        pf[nb] = *reinterpret_cast<const v8bf*>(pt + (16 * nb + c16) * PP + (32 * ks + 8 * g) * 2);
      // V^T fragment via LDS transpose reads: in each 16-lane group, lane j points at
      // 4 values of row (kb + j/4), columns d0 + 4(j%4) .. +3; ds_read_b64_tr_b16 hands
      // lane i the 4 rows of column d0 + i.  Two reads give keys kb .. kb+7.
      const int kb = 32 * ks + 8 * g;
      const int toff = (kb + (c16 >> 2)) * kPitch + (128 * wave + 4 * (c16 & 3)) * 2;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int o = toff + 32 * mb;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(kt_lds + o));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(kt_lds + o + 4 * kPitch));
        const v8bf vf = __builtin_bit_cast(v8bf, v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc_o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[nb], acc_o[mb][nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[d = 128 wave + 16 mb + 4 g + i][head h0 + 16 nb + c16]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int h = h0 + 16 * nb + c16;
    if constexpr (FINAL) {
      const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(m_run[nb], sk);
      const float f = m_run[nb] == -INFINITY ? 0.f : exp2f(m_run[nb] - M);
      const float den = l_run[nb] * f + (sk == -INFINITY ? 0.f : exp2f(sk - M));
      const float inv = den > 0.f ? f / den : 0.f;
      u16* orow = a.out + ((long)t * a.Hq + h) * kDv + 128 * wave + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(acc_o[mb][nb][0] * inv) | ((uint32_t)f32_to_bf16(acc_o[mb][nb][1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc_o[mb][nb][2] * inv) | ((uint32_t)f32_to_bf16(acc_o[mb][nb][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * mb) = pk;
      }
    } else {
      const long base = ((long)t * a.n_split + split) * a.Hq + h;
      float* orow = a.ws_o + base * kDv + 128 * wave + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<v4f*>(orow + 16 * mb) = acc_o[mb][nb];
      if (wave == 0 && g == 0) {
        a.ws_ml[base * 2 + 0] = m_run[nb];
        a.ws_ml[base * 2 + 1] = l_run[nb];
      }
    }
  }
}

// Merge split partials: o = sum_s 2^(m_s - M) O_s / (sum_s 2^(m_s - M) l_s + 2^(sink - M)).
__global__ void __launch_bounds__(128) sfa_combine(SfaArgs a) {
  const int t = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  float M = sk;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.ws_ml[(((long)t * a.n_split + s) * a.Hq + h) * 2]);
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  float den = (sk == -INFINITY) ? 0.f : exp2f(sk - M);
  const int d = threadIdx.x * 4;
  for (int s = 0; s < a.n_split; ++s) {
    const long base = ((long)t * a.n_split + s) * a.Hq + h;
    const float ms = a.ws_ml[base * 2];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - M);
    den += f * a.ws_ml[base * 2 + 1];
    const v4f o = *reinterpret_cast<const v4f*>(a.ws_o + base * kDv + d);
#pragma unroll
    for (int i = 0; i < 4; ++i) num[i] += f * o[i];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint2 pk;
  pk.x = (uint32_t)f32_to_bf16(num[0] * inv) | ((uint32_t)f32_to_bf16(num[1] * inv) << 16);
  pk.y = (uint32_t)f32_to_bf16(num[2] * inv) | ((uint32_t)f32_to_bf16(num[3] * inv) << 16);
  *reinterpret_cast<uint2*>(a.out + ((long)t * a.Hq + h) * kDv + d) = pk;
}

struct SfaPlan { int nb, n_hg, n_split, kps; };

static SfaPlan plan(int T, int Hq, int k) {
  SfaPlan p{};
  p.nb = (Hq % 32 == 0) ? 2 : 1;
  p.n_hg = Hq / (16 * p.nb);
  const long base = (long)T * p.n_hg;
  const int max_split = (k + kKT - 1) / kKT;
  long ns = (512 + base - 1) / base;
  if (ns < 1) ns = 1;
  if (ns > max_split) ns = max_split;
  int kps = (int)((k + ns - 1) / ns);
  kps = (kps + kKT - 1) / kKT * kKT;
  p.kps = kps;
  p.n_split = (k + kps - 1) / kps;
  return p;
}

}  // namespace dsa

using dsa_host::fail;
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn);

extern "C" size_t dsa_sparse_attn_workspace_size(int32_t num_q, int32_t Hq, int32_t k) {
  if (num_q <= 0 || Hq <= 0 || k <= 0 || Hq % 16) return 0;
  const dsa::SfaPlan p = dsa::plan(num_q, Hq, k);
  if (p.n_split <= 1) return 0;
  const size_t n = (size_t)num_q * p.n_split * Hq;
  const size_t o = (n * dsa::kDv * 4 + 255) / 256 * 256;
  return o + (n * 2 * 4 + 255) / 256 * 256;
}

extern "C" dsa_status dsa_sparse_attn_decode(const dsa_batch* bt, int32_t Hq, const void* q,
                                             const void* kv, int64_t kv_row_stride,
                                             const int32_t* idx, int32_t k, const float* sink,
                                             float scale, void* out, void* ws, size_t ws_bytes,
                                             void* stream) {
  const char* fn = "dsa_sparse_attn_decode";
  dsa_status st = dsa_check_batch(bt, fn);
  if (st != DSA_OK) return st;
  if (Hq != 16 && Hq != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: Hq must be 16 or 128 (got %d)", fn, Hq);
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "%s: k must be in [1, 2048] (got %d)", fn, k);
  if (kv_row_stride < dsa::kDqk || kv_row_stride % 8) return fail(DSA_ERR_INVALID_ARG, "%s: kv_row_stride must be >= 576 and a multiple of 8", fn);
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(DSA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (bt->num_q == 0) return DSA_OK;
  if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "%s: a data pointer is NULL", fn);
  if (((uintptr_t)q | (uintptr_t)kv | (uintptr_t)out) & 15) return fail(DSA_ERR_INVALID_ARG, "%s: q/kv/out must be 16-byte aligned", fn);
  const dsa::SfaPlan p = dsa::plan(bt->num_q, Hq, k);
  const size_t need = dsa_sparse_attn_workspace_size(bt->num_q, Hq, k);
  if (need && (!ws || ws_bytes < need)) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  if (need && ((uintptr_t)ws & 255)) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  const long nwg = (long)bt->num_q * p.n_hg * p.n_split;
  if (nwg > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "%s: too many workgroups", fn);

  dsa::SfaArgs a{};
  a.q_seq = bt->q_seq; a.kv_start = bt->kv_start; a.q = (const dsa::u16*)q;
  a.kv = (const dsa::u16*)kv; a.kv_stride = kv_row_stride; a.idx = idx; a.k = k; a.sink = sink;
  a.scale_log2 = scale * dsa::kLog2e; a.out = (dsa::u16*)out;
  a.T = bt->num_q; a.Hq = Hq; a.n_hg = p.n_hg; a.n_split = p.n_split; a.kps = p.kps;
  if (p.n_split > 1) {
    const size_t n = (size_t)bt->num_q * p.n_split * Hq;
    a.ws_o = (float*)ws;
    a.ws_ml = (float*)((char*)ws + (n * dsa::kDv * 4 + 255) / 256 * 256);
  }
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)nwg);
  if (p.n_split == 1) {
    if (p.nb == 2) hipLaunchKernelGGL((dsa::sfa_kernel<2, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dsa::sfa_kernel<1, true>), grid, dim3(256), 0, s, a);
  } else {
    if (p.nb == 2) hipLaunchKernelGGL((dsa::sfa_kernel<2, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dsa::sfa_kernel<1, false>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(dsa::sfa_combine, dim3((unsigned)(bt->num_q * Hq)), dim3(128), 0, s, a);
  }
  return dsa_host::check_launch(fn);
}
