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
// A split writes its own softmax average O / l in bf16 with its running max and sum (fp32)
// when the selection is spread over several workgroups; the combine kernel merges them in fp32
// with the sink.  With one split the main
// kernel applies the sink and writes bf16 directly.
#include "common.h"

namespace dsa {

constexpr int kDqk = 576, kDv = 512;
constexpr int kKT = 32;                              // keys per tile
constexpr int kRowB = kDqk * 2;                      // 1152 bytes per latent row
constexpr int kTileB = kKT * kRowB;                  // 36864 bytes per tile
constexpr int kPairLoads = 2 * kTileB / 16 / 512;    // 9 DMA loads per thread per tile pair
constexpr int kNBuf = 4;                             // tiles in the LDS ring
constexpr int kMaxKps = 2048;                        // keys per split (LDS index stage)
constexpr int kQLoads = 5;                           // Q DMA loads per thread (40 x 1 KiB)
constexpr float kLog2e = 1.4426950408889634f;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

struct SfaArgs {
  const int32_t* q_seq; const int64_t* kv_start;
  const u16* q; const u16* kv; long kv_stride; const int32_t* idx; int k;
  const float* sink; float scale_log2;
  u16* out; u16* ws_o; float* ws_ml;
  int T, B, Hq, n_hg, n_split, kps;
};

__device__ __forceinline__ float exp2_or_zero(float x) { return x == -INFINITY ? 0.f : exp2f(x); }

// Rows are stored unpadded (1152 B) with the 16-byte chunk c of row r at chunk c ^ (r & 7):
// 16-byte reads of one logical chunk from 8 consecutive rows then fall in distinct banks.
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowB + ((c ^ (r & 7)) << 4); }

// Pipeline control.  Tiles move HBM -> LDS with global_load_lds_dwordx4 (each lane's 16 bytes
// land at M0 + 16 * lane), issued from inline asm together with explicit s_waitcnt vmcnt(N)
// and an LDS-only barrier:
//  * __syncthreads() also fences global memory and waits for every load in flight;
//  * for a compiler-issued LDS DMA the compiler waits for all DMA traffic before any LDS
//    read, as it cannot tell ring slots apart;
// either would serialise the ring.  Inside the tile loop the only vector-memory operations
// in flight are these tile loads, so vmcnt(N) with N = loads issued after tile i is exact.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

struct SfaState {
  v4f acc_o[4][2];             // O^T[64-dim slice of this wave][32 heads]
  float m_run[2], l_run[2];    // per head 16 nb + c16 (identical in every wave)
};

constexpr float kLazy = 8.f;   // log2-domain headroom before the running max is moved
constexpr int kPP = 2 * kKT * 2 + 16;   // P row pitch: 64 keys (a tile pair) + 16 B pad

// One tile pair (64 keys) on 8 waves.
//  S^T = K Q^T : wave w takes tile 2k + (w>>2), keys 16 (w&1) .. +15, heads 16 ((w>>1)&1) .. +15
//                (Q of its 16 heads stays in VGPRs as the MFMA B operand).
//  softmax     : per-head pair max through LDS; the reference max m only moves when the pair's
//                max exceeds it by more than kLazy, so P < 2^kLazy and the accumulators are
//                rarely rescaled (the final normalisation uses the same m: exact).
//  O^T += V^T P^T : wave w owns value dims 64 w .. +63 for all 32 heads over both tiles
//                (V^T via ds_read_b64_tr_b16, P^T from LDS).
__device__ __forceinline__ void pair_step(SfaState& st, const unsigned char* t0,
                                          const unsigned char* t1, const v8bf* qf,
                                          const int* sidx, int key0, int nkeys, float scale_log2,
                                          unsigned char* pt, float (*red_max)[32],
                                          float (*red_sum)[32]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int th = wave >> 2, kh = wave & 1, hb = (wave >> 1) & 1;
  const int q4 = 2 * th + kh;                          // key quarter of the pair
  const unsigned char* tile = th ? t1 : t0;
  v4f s0 = v4f{0.f, 0.f, 0.f, 0.f}, s1 = s0;
  {
    const int r = 16 * kh + c16;
    // K fragments are read two k-steps ahead of their MFMAs; the scheduling barriers keep the
    // compiler from hoisting all 18 reads to the top.
    v8bf a0 = *reinterpret_cast<const v8bf*>(tile + tile_off(r, g));
    v8bf a1 = *reinterpret_cast<const v8bf*>(tile + tile_off(r, 4 + g));
#pragma unroll
    for (int ks = 0; ks < 18; ks += 2) {
      v8bf n0 = a0, n1 = a1;
      if (ks + 2 < 18) {
        n0 = *reinterpret_cast<const v8bf*>(tile + tile_off(r, 4 * ks + 8 + g));
        n1 = *reinterpret_cast<const v8bf*>(tile + tile_off(r, 4 * ks + 12 + g));
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks + 1], s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      a0 = n0; a1 = n1;
    }
  }
  v4f s = s0 + s1;
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = key0 + 16 * q4 + 4 * g + e;
    const float z = (key < nkeys && sidx[key] >= 0) ? s[e] * scale_log2 : -INFINITY;
    s[e] = z;
    m = fmaxf(m, z);
  }
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  if (g == 0) red_max[q4][16 * hb + c16] = m;
  lds_barrier();
  float alpha[2], mnew[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int h = 16 * nb + c16;
    const float tm = fmaxf(fmaxf(red_max[0][h], red_max[1][h]), fmaxf(red_max[2][h], red_max[3][h]));
    const float mo = st.m_run[nb];
    const bool move = (mo == -INFINITY) ? (tm != -INFINITY) : (tm > mo + kLazy);
    mnew[nb] = move ? tm : mo;
    alpha[nb] = move ? ((mo == -INFINITY) ? 0.f : exp2f(mo - tm)) : 1.f;
  }
  {
    const float mn = mnew[hb];
    float ps = 0.f;
    u16 pb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pv = mn == -INFINITY ? 0.f : exp2_or_zero(s[e] - mn);
      pb[e] = f32_to_bf16(pv);
      ps += bf16_to_f32(pb[e]);
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    const int h = 16 * hb + c16;
    if (g == 0) red_sum[q4][h] = ps;
    uint2 pk;
    pk.x = (uint32_t)pb[0] | ((uint32_t)pb[1] << 16);
    pk.y = (uint32_t)pb[2] | ((uint32_t)pb[3] << 16);
    *reinterpret_cast<uint2*>(pt + h * kPP + (16 * q4 + 4 * g) * 2) = pk;
  }
  lds_barrier();
  bool rescale = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int h = 16 * nb + c16;
    st.l_run[nb] = alpha[nb] * st.l_run[nb] + (red_sum[0][h] + red_sum[1][h]) + (red_sum[2][h] + red_sum[3][h]);
    st.m_run[nb] = mnew[nb];
    rescale |= alpha[nb] != 1.f;
  }
  if (__any(rescale)) {                                // wave-uniform, rare after the first pair
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) { st.acc_o[mb][0] *= alpha[0]; st.acc_o[mb][1] *= alpha[1]; }
  }
  // V^T via ds_read_b64_tr_b16: in each 16-lane group lane j points at 4 values of row
  // kb + j/4, columns d0 + 4 (j%4) .. +3; lane i receives the 4 rows of column d0 + i.
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const lds_u8* tl = (const lds_u8*)(tt ? t1 : t0);
    v8bf pf[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      pf[nb] = *reinterpret_cast<const v8bf*>(pt + (16 * nb + c16) * kPP + (32 * tt + 8 * g) * 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int col = 64 * wave + 16 * mb + 4 * (c16 & 3);
      const int r0 = 8 * g + (c16 >> 2), r1 = r0 + 4;
      const int c = col >> 3, wi = (col & 7) * 2;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tl + tile_off(r0, c) + wi));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tl + tile_off(r1, c) + wi));
      const v8bf vf = __builtin_bit_cast(v8bf, v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      st.acc_o[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0], st.acc_o[mb][0], 0, 0, 0);
      st.acc_o[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[1], st.acc_o[mb][1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One workgroup (8 waves): token t, query heads h0 .. h0+31, selected keys [kbeg, kbeg+nkeys),
// consumed as pairs of 32-key tiles.  Tiles flow HBM -> 4-slot LDS ring (the next pair in
// flight while the current pair is consumed) -> MFMA; 8 waves give each SIMD two waves that
// hide each other's latency.
template <bool FINAL>
__global__ void __launch_bounds__(512) sfa_kernel(SfaArgs a) {
  constexpr int NH = 32;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char pt[NH * kPP];
  __shared__ float red_max[4][NH];
  __shared__ float red_sum[4][NH];
  __shared__ int sidx[kMaxKps];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15, hb = (wave >> 1) & 1;
  const int nwg = a.T * a.n_hg * a.n_split;
  const int lid = xcd_remap(blockIdx.x, nwg);
  const int hg = lid % a.n_hg;
  const int ts = lid / a.n_hg;
  const int t = ts / a.n_split, split = ts % a.n_split;
  const int h0 = hg * NH;
  const int kbeg = split * a.kps;
  const int nkeys = min(a.k, kbeg + a.kps) - kbeg;
  const unsigned ring_base = (unsigned)(uintptr_t)(lds_u8*)ring;

  // Prologue, two memory round trips before the first MFMA:
  //  1. Q (this workgroup's 32 heads x 1152 B, laid out like a KV tile) is moved into the ring
  //     slot of tile 2 with coalesced direct-to-LDS loads; the selected indices, the token's
  //     sequence and -- for up to 64 sequences -- every sequence's first cache row (picked by
  //     lane, no dependent load) are loaded alongside;
  //  2. the first tile pair is gathered (below) while Q moves from LDS into registers.
  {
    const u16* qbase = uniform_ptr(a.q + (long)t * a.Hq * kDqk);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int it = 0; it < kQLoads; ++it) {
      const int j = min(wave + 8 * it, kTileB / 1024 - 1);   // 36 KiB = 36 x 1 KiB, padded to 40
      const int o = j * 1024 + ln * 16;
      const int r = o / kRowB;
      const int c = ((o % kRowB) >> 4) ^ (r & 7);
      const uint32_t off = (uint32_t)min(h0 + r, a.Hq - 1) * (uint32_t)kRowB + (uint32_t)c * 16u;
      asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(qbase),
                   "{m0}"(ring_base + 2 * kTileB + j * 1024));
    }
  }
  const int seq = a.q_seq[t];
  int32_t iv[kMaxKps / 512];
#pragma unroll
  for (int u = 0; u < kMaxKps / 512; ++u) {
    const int j = tid + 512 * u;
    iv[u] = j < nkeys ? a.idx[(long)t * a.k + kbeg + j] : 0;
  }
  const long kv_lane = a.kv_start[min(lane, a.B - 1)];
#pragma unroll
  for (int u = 0; u < kMaxKps / 512; ++u) {
    const int j = tid + 512 * u;
    if (j < nkeys) sidx[j] = iv[u];
  }
  long kv0;
  if (a.B <= 64) {
    kv0 = (long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kv_lane >> 32), seq) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)kv_lane, seq));
  } else {
    kv0 = a.kv_start[seq];
  }
  // DMA addressing: a wave-uniform base (the sequence's first latent row, SGPRs) plus a
  // 32-bit per-lane byte offset (the host checks that a sequence spans < 4 GiB)
  const u16* kv_seq = uniform_ptr(a.kv + kv0 * a.kv_stride);
  const uint32_t row_bytes = (uint32_t)a.kv_stride * 2u;
  retire(kv_lane);
  __syncthreads();                                     // indices and Q (in LDS) visible

  SfaState st;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) { st.acc_o[mb][0] = v4f{0.f, 0.f, 0.f, 0.f}; st.acc_o[mb][1] = st.acc_o[mb][0]; }
  st.m_run[0] = st.m_run[1] = -INFINITY;
  st.l_run[0] = st.l_run[1] = 0.f;

  const int nt = (nkeys + kKT - 1) / kKT;
  const int npairs = (nt + 1) / 2;
  // a pair = tiles 2k, 2k+1 in ring slots (2k)%4, (2k+1)%4: 72 wave-instructions of 1 KiB,
  // J = wave + 8 it (it < 9), so every thread issues exactly kPairLoads DMA loads per pair.
  // A tile past nt (odd tile count) loads clamped, valid rows whose keys are masked.
  auto issue_pair = [&](int k) {
    // opaque lane id: keeps the per-load offsets from being hoisted out of the pair loop
    // (hoisted, they do not fit the register budget and get spilled)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // all index reads first (one LDS round trip), then the nine loads back to back
    uint32_t off[kPairLoads];
#pragma unroll
    for (int it = 0; it < kPairLoads; ++it) {
      const int J = wave + 8 * it;
      const int half = J >= kTileB / 1024 ? 1 : 0;
      const int j = J - half * (kTileB / 1024);
      const int tl = 2 * k + half;
      const int o = j * 1024 + ln * 16;
      const int r = o / kRowB;
      const int c = ((o % kRowB) >> 4) ^ (r & 7);
      const int key = min(tl * kKT + r, nkeys - 1);
      const int ix = max(sidx[key], 0);                // unused slot: any valid row (masked)
      off[it] = (uint32_t)ix * row_bytes + (uint32_t)c * 16u;
    }
#pragma unroll
    for (int it = 0; it < kPairLoads; ++it) {
      const int J = wave + 8 * it;
      const int half = J >= kTileB / 1024 ? 1 : 0;
      const int j = J - half * (kTileB / 1024);
      const int tl = 2 * k + half;
      asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(off[it]), "s"(kv_seq),
                   "{m0}"(ring_base + (tl % kNBuf) * kTileB + j * 1024));
    }
  };
  if (npairs > 0) issue_pair(0);
  // Q fragments from LDS (rows 16 hb + c16, the MFMA B operand); heads past Hq stay zero
  v8bf qf[18];
  {
    const int r = 16 * hb + c16;
    const unsigned char* qt = ring + 2 * kTileB;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      qf[ks] = *reinterpret_cast<const v8bf*>(qt + tile_off(r, 4 * ks + g));
      if (h0 + r >= a.Hq) qf[ks] = v8bf{};
    }
  }
  for (int k = 0; k < npairs; ++k) {
    lds_barrier();                                     // pair k-1 fully consumed (ring slots free)
    if (k + 1 < npairs) { issue_pair(k + 1); wait_vm<kPairLoads>(); } else { wait_vm<0>(); }
    lds_barrier();                                     // pair k landed for every thread
    pair_step(st, ring + ((2 * k) % kNBuf) * kTileB, ring + ((2 * k + 1) % kNBuf) * kTileB, qf,
              sidx, 2 * k * kKT, nkeys, a.scale_log2, pt, red_max, red_sum);
  }
  const int wave4 = wave;                              // value-dim slice (64 wide) of this wave

  // ---- epilogue: lane holds O^T[d = 64 wave + 16 mb + 4 g + e][head h0 + 16 nb + c16]
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int h = h0 + 16 * nb + c16;
    if (h >= a.Hq) continue;
    if constexpr (FINAL) {
      const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(st.m_run[nb], sk);
      const float f = st.m_run[nb] == -INFINITY ? 0.f : exp2f(st.m_run[nb] - M);
      const float den = st.l_run[nb] * f + (sk == -INFINITY ? 0.f : exp2f(sk - M));
      const float inv = den > 0.f ? f / den : 0.f;
      u16* orow = a.out + ((long)t * a.Hq + h) * kDv + 64 * wave4 + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(st.acc_o[mb][nb][0] * inv) | ((uint32_t)f32_to_bf16(st.acc_o[mb][nb][1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(st.acc_o[mb][nb][2] * inv) | ((uint32_t)f32_to_bf16(st.acc_o[mb][nb][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * mb) = pk;
      }
    } else {
      // the split's own softmax average O / l (a convex combination of value rows) in bf16;
      // the merge weighs it by 2^(m - M) l in fp32
      const long base = ((long)t * a.n_split + split) * a.Hq + h;
      const float inv = st.l_run[nb] > 0.f ? 1.f / st.l_run[nb] : 0.f;
      u16* orow = a.ws_o + base * kDv + 64 * wave4 + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(st.acc_o[mb][nb][0] * inv) | ((uint32_t)f32_to_bf16(st.acc_o[mb][nb][1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(st.acc_o[mb][nb][2] * inv) | ((uint32_t)f32_to_bf16(st.acc_o[mb][nb][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * mb) = pk;
      }
      if (wave4 == 0 && g == 0) {
        a.ws_ml[base * 2 + 0] = st.m_run[nb];
        a.ws_ml[base * 2 + 1] = st.l_run[nb];
      }
    }
  }
}

// Merge split partials: with a_s = O_s / l_s (stored bf16), m_s, l_s (fp32) per split,
//   o = sum_s 2^(m_s - M) l_s a_s / (sum_s 2^(m_s - M) l_s + 2^(sink - M)),  M = max(m_s, sink).
// One wave per (token, head): lane s reads split s's (m, l) (n_split <= 64), the wave reduces
// them with shuffles, then each lane accumulates 8 value dims over the splits.
__global__ void __launch_bounds__(256) sfa_combine(SfaArgs a) {
  constexpr int kPre = 8;                              // splits whose partials load up front
  const int lane = threadIdx.x & 63;
  const int th = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (th >= a.T * a.Hq) return;                        // whole waves only; no barriers below
  const int t = th / a.Hq, h = th % a.Hq;
  const u16* src = a.ws_o + (((long)t * a.n_split) * a.Hq + h) * kDv + lane * 8;
  const long sstride = (long)a.Hq * kDv;
  // one memory round trip: the first kPre splits' partial outputs and every split's (m, l)
  uint4 pv[kPre];
#pragma unroll
  for (int sp = 0; sp < kPre; ++sp) {
    pv[sp] = uint4{0u, 0u, 0u, 0u};
    if (sp < a.n_split) pv[sp] = *reinterpret_cast<const uint4*>(src + sp * sstride);
  }
  const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  float ms = -INFINITY, ls = 0.f;
  if (lane < a.n_split) {
    const long base = ((long)t * a.n_split + lane) * a.Hq + h;
    ms = a.ws_ml[base * 2];
    ls = a.ws_ml[base * 2 + 1];
  }
  float M = ms;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
  M = fmaxf(M, sk);
  const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - M) * ls;   // split weight
  float den = f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, kWave);
  den += (sk == -INFINITY) ? 0.f : exp2f(sk - M);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](float fs, const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += fs * bf16_to_f32((u16)w[i]);
      acc[2 * i + 1] += fs * bf16_to_f32((u16)(w[i] >> 16));
    }
  };
#pragma unroll
  for (int sp = 0; sp < kPre; ++sp) add(__shfl(f, sp, kWave), pv[sp]);   // 0 past n_split
  for (int sp = kPre; sp < a.n_split; ++sp)
    add(__shfl(f, sp, kWave), *reinterpret_cast<const uint4*>(src + sp * sstride));
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint4 pk;
  pk.x = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
  pk.y = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
  pk.z = (uint32_t)f32_to_bf16(acc[4] * inv) | ((uint32_t)f32_to_bf16(acc[5] * inv) << 16);
  pk.w = (uint32_t)f32_to_bf16(acc[6] * inv) | ((uint32_t)f32_to_bf16(acc[7] * inv) << 16);
  *reinterpret_cast<uint4*>(a.out + ((long)t * a.Hq + h) * kDv + lane * 8) = pk;
}

struct SfaPlan { int n_hg, n_split, kps; };

// One workgroup per CU (the LDS ring takes ~150 KiB): aim for 256 workgroups.
static SfaPlan plan(int T, int Hq, int k) {
  SfaPlan p{};
  p.n_hg = (Hq + 31) / 32;
  const long base = (long)T * p.n_hg;
  const int max_split = (k + kKT - 1) / kKT;
  long ns = (256 + base - 1) / base;
  if (ns < 1) ns = 1;
  if (ns > max_split) ns = max_split;
  if (ns > 64) ns = 64;                                // the combine reads splits lane-wise
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
  const size_t o = (n * dsa::kDv * 2 + 255) / 256 * 256;
  return o + (n * 2 * 4 + 255) / 256 * 256;
}

// Validates a sparse-attention call and fills the kernel arguments (no launch).
static dsa_status sfa_prepare(const dsa_batch* bt, int32_t Hq, const void* q, const void* kv,
                              int64_t kv_row_stride, const int32_t* idx, int32_t k,
                              const float* sink, float scale, void* out, void* ws, size_t ws_bytes,
                              const char* fn, dsa::SfaArgs* args, dsa::SfaPlan* plan) {
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
  if ((double)bt->max_kv_len * (double)kv_row_stride * 2.0 >= 4294967296.0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: a sequence's latent rows must span < 4 GiB", fn);
  const long nwg = (long)bt->num_q * p.n_hg * p.n_split;
  if (nwg > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "%s: too many workgroups", fn);
  dsa::SfaArgs a{};
  a.q_seq = bt->q_seq; a.kv_start = bt->kv_start; a.q = (const dsa::u16*)q;
  a.kv = (const dsa::u16*)kv; a.kv_stride = kv_row_stride; a.idx = idx; a.k = k; a.sink = sink;
  a.scale_log2 = scale * dsa::kLog2e; a.out = (dsa::u16*)out;
  a.T = bt->num_q; a.B = bt->num_seqs; a.Hq = Hq; a.n_hg = p.n_hg; a.n_split = p.n_split; a.kps = p.kps;
  if (p.n_split > 1) {
    const size_t n = (size_t)bt->num_q * p.n_split * Hq;
    a.ws_o = (dsa::u16*)ws;
    a.ws_ml = (float*)((char*)ws + (n * dsa::kDv * 2 + 255) / 256 * 256);
  }
  *args = a;
  *plan = p;
  return DSA_OK;
}

static void sfa_launch_split(const dsa::SfaArgs& a, const dsa::SfaPlan& p, hipStream_t s) {
  const dim3 grid((unsigned)((long)a.T * p.n_hg * p.n_split));
  if (p.n_split == 1) hipLaunchKernelGGL((dsa::sfa_kernel<true>), grid, dim3(512), 0, s, a);
  else hipLaunchKernelGGL((dsa::sfa_kernel<false>), grid, dim3(512), 0, s, a);
}

static void sfa_launch_merge(const dsa::SfaArgs& a, const dsa::SfaPlan& p, hipStream_t s) {
  if (p.n_split > 1)
    hipLaunchKernelGGL(dsa::sfa_combine, dim3((unsigned)((a.T * a.Hq + 3) / 4)), dim3(256), 0, s, a);
}

extern "C" dsa_status dsa_sparse_attn_decode(const dsa_batch* bt, int32_t Hq, const void* q,
                                             const void* kv, int64_t kv_row_stride,
                                             const int32_t* idx, int32_t k, const float* sink,
                                             float scale, void* out, void* ws, size_t ws_bytes,
                                             void* stream) {
  const char* fn = "dsa_sparse_attn_decode";
  dsa::SfaArgs a{};
  dsa::SfaPlan p{};
  const dsa_status st = sfa_prepare(bt, Hq, q, kv, kv_row_stride, idx, k, sink, scale, out, ws,
                                    ws_bytes, fn, &a, &p);
  if (st != DSA_OK || bt->num_q == 0) return st;
  sfa_launch_split(a, p, (hipStream_t)stream);
  sfa_launch_merge(a, p, (hipStream_t)stream);
  return dsa_host::check_launch(fn);
}

extern "C" dsa_status dsa_sparse_attn_split(const dsa_batch* bt, int32_t Hq, const void* q,
                                            const void* kv, int64_t kv_row_stride,
                                            const int32_t* idx, int32_t k, const float* sink,
                                            float scale, void* out, void* ws, size_t ws_bytes,
                                            void* stream) {
  const char* fn = "dsa_sparse_attn_split";
  dsa::SfaArgs a{};
  dsa::SfaPlan p{};
  const dsa_status st = sfa_prepare(bt, Hq, q, kv, kv_row_stride, idx, k, sink, scale, out, ws,
                                    ws_bytes, fn, &a, &p);
  if (st != DSA_OK || bt->num_q == 0) return st;
  sfa_launch_split(a, p, (hipStream_t)stream);
  return dsa_host::check_launch(fn);
}

extern "C" dsa_status dsa_sparse_attn_merge(const dsa_batch* bt, int32_t Hq, int32_t k,
                                            const float* sink, void* out, void* ws,
                                            size_t ws_bytes, void* stream) {
  const char* fn = "dsa_sparse_attn_merge";
  dsa::SfaArgs a{};
  dsa::SfaPlan p{};
  // the merge reads no q / kv / idx: any non-NULL aligned value passes their checks
  const dsa_status st = sfa_prepare(bt, Hq, out, out, dsa::kDqk, (const int32_t*)out, k, sink,
                                    1.f, out, ws, ws_bytes, fn, &a, &p);
  if (st != DSA_OK || bt->num_q == 0) return st;
  sfa_launch_merge(a, p, (hipStream_t)stream);
  return dsa_host::check_launch(fn);
}
