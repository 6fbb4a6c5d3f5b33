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
// workgroup (8 waves) handles one query token, 32 query heads and a contiguous range (split)
// of its selected keys, in tiles of 32 keys:
//   gather : 32 rows x 1152 B straight into LDS by two loader waves; a 4-slot ring (144 KiB)
//            holds the tile being scored, the tile being multiplied with V and two in flight
//   QK^T   : S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 by two score waves (16 heads each, all 32
//            keys and 576 dims); Q stays in VGPRs as the B operand
//   softmax: inside the score wave (tile max across lanes with the gfx950 row swaps), exp2 in
//            the log2 domain, P in bf16 through LDS
//   PV     : O^T = V^T . P^T by four value waves, wave owns value dims 128w..128w+127 for all 32
//            heads, one tile behind the score waves, so the accumulator of head h lives in the
//            lanes with lane%16 == h%16 and the softmax rescale is per lane
// A split writes its own softmax average O / l in bf16 with its running max and sum (fp32)
// when the selection is spread over several workgroups; the combine kernel merges them in fp32
// with the sink.  With one split the main kernel applies the sink and writes bf16 directly.
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"

namespace dsa {

constexpr int kDqk = 576, kDv = 512;
constexpr int kKT = 32;                              // keys per tile
constexpr int kRowB = kDqk * 2;                      // 1152 bytes per latent row
constexpr int kTileB = kKT * kRowB;                  // 36864 bytes per tile
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
  const int32_t* bt; int bps; int bs_log2;   // paged cache: block table (NULL: flat rows)
  int poison;                                // debug: poison LDS before use
  // selection resolved by the kernel itself (sfa_kernel<false, true>) from the top-k select
  // pass's state: the rows' scores (overflow rows re-read them), query positions, the per-row
  // threshold digit and count above it, per-chunk counts, bitmaps and candidate slots, the
  // first-digit histograms (zeroed by the attention for the next call), the candidates'
  // second-digit histograms (zeroed by the merge) and the index output (may be NULL)
  const int32_t* q_pos; const float* scores; long ld;
  const uint32_t* tk_bg; const uint32_t* tk_cnt; const uint32_t* tk_bits; const uint64_t* tk_slots;
  uint32_t* tk_hist; uint32_t* tk_hist2; int tk_nch; int32_t* idx_out;
};
constexpr int kMaxBps = 2048;                        // paged: block-table entries per sequence


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

// Reductions over the four 16-lane rows of a wave (lane l with l ^ 16, l ^ 32, l ^ 48) on the
// gfx950 row-swap instructions: two VALU steps instead of two LDS-path shuffles.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr float kLazy = 8.f;   // log2-domain headroom before the running max is moved
constexpr int kPP = kKT * 2 + 16;        // P row pitch: 32 keys (a tile) + 16 B pad

// The workgroup's eight waves take three roles and work one tile apart:
//  * score waves 0-1, wave = head half hb: S^T = K Q^T for all 32 keys of tile k and heads
//    16 hb .. +15 over all 576 dims (two key blocks x eighteen v_mfma_f32_16x16x32_bf16 steps;
//    Q of the 16 heads stays in VGPRs as the B operand), then the online softmax of tile k inside
//    the wave: tile max, P = 2^(z - m) in bf16 and the rescale factor of the accumulators;
//  * loader waves 2-3: the gather of the tiles into the LDS ring;
//  * value waves 4-7, wave = value dims 128 (w - 4) .. +127 for all 32 heads: O^T += V^T P^T for
//    tile k - 1 (V^T through ds_read_b64_tr_b16 at the end of step k - 1, P^T from LDS).
// Step k has one barrier (tile k landed; P and the rescale factors of tile k - 1 published).  P
// and the factors are double buffered, so the score waves may publish tile k while the value
// waves still read P of tile k - 1.  The reference max m only moves when the tile's max exceeds it by
// more than kLazy, so P < 2^kLazy and the accumulators are rarely rescaled (the final
// normalisation uses the same m: exact).

// Score wave, tile k: masked S^T blocks in the log2 domain and the softmax of tile k for heads
// 16 hb .. +15.  Publishes P (bf16) and the rescale factor; updates the running max and sum.
// BOUND: only the tile's first `valid` keys count (the index entries past them are not -1).
template <bool BOUND = false>
__device__ __forceinline__ void score_tile(const unsigned char* tile, const v8bf* qf, const int* sidx,
                                           int key0, float scale_log2, float& m_run,
                                           float& l_run, unsigned char* pt, float* alpha_out,
                                           int valid = kKT) {
  const int lane = threadIdx.x & 63, hb = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // the keys' indices (-1 = unused slot), four per lane in one read; entries past nkeys are
  // stale but masked by the bound
  int4 iv[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) iv[kb] = *reinterpret_cast<const int4*>(sidx + key0 + 16 * kb + 4 * g);
  // K fragments in the order the MFMAs consume them (key block 0 and 1 of each 32-dim step).
  // One wave keeps at most ~15 LDS reads in flight and reads 1 KiB per b128 instruction at
  // ~46 B/clk, more than an MFMA's 16 cycles, so the schedule below keeps a window of reads
  // ahead of the MFMAs (issue kPre reads, then alternate one MFMA and one read): the MFMAs
  // run under the reads instead of after them.  Four independent accumulation chains (two per
  // key block) keep the matrix core's issue rate, not its latency, the limit.
  // Addresses: chunk 4 ks + g of row r (r & 7 = c16 & 7) sits at chunk (4 ks + g) ^ (c16 & 7);
  // for ks = 2 m + e that is byte 128 m + 64 (e ^ bit 2 of c16) + 16 (g ^ (c16 & 3)) of the row,
  // so the 36 reads use four lane bases and immediate offsets (no per-read arithmetic).
  const int sw = c16 & 7;
  const int lb0 = 64 * ((sw >> 2) & 1) + 16 * (g ^ (sw & 3)), lb1 = lb0 ^ 64;
  const unsigned char* kb0 = tile + c16 * kRowB;
  const unsigned char* kb1 = tile + (16 + c16) * kRowB;
  const unsigned char* kbase[2][2] = {{kb0 + lb0, kb0 + lb1}, {kb1 + lb0, kb1 + lb1}};
  v8bf kf[36];
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    kf[2 * ks] = *reinterpret_cast<const v8bf*>(kbase[0][ks & 1] + 128 * (ks >> 1));
    kf[2 * ks + 1] = *reinterpret_cast<const v8bf*>(kbase[1][ks & 1] + 128 * (ks >> 1));
  }
  v4f sa[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) sa[0][c] = sa[1][c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    sa[0][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[2 * ks], qf[ks], sa[0][ks & 1], 0, 0, 0);
    sa[1][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[2 * ks + 1], qf[ks], sa[1][ks & 1], 0, 0, 0);
  }
  constexpr int kPre = 12;                 // reads ahead of the first MFMA (2 index + 10 K)
  __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
  for (int i = 0; i < 38 - kPre; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 36 - (38 - kPre), 0);
  const v4f s0 = sa[0][0] + sa[0][1], s1 = sa[1][0] + sa[1][1];
  // Raw scores; unused slots and keys past the split's end carry index -1 (the prologue pads the
  // index stage to whole tiles) and are masked to -inf, in the tiles that hold any.  The scale
  // (> 0) joins the exponent's argument in one FMA; the tile max of the raw scores times the
  // scale is the max of the scaled scores.
  float z[2][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { z[0][e] = s0[e]; z[1][e] = s1[e]; }
  const int imin = min(min(min(iv[0].x, iv[0].y), min(iv[0].z, iv[0].w)),
                       min(min(iv[1].x, iv[1].y), min(iv[1].z, iv[1].w)));
  if (!__all(imin >= 0) || (BOUND && valid < kKT)) {   // wave-uniform: a tile with unused slots
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int ix[4] = {iv[kb].x, iv[kb].y, iv[kb].z, iv[kb].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        z[kb][e] = ix[e] >= 0 && (!BOUND || 16 * kb + 4 * g + e < valid) ? z[kb][e] : -INFINITY;
    }
  }
  const float m = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                        fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
  const float tm = rows_max(m) * scale_log2;
  const bool move = (m_run == -INFINITY) ? (tm != -INFINITY) : (tm > m_run + kLazy);
  const float mnew = move ? tm : m_run;
  // v_exp_f32 directly: its arguments are <= kLazy, and -inf gives 0
  const float alpha = move ? __builtin_amdgcn_exp2f(m_run - tm) : 1.f;   // m_run = -inf: 0
  const float nref = mnew == -INFINITY ? 0.f : -mnew;  // all keys masked so far: every z is -inf
  float ps = 0.f;
  const int h = 16 * hb + c16;
  auto p_of = [&](float zr) { return __builtin_amdgcn_exp2f(fmaf(zr, scale_log2, nref)); };
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    uint2 pk;
    pk.x = pack_bf16x2(p_of(z[kb][0]), p_of(z[kb][1]));
    pk.y = pack_bf16x2(p_of(z[kb][2]), p_of(z[kb][3]));
    // the sum uses the rounded values the value waves multiply with
    ps += (__uint_as_float(pk.x << 16) + __uint_as_float(pk.x & 0xFFFF0000u)) +
          (__uint_as_float(pk.y << 16) + __uint_as_float(pk.y & 0xFFFF0000u));
    *reinterpret_cast<uint2*>(pt + h * kPP + (16 * kb + 4 * g) * 2) = pk;
  }
  l_run = alpha * l_run + rows_sum(ps);
  m_run = mnew;
  if (g == 0) alpha_out[h] = alpha;
}

// Value wave ow: its V^T fragments of one tile (value dims 128 ow .. +127, the tile's 32 keys).
struct VFrag { v4s lo[8], hi[8]; };
__device__ __forceinline__ VFrag value_read(const unsigned char* tile, int ow) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const lds_u8* tl = (const lds_u8*)tile;
  // V^T via ds_read_b64_tr_b16: in each 16-lane group lane j points at 4 values of row
  // 8 g + j/4 (+4), columns d0 + 4 (j%4) .. +3; lane i receives the 4 rows of column d0 + i.
  // Addresses: column block mb = 4 h + q of rows r0 = 8 g + c16 / 4 and r1 = r0 + 4 is chunk
  // c = 16 ow + 2 mb + x (x = (c16 & 3) / 2) at (c ^ y) with y = r & 7, i.e. byte
  // 256 ow + 128 h + 32 (q ^ y / 2) + 16 (x ^ (y & 1)) (+ 8 (c16 & 1) within the chunk): eight
  // lane bases (row, q) and an immediate offset for h.
  const int r0 = 8 * g + (c16 >> 2), y0 = c16 >> 2, y1 = y0 + 4, x = (c16 & 3) >> 1;
  const lds_u8* vbase[2][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    vbase[0][q] = tl + r0 * kRowB + 256 * ow + 32 * (q ^ (y0 >> 1)) + 16 * (x ^ (y0 & 1)) + 8 * (c16 & 1);
    vbase[1][q] = tl + (r0 + 4) * kRowB + 256 * ow + 32 * (q ^ (y1 >> 1)) + 16 * (x ^ (y1 & 1)) + 8 * (c16 & 1);
  }
  VFrag v;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    v.lo[mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase[0][mb & 3] + 128 * (mb >> 2)));
    v.hi[mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase[1][mb & 3] + 128 * (mb >> 2)));
  }
  return v;
}

// O^T[128 dims][16 NB heads] += V^T P^T for one tile, its rescale applied first (P and the
// factors from LDS).
template <int NB = 2>
__device__ __forceinline__ void value_mma(v4f (*acc)[NB], const VFrag& v, const unsigned char* pt,
                                          const float* alpha) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  v8bf pf[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    pf[nb] = *reinterpret_cast<const v8bf*>(pt + (16 * nb + c16) * kPP + (8 * g) * 2);
  float al[NB];
  bool rescale = false;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { al[nb] = alpha[16 * nb + c16]; rescale |= al[nb] != 1.f; }
  if (__any(rescale)) {                                // wave-uniform, rare after the first tile
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= al[nb];
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const v8bf vf = __builtin_bit_cast(v8bf, v8s{v.lo[mb][0], v.lo[mb][1], v.lo[mb][2], v.lo[mb][3],
                                                 v.hi[mb][0], v.hi[mb][1], v.hi[mb][2], v.hi[mb][3]});
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[nb], acc[mb][nb], 0, 0, 0);
  }
}

// The selection of token t in ascending position order, slots [kbeg, kbeg + nkeys) of it, into
// sidx (padded with -1 to nkeys_pad), resolved from what the select pass left in the top-k
// workspace: the threshold digit b1 of the row (the top 11 bits of the k-th largest key), the
// count G of keys above it, per 4096-position chunk the bitmap of positions above b1 and the
// candidates with digit b1.  Two more radix digits over the candidates give the exact k-th
// key K*; the selection is then the bitmap, the candidates above K* and the lowest-position
// ties at K* ([LI] "Lightning Indexer": the indexer's TopK keeps the k highest scores; ties to
// the lower position, the rule of the separate top-k call).  Every workgroup of the token
// computes the same K* (no hand-over between workgroups).
//
// slice_loads issues the one memory round trip (before the workgroup's Q loads, so that waiting
// for it does not wait for them); select_slice then works in LDS only, with LDS-only barriers.
// `scr` is LDS scratch: 2 x 32 KiB of row bitmaps and 9 KiB of histogram and counters.  Rows
// whose candidate lists overflow the first trip read every slot in a second trip (at most 16
// chunks, no chunk beyond its slots), else re-read the row's scores.  The select pass also
// counted the candidates' second digits per row (hist2): the second digit b2 is one scan of
// those counts, and the k-th key is ranked among the few candidates in bin b2 by one wave
// (a third histogram pass only when that bin holds more than 64 keys, or on overflow rows).
// The slice ends in sidx, not yet behind a barrier.
constexpr int kSelNT = 512;                            // threads of the attention workgroup
constexpr int kSelLoad = kTkLoad / kSelNT;             // first-trip candidate entries per thread
constexpr int kSelLoad2 = 16 * kTkCap / kSelNT;        // second trip: every slot of <= 16 chunks
constexpr int kSelG = 4;                               // 16-byte bitmap groups per thread (<= 64 chunks)
struct SliceIn {
  int p, sl, gpt;
  uint32_t b1, G, my_cnt;
  uint64_t ev[kSelLoad];
  uint4 wv[kSelG];
  uint4 h2;                                            // second-digit bins 2047 - 4 tid - 3 .. 2047 - 4 tid
};

__device__ __forceinline__ SliceIn slice_loads(const SfaArgs& a, int t) {
  const int tid = threadIdx.x, nch_m = a.tk_nch;
  SliceIn in;
  in.p = a.q_pos[t];
  in.b1 = a.tk_bg[2 * t];
  in.G = a.tk_bg[2 * t + 1];
  in.my_cnt = a.tk_cnt[(long)t * nch_m + min(tid, nch_m - 1)];   // masked later
  // first-trip candidate entries: entry f of the row's lists is chunk f >> sl, slot f & (2^sl - 1)
  in.sl = min(31 - __clz(kTkLoad / nch_m), 9);         // kTkCap = 512
  const uint64_t* srow = a.tk_slots + (long)t * nch_m * kTkCap;
#pragma unroll
  for (int u = 0; u < kSelLoad; ++u) {
    const int f = tid + u * kSelNT;
    in.ev[u] = srow[(long)min(f >> in.sl, nch_m - 1) * kTkCap + (f & ((1 << in.sl) - 1))];
  }
  // this thread's bitmap words: 16-byte groups gpt * tid .. + gpt - 1 (position order)
  const int ngr = nch_m * kTkCW / 4;
  in.gpt = (ngr + kSelNT - 1) / kSelNT;
  const uint4* brow = reinterpret_cast<const uint4*>(a.tk_bits + (long)t * nch_m * kTkCW);
#pragma unroll
  for (int j = 0; j < kSelG; ++j) {
    const int gi = in.gpt * tid + j;
    const bool own = j < in.gpt && gi < ngr;
    const uint4 v = brow[own ? gi : 0];                // any valid group, masked
    const uint32_t m = own ? 0xFFFFFFFFu : 0u;
    in.wv[j] = uint4{v.x & m, v.y & m, v.z & m, v.w & m};
  }
  in.h2 = reinterpret_cast<const uint4*>(a.tk_hist2 + (long)t * kHistBins)[kHistBins / 4 - 1 - tid];
  return in;
}

__device__ __forceinline__ void select_slice(const SfaArgs& a, const SliceIn& in, int t, int kbeg, int nkeys,
                             int nkeys_pad, unsigned char* scr, int* sidx, bool write_idx,
                             bool zero_hist) {
  constexpr int NT = kSelNT;
  const int tid = threadIdx.x;
  const int k = a.k, nch_m = a.tk_nch, p = in.p, sl = in.sl, gpt = in.gpt;
  if (p + 1 <= k) {                                    // short row: every visible position, then -1
    for (int j = tid; j < nkeys_pad; j += NT) {
      const int r = kbeg + j, v = (j < nkeys && r <= p) ? r : -1;
      sidx[j] = v;
      if (write_idx && j < nkeys) a.idx_out[(long)t * k + r] = v;
    }
    return;
  }
  if (zero_hist) {                                     // read by the select pass only
    uint32_t* gh = a.tk_hist + (long)t * kHistShards * kHistBins;
    for (int i = tid; i < kHistShards * kHistBins; i += NT) gh[i] = 0u;
  }
  const int nch = p / kTkChunk + 1;                    // chunks of this row (later ones are stale)
  const int ngr = nch_m * kTkCW / 4, gvalid = nch * kTkCW / 4;
  uint4* sel = reinterpret_cast<uint4*>(scr);          // [64 * kTkCW / 4] selection bitmap
  uint4* tie = sel + 64 * kTkCW / 4;                   // [64 * kTkCW / 4] positions with key K*
  uint32_t* h = reinterpret_cast<uint32_t*>(tie + 64 * kTkCW / 4);   // [kHistBins]
  uint32_t* sh = h + kHistBins;                        // [NT / 64]
  uint32_t* res = sh + NT / 64;                        // [4]
  uint32_t* flag = res + 4;                            // [1]
  uint32_t* n3 = flag + 1;                             // [1]
  uint32_t* scnt = n3 + 2;                             // [64]
  uint32_t* list = scnt + 64;                          // [64] candidates in bin b2
  uint32_t* kres = list + 64;                          // [4] K*, keys equal to it, ties kept
  if (tid < 64) {                                      // wave 0
    scnt[tid] = tid < nch ? in.my_cnt : 0u;            // tid < nch <= nch_m
    // does any chunk's candidate list overflow the first trip (bit 0), or its slots (bit 1)?
    const uint32_t nc = in.my_cnt >> 16;
    const bool ov = tid < nch && nc > (1u << sl), ovc = tid < nch && nc > (uint32_t)kTkCap;
    const uint32_t fl = (__ballot(ov) != 0 ? 1u : 0u) | (__ballot(ovc) != 0 ? 2u : 0u);
    if (tid == 0) { *flag = fl; *n3 = 0u; }
  }
  // selects below are written as masks: a select between two arrays becomes a select of
  // addresses, which puts both in scratch memory
  auto masked = [](uint4 v, bool keep) {
    const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
    return uint4{v.x & m, v.y & m, v.z & m, v.w & m};
  };
#pragma unroll
  for (int j = 0; j < kSelG; ++j) {
    const int gi = gpt * tid + j;
    if (j < gpt && gi < ngr) { sel[gi] = masked(in.wv[j], gi < gvalid); tie[gi] = uint4{0u, 0u, 0u, 0u}; }
  }
  block_barrier<true>();
  // candidate validity without branches: every count first (chunk f >> sl <= 63; chunks past
  // the row read 0)
  uint32_t cn[kSelLoad];
#pragma unroll
  for (int u = 0; u < kSelLoad; ++u) cn[u] = scnt[(tid + u * NT) >> sl];
  uint32_t cvalid = 0;
#pragma unroll
  for (int u = 0; u < kSelLoad; ++u)
    cvalid |= (uint32_t)((uint32_t)((tid + u * NT) & ((1 << sl) - 1)) < (cn[u] >> 16)) << u;
  // Rows of at most 16 chunks whose lists fit their slots but not the first trip's share (a
  // short row with a crowded digit) read every slot in a second trip; the rest re-read the row.
  const uint32_t fl = *flag;
  const bool streamed = (fl & 2u) != 0u || (fl != 0u && nch * kTkCap > kSelLoad2 * NT);
  const bool second = fl != 0u && !streamed;
  // the entries: the first trip's in ev1; a second trip's first half replaces them, its second
  // half in ev2
  static_assert(kSelLoad2 == 2 * kSelLoad, "the second trip is two halves of the first's size");
  uint64_t ev1[kSelLoad], ev2[kSelLoad];
#pragma unroll
  for (int u = 0; u < kSelLoad; ++u) ev1[u] = in.ev[u];
  uint32_t cvalid2 = 0;
  if (second) {                                        // block-uniform
    const uint64_t* srow = a.tk_slots + (long)t * nch_m * kTkCap;
#pragma unroll
    for (int u = 0; u < kSelLoad2; ++u) {
      const int f = tid + u * NT;                      // chunk f >> 9 < 16, slot f & 511
      const uint64_t e = srow[(long)min(f >> 9, nch_m - 1) * kTkCap + (f & (kTkCap - 1))];
      if (u < kSelLoad) ev1[u] = e; else ev2[u - kSelLoad] = e;
    }
    cvalid = 0;
#pragma unroll
    for (int u = 0; u < kSelLoad2; ++u) {
      const int f = tid + u * NT;
      const uint32_t v = (uint32_t)((uint32_t)(f & (kTkCap - 1)) < (scnt[f >> 9] >> 16));
      if (u < kSelLoad) cvalid |= v << u; else cvalid2 |= v << (u - kSelLoad);
    }
  }
  const uint32_t b1 = in.b1;
  const uint32_t need = (uint32_t)k - in.G;            // 1 <= need <= #candidates
  const float* row = a.scores + (long)t * a.ld;
  auto each_cand = [&](auto&& fn) {
    if (!streamed) {
      // one pass over the first trip's entries, two over the second trip's halves (one copy
      // of fn; the halves are selected by value)
#pragma unroll 1
      for (int hf = 0; hf < (second ? 2 : 1); ++hf) {
        const uint32_t cv = hf ? cvalid2 : cvalid;
#pragma unroll
        for (int u = 0; u < kSelLoad; ++u) {
          const uint64_t e = hf ? ev2[u] : ev1[u];
          if ((cv >> u) & 1u) fn((uint32_t)(e >> 32), (uint32_t)e);
        }
      }
    } else {
      // the row's chunks in a rolled loop (little code: this path is rare) with the next
      // chunk's loads in flight while one is processed
      constexpr int PER = kTkChunk / (4 * NT);         // float4 per thread per chunk
      auto load_chunk = [&](int c, float4 (&x)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const long e0 = (long)c * kTkChunk + 4 * (tid + NT * j);
          x[j] = *reinterpret_cast<const float4*>(row + min(e0, (a.ld & ~3L) - 4));
        }
      };
      float4 cur[PER];
      load_chunk(0, cur);
#pragma unroll 1
      for (int c = 0; c < nch; ++c) {
        float4 nxt[PER];
        load_chunk(min(c + 1, nch - 1), nxt);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const long e0 = (long)c * kTkChunk + 4 * (tid + NT * j);
          const float ff[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t key = order_key(ff[q]);
            if (e0 + q <= p && (key >> 21) == b1) fn(key, (uint32_t)(e0 + q));
          }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) cur[j] = nxt[j];
      }
    }
  };
  // ---- the second digit b2 and how many candidates share it (c3)
  uint32_t b2, need2, c3;
  if (!streamed) {                                     // from the select pass's counts, in registers
    const uint32_t loc[4] = {in.h2.w, in.h2.z, in.h2.y, in.h2.x};   // bins 2047 - 4 tid - j
    uint32_t all;
    uint32_t before = block_excl_scan<NT, true>(loc[0] + loc[1] + loc[2] + loc[3], sh, all);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (before < need && need <= before + loc[j]) {
        res[0] = kHistBins - 1 - (4 * tid + j); res[1] = before; res[2] = loc[j];
      }
      before += loc[j];
    }
    block_barrier<true>();
    b2 = res[0]; need2 = need - res[1]; c3 = res[2];
  } else {                                             // a histogram pass over the re-read row
    for (int i = tid; i < kHistBins; i += NT) h[i] = 0u;
    block_barrier<true>();
    each_cand([&](uint32_t key, uint32_t) { atomicAdd(&h[(key >> 10) & 0x7FFu], 1u); });
    block_barrier<true>();
    find_digit_desc<NT, true>(h, need, sh, res);
    b2 = res[0]; need2 = need - res[1]; c3 = h[b2];
  }
  block_barrier<true>();                               // res and h read
  // ---- the k-th key K* among the candidates of bin b2 (need2 of them rank at or above it)
  uint32_t kstar, n_eq, take_eq;
  if (c3 <= 64) {                                      // the bin's keys listed, ranked by one wave
    each_cand([&](uint32_t key, uint32_t) {
      if (((key >> 10) & 0x7FFu) == b2) list[atomicAdd(n3, 1u) & 63u] = key;
    });
    block_barrier<true>();
    if (tid < 64) {
      const uint32_t key = tid < (int)c3 ? list[tid] : 0u;
      uint32_t gt = 0, eq = 0;
      for (uint32_t j = 0; j < c3; ++j) {
        const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, (int)j);
        gt += kj > key;
        eq += kj == key;
      }
      if (tid < (int)c3 && gt < need2 && need2 <= gt + eq) { kres[0] = key; kres[1] = eq; kres[2] = need2 - gt; }
    }
    block_barrier<true>();
    kstar = kres[0]; n_eq = kres[1]; take_eq = kres[2];
  } else {                                             // a third-digit histogram pass
    for (int i = tid; i < kHistBins; i += NT) h[i] = 0u;
    block_barrier<true>();
    each_cand([&](uint32_t key, uint32_t) {
      if (((key >> 10) & 0x7FFu) == b2) atomicAdd(&h[key & 0x3FFu], 1u);
    });
    block_barrier<true>();
    find_digit_desc<NT, true>(h, need2, sh, res);
    kstar = (b1 << 21) | (b2 << 10) | res[0];
    n_eq = h[res[0]];
    take_eq = need2 - res[1];                          // >= 1
  }
  uint32_t* selw = reinterpret_cast<uint32_t*>(sel);
  uint32_t* tiew = reinterpret_cast<uint32_t*>(tie);
  each_cand([&](uint32_t key, uint32_t pos) {
    if (key > kstar) atomicOr(&selw[pos >> 5], 1u << (pos & 31));
    else if (key == kstar) atomicOr(&tiew[pos >> 5], 1u << (pos & 31));
  });
  block_barrier<true>();
  // this thread's words, in position order: the selection with the kept ties
  uint32_t sw[4 * kSelG], tw[4 * kSelG];
  uint32_t ntie = 0, nsel = 0;
#pragma unroll
  for (int j = 0; j < kSelG; ++j) {
    const int gi = gpt * tid + j;
    const bool own = j < gpt && gi < ngr;
    const int gr = own ? gi : 0;                       // any valid group, masked
    const uint4 s4 = masked(sel[gr], own), t4 = masked(tie[gr], own);
    sw[4 * j] = s4.x; sw[4 * j + 1] = s4.y; sw[4 * j + 2] = s4.z; sw[4 * j + 3] = s4.w;
    tw[4 * j] = t4.x; tw[4 * j + 1] = t4.y; tw[4 * j + 2] = t4.z; tw[4 * j + 3] = t4.w;
  }
#pragma unroll
  for (int i = 0; i < 4 * kSelG; ++i) ntie += (uint32_t)__popc(tw[i]);
  if (n_eq == take_eq) {
#pragma unroll
    for (int i = 0; i < 4 * kSelG; ++i) sw[i] |= tw[i];
  } else {                                             // the take_eq lowest positions at K*
    uint32_t tt;
    uint32_t r = block_excl_scan<NT, true>(ntie, sh, tt);
#pragma unroll
    for (int i = 0; i < 4 * kSelG; ++i) {
      uint32_t m = tw[i];
      while (m && r < take_eq) { const uint32_t lb = m & (0u - m); sw[i] |= lb; m ^= lb; ++r; }
    }
    block_barrier<true>();                             // sh reuse
  }
#pragma unroll
  for (int i = 0; i < 4 * kSelG; ++i) nsel += (uint32_t)__popc(sw[i]);
  uint32_t tot;
  uint32_t o = block_excl_scan<NT, true>(nsel, sh, tot);   // rank of this thread's first position
  const uint32_t lo = (uint32_t)kbeg, hi = (uint32_t)(kbeg + nkeys);
  if (o < hi && o + nsel > lo) {                       // this thread holds slots of the slice
#pragma unroll
    for (int i = 0; i < 4 * kSelG; ++i) {
      uint32_t word = sw[i];
      const int base = (4 * gpt * tid + i) * 32;
      while (word && o < hi) {
        const int bit = __ffs(word) - 1;
        word &= word - 1;
        if (o >= lo) {
          sidx[o - lo] = base + bit;
          if (write_idx) a.idx_out[(long)t * k + o] = base + bit;
        }
        ++o;
      }
    }
  }
  for (int j = nkeys + tid; j < nkeys_pad; j += NT) sidx[j] = -1;
}

// One workgroup (8 waves): token t, query heads h0 .. h0+31, selected keys [kbeg, kbeg+nkeys),
// consumed as 32-key tiles through a 4-slot LDS ring: while the score waves work on tile k and
// the value waves on tile k - 1, tiles k + 1 and k + 2 are in flight.
template <bool FINAL, bool TK>
__global__ void __launch_bounds__(512) sfa_kernel(SfaArgs a) {
  constexpr int NH = 32;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[2][NH * kPP];
  __shared__ float abuf[2][NH];
  __shared__ float fin[2][NH];
  __shared__ __attribute__((aligned(16))) int sidx[kMaxKps];
  if (a.poison) {
    poison_lds(&ring, sizeof(ring));
    poison_lds(&pbuf, sizeof(pbuf));
    poison_lds(&abuf, sizeof(abuf));
    poison_lds(&fin, sizeof(fin));
    poison_lds(&sidx, sizeof(sidx));
    __syncthreads();
  }

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int nwg = a.T * a.n_hg * a.n_split;
  const int lid = xcd_remap(blockIdx.x, nwg);
  const int hg = lid % a.n_hg;
  const int ts = lid / a.n_hg;
  const int t = ts / a.n_split, split = ts % a.n_split;
  const int h0 = hg * NH;
  const int kbeg = split * a.kps;
  const int nkeys = min(a.k, kbeg + a.kps) - kbeg;
  const unsigned ring_base = (unsigned)(uintptr_t)(lds_u8*)ring;

  // the selection's state first (fused top-k): waiting for it must not wait for Q
  SliceIn slin;
  if constexpr (TK) slin = slice_loads(a, t);
  asm volatile("" ::: "memory");
  // Prologue, two memory round trips before the first MFMA:
  //  1. Q (this workgroup's 32 heads x 1152 B, laid out like a KV tile) is moved into ring slot
  //     3 with coalesced direct-to-LDS loads; the selected indices, the token's sequence and --
  //     for up to 64 sequences -- every sequence's first cache row (picked by lane, no dependent
  //     load) are loaded alongside;
  //  2. tiles 0 and 1 are gathered while the score waves move Q from LDS into registers.
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
                   "{m0}"(ring_base + 3 * kTileB + j * 1024));
    }
  }
  // the selected indices (clamped reads, masked below) and the batch's first cache rows are
  // issued before the token's sequence id: that id goes to a scalar register, and waiting for
  // it waits for every load issued before it
  int32_t iv[kMaxKps / 512];
  if constexpr (!TK) {
#pragma unroll
    for (int u = 0; u < kMaxKps / 512; ++u) {
      const int j = tid + 512 * u;
      iv[u] = a.idx[(long)t * a.k + kbeg + min(j, nkeys - 1)];
    }
  }
  const long kv_lane = a.bt ? 0 : a.kv_start[min(lane, a.B - 1)];
  asm volatile("" ::: "memory");                       // keep the loads above issued here
  const int seq = a.q_seq[t];
  const int nkeys_pad = (nkeys + kKT - 1) / kKT * kKT;
  if constexpr (TK) {
    // the slice of the selection (flat caches only); ring slots 0-2 are free until the first
    // tiles are issued after the barrier below
    select_slice(a, slin, t, kbeg, nkeys, nkeys_pad, ring, sidx, hg == 0 && a.idx_out,
                 hg == 0 && split == 0);
  } else if (a.bt) {
    // Paged cache: the sequence's block table goes through ring slot 2 (free until tile 2 is
    // issued) and the selected positions become cache rows before they are staged.
    int32_t bv[kMaxBps / 512];
#pragma unroll
    for (int u = 0; u < kMaxBps / 512; ++u) {
      const int j = tid + 512 * u;
      bv[u] = j < a.bps ? a.bt[(long)seq * a.bps + j] : 0;
    }
    int* sbt = reinterpret_cast<int*>(ring + 2 * kTileB);
#pragma unroll
    for (int u = 0; u < kMaxBps / 512; ++u) {
      const int j = tid + 512 * u;
      if (j < a.bps) sbt[j] = bv[u];
    }
    lds_barrier();
    const int bmask = (1 << a.bs_log2) - 1;
#pragma unroll
    for (int u = 0; u < kMaxBps / 512; ++u) {
      const int ix = iv[u];
      if (tid + 512 * u < nkeys && ix >= 0)
        iv[u] = (sbt[min(ix >> a.bs_log2, a.bps - 1)] << a.bs_log2) | (ix & bmask);
    }
  }
  if constexpr (!TK) {
#pragma unroll
    for (int u = 0; u < kMaxKps / 512; ++u) {
      const int j = tid + 512 * u;
      if (j < nkeys_pad) sidx[j] = j < nkeys ? iv[u] : -1;
    }
  }
  long kv0;
  if (a.bt) {
    kv0 = 0;                                           // paged: rows index the whole cache
  } else if (a.B <= 64) {
    kv0 = (long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kv_lane >> 32), seq) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)kv_lane, seq));
  } else {
    kv0 = a.kv_start[seq];
  }
  // DMA addressing: a wave-uniform base (the sequence's first latent row, or the cache when
  // paged; SGPRs) plus a 32-bit per-lane byte offset (the host checks that a sequence, or the
  // paged cache, spans < 4 GiB)
  const u16* kv_seq = uniform_ptr(a.kv + kv0 * a.kv_stride);
  const uint32_t row_bytes = (uint32_t)a.kv_stride * 2u;
  retire(kv_lane);
  wait_vm<0>();                                        // this wave's Q loads have landed
  lds_barrier();                                       // indices and Q (in LDS) visible

  const int nt = (nkeys + kKT - 1) / kKT;
  const int role = __builtin_amdgcn_readfirstlane(wave < 2 ? 0 : (wave < 4 ? 1 : 2));  // score, loader, value
  // Loader wave lw gathers 1-KiB pieces J = lw + 2 it (it < 18) of tile i into ring slot i % 4.
  // A lane's piece it is always row prow[it] of the tile at (swizzled) byte pcol[it] of the
  // row, so only the row's cache index changes from tile to tile; the index stage is padded
  // with -1 to whole tiles (read as row 0: any valid row, masked).  The per-lane offsets of
  // the next tile are read ahead (offs), so a tile's loads issue right after the barrier.
  uint32_t offs[18], prow[18], pcol[18];
  auto piece_rows = [&]() {
#pragma unroll
    for (int it = 0; it < 18; ++it) {
      const int o = ((wave - 2) + 2 * it) * 1024 + lane * 16;
      const int r = o / kRowB;
      prow[it] = (uint32_t)r;
      pcol[it] = (uint32_t)((((o % kRowB) >> 4) ^ (r & 7)) << 4);
    }
  };
  auto tile_offsets = [&](int i) {
#pragma unroll
    for (int it = 0; it < 18; ++it) {
      const int ix = max(sidx[i * kKT + (int)prow[it]], 0);
      offs[it] = (uint32_t)ix * row_bytes + pcol[it];
    }
  };
  // the LDS destinations are wave-uniform: scalar arithmetic from one base
  const unsigned m0w = (unsigned)__builtin_amdgcn_readfirstlane((int)(ring_base + (wave - 2) * 1024));
  auto issue_tile = [&](int i) {
#pragma unroll
    for (int it = 0; it < 18; ++it)
      asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(offs[it]), "s"(kv_seq),
                   "{m0}"(m0w + (unsigned)((i % kNBuf) * kTileB + it * 2048)));
  };

  // One loop per role, each with one barrier per step (nt + 1 steps), so that each role's
  // registers (Q, gather offsets, accumulators) are live only in its own loop.
  if (role == 0) {
    v8bf qf[18];                                       // Q of heads 16 wave + c16
    float m_run = -INFINITY, l_run = 0.f;              // head 16 wave + c16
    const int r = 16 * wave + c16;
    const unsigned char* qt = ring + 3 * kTileB;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      qf[ks] = *reinterpret_cast<const v8bf*>(qt + tile_off(r, 4 * ks + g));
      if (h0 + r >= a.Hq) qf[ks] = v8bf{};
    }
    for (int k = 0; k <= nt; ++k) {
      lds_barrier();                                   // tile k landed; P of tile k - 1 consumed
      if (k < nt)
        score_tile(ring + (k % kNBuf) * kTileB, qf, sidx, k * kKT, a.scale_log2, m_run, l_run,
                   pbuf[k & 1], abuf[k & 1]);
    }
    // running max and sum, per head, to the value waves
    if (g == 0) {
      fin[0][r] = m_run;
      fin[1][r] = l_run;
    }
    lds_barrier();
    return;
  }
  if (role == 1) {
    piece_rows();
    tile_offsets(0);
    issue_tile(0);
    if (nt > 1) { tile_offsets(1); issue_tile(1); }
    if (nt > 2) tile_offsets(2);
    for (int k = 0; k <= nt; ++k) {
      if (k < nt) {                                    // tile k landed (k + 1 may be in flight)
        if (k + 1 < nt) wait_vm<18>(); else wait_vm<0>();
      }
      lds_barrier();
      if (k + 2 < nt) {                                // into the slot of tile k - 2
        issue_tile(k + 2);
        if (k + 3 < nt) tile_offsets(k + 3);
      }
    }
    lds_barrier();
    return;
  }
  v4f acc[8][2];                                       // O^T
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) { acc[mb][0] = v4f{0.f, 0.f, 0.f, 0.f}; acc[mb][1] = acc[mb][0]; }
  // V^T of tile k is read at the end of step k (the tile landed at that step's barrier) and
  // multiplied at step k + 1 with P of tile k; tile k's slot is refilled at step k + 2
  VFrag vnext;
  for (int k = 0; k <= nt; ++k) {
    lds_barrier();                                     // P of tile k - 1 published
    if (k >= 1) value_mma<2>(acc, vnext, pbuf[(k - 1) & 1], abuf[(k - 1) & 1]);
    if (k < nt) vnext = value_read(ring + (k % kNBuf) * kTileB, wave - 4);
  }
  lds_barrier();                                       // running max and sum published
  const int ow = wave - 4;

  // ---- epilogue: lane holds O^T[d = 128 ow + 16 mb + 4 g + e][head h0 + 16 nb + c16].
  // The scaled rows go through LDS (ring slot 0: every tile has been consumed and no gather is
  // in flight) so that each head's 1 KiB row is stored by one wave instruction of 16 bytes per
  // lane, instead of 16 strided 32-byte pieces per instruction.  Only the value waves are left
  // in the workgroup (the others have ended), so the barrier below waits for them alone.
  constexpr int kOP = kDv * 2 + 16;                    // LDS row pitch: rows in distinct banks
  static_assert(32 * kOP <= kTileB, "the output rows do not fit a ring slot");
  unsigned char* ot = ring;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int hl = 16 * nb + c16;
    const int h = h0 + hl;
    if (h >= a.Hq) continue;
    const float mh = fin[0][hl], lh = fin[1][hl];
    float inv;
    if constexpr (FINAL) {
      const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(mh, sk);
      const float f = mh == -INFINITY ? 0.f : exp2f(mh - M);
      const float den = lh * f + (sk == -INFINITY ? 0.f : exp2f(sk - M));
      inv = den > 0.f ? f / den : 0.f;
    } else {
      // the split's own softmax average O / l (a convex combination of value rows) in bf16;
      // the merge weighs it by 2^(m - M) l in fp32
      inv = lh > 0.f ? 1.f / lh : 0.f;
      if (ow == 0 && g == 0) {
        const long base = ((long)t * a.n_split + split) * a.Hq + h;
        a.ws_ml[base * 2 + 0] = mh;
        a.ws_ml[base * 2 + 1] = lh;
      }
    }
    unsigned char* orow = ot + hl * kOP + (128 * ow + 4 * g) * 2;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[mb][nb][0] * inv, acc[mb][nb][1] * inv);
      pk.y = pack_bf16x2(acc[mb][nb][2] * inv, acc[mb][nb][3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * mb) = pk;
    }
  }
  lds_barrier();
  // 32 rows x 64 pieces of 16 bytes over the 256 value-wave threads; row hl = piece / 64
  u16* obase = FINAL ? a.out + ((long)t * a.Hq + h0) * kDv
                     : a.ws_o + (((long)t * a.n_split + split) * a.Hq + h0) * kDv;
  const int vt = tid - 256;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int piece = vt + 256 * i, hl = piece >> 6, c = piece & 63;
    if (h0 + hl < a.Hq)
      *reinterpret_cast<uint4*>(obase + (long)hl * kDv + c * 8) =
          *reinterpret_cast<const uint4*>(ot + hl * kOP + c * 16);
  }
}

// Prefill-sized batches (one split per token, flat caches): one workgroup (8 waves) per token
// and 64 query heads, so each gathered row serves twice the heads of sfa_kernel and the QK^T
// MFMAs spread over all four SIMDs:
//  * score waves 0-3, wave = 16 heads (score_tile as in sfa_kernel, one per SIMD);
//  * value waves 4-7, wave = value dims 128 (w - 4) .. +127 for all 64 heads (value_mma over
//    four head blocks), each also gathering 9 of the 36 1-KiB pieces of every tile (no loader
//    waves: the 8 waves share the SIMDs two by two, so a value wave may take 256 VGPRs).
// The 8 KiB index stage of sfa_kernel does not fit beside the larger P buffer: the selected
// indices move through an 8-tile ring in LDS instead, each value wave bringing 8 indices of tile
// k + 5 per step with one direct-to-LDS dword load (the first five tiles' from the prologue).
// Tiles past the selection's end read clamped indices; score_tile masks them by count.
// Results are bit-identical to sfa_kernel<true, false>: the same tiles, per-head arithmetic and
// order.
constexpr int kIR = 8;                                 // index ring: tiles
__global__ void __launch_bounds__(512) sfa_kernel64(SfaArgs a) {
  constexpr int NH = 64;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kNBuf * kTileB];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[2][NH * kPP];
  __shared__ float abuf[2][NH];
  __shared__ float fin[2][NH];
  __shared__ __attribute__((aligned(16))) int sring[kIR * kKT];
  if (a.poison) {
    poison_lds(&ring, sizeof(ring));
    poison_lds(&pbuf, sizeof(pbuf));
    poison_lds(&abuf, sizeof(abuf));
    poison_lds(&fin, sizeof(fin));
    poison_lds(&sring, sizeof(sring));
    __syncthreads();
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int nwg = a.T * a.n_hg;                        // n_split == 1
  const int lid = xcd_remap(blockIdx.x, nwg);
  const int hg = lid % a.n_hg, t = lid / a.n_hg;
  const int h0 = hg * NH;
  const int nkeys = a.k;
  const int nt = (nkeys + kKT - 1) / kKT;
  const unsigned ring_base = (unsigned)(uintptr_t)(lds_u8*)ring;
  const unsigned sring_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)sring;
  // ---- prologue: Q (64 heads x 1152 B, laid out like a tile) into ring slots 2-3, the first
  // five tiles' indices into the index ring, the token's sequence and its first cache row
  {
    const u16* qbase = uniform_ptr(a.q + (long)t * a.Hq * kDqk);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int it = 0; it < 2 * kTileB / 1024 / 8; ++it) {   // 72 pieces of 1 KiB, 9 per wave
      const int j = wave + 8 * it;
      const int o = j * 1024 + ln * 16;
      const int r = o / kRowB;
      const int c = ((o % kRowB) >> 4) ^ (r & 7);
      const uint32_t off = (uint32_t)min(h0 + r, a.Hq - 1) * (uint32_t)kRowB + (uint32_t)c * 16u;
      asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(qbase),
                   "{m0}"(ring_base + 2 * kTileB + j * 1024));
    }
  }
  const int32_t* irow = a.idx + (long)t * a.k;
  int32_t iv0 = 0;
  if (tid < 5 * kKT) iv0 = irow[min(tid, nkeys - 1)];  // tiles 0-4 (clamped past the selection)
  const long kv_lane = a.kv_start[min(lane, a.B - 1)];
  asm volatile("" ::: "memory");                       // keep the loads above issued here
  const int seq = a.q_seq[t];
  if (tid < 5 * kKT) sring[tid] = iv0;
  long kv0;
  if (a.B <= 64) {
    kv0 = (long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kv_lane >> 32), seq) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)kv_lane, seq));
  } else {
    kv0 = a.kv_start[seq];
  }
  const u16* kv_seq = uniform_ptr(a.kv + kv0 * a.kv_stride);
  const uint32_t row_bytes = (uint32_t)a.kv_stride * 2u;
  retire(kv_lane);
  wait_vm<0>();                                        // this wave's Q loads have landed
  lds_barrier();                                       // Q and the first indices visible

  if (wave < 4) {
    // ---- score waves
    v8bf qf[18];                                       // Q of heads 16 wave + c16
    float m_run = -INFINITY, l_run = 0.f;
    const int r = 16 * wave + c16;
    const unsigned char* qt = ring + 2 * kTileB;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      qf[ks] = *reinterpret_cast<const v8bf*>(qt + tile_off(r, 4 * ks + g));
      if (h0 + r >= a.Hq) qf[ks] = v8bf{};
    }
    for (int k = 0; k <= nt; ++k) {
      lds_barrier();                                   // tile k landed; P of tile k - 1 consumed
      if (k < nt)
        score_tile<true>(ring + (k % kNBuf) * kTileB, qf, sring + (k % kIR) * kKT, 0, a.scale_log2,
                         m_run, l_run, pbuf[k & 1], abuf[k & 1], nkeys - k * kKT);
    }
    if (g == 0) {
      fin[0][r] = m_run;
      fin[1][r] = l_run;
    }
    lds_barrier();
    return;
  }
  // ---- value waves, also the gatherers: pieces J = ow + 4 it (it < 9) of every tile
  const int ow = wave - 4;
  uint32_t offs[9], prow[9], pcol[9];
#pragma unroll
  for (int it = 0; it < 9; ++it) {
    const int o = (ow + 4 * it) * 1024 + lane * 16;
    const int r = o / kRowB;
    prow[it] = (uint32_t)r;
    pcol[it] = (uint32_t)((((o % kRowB) >> 4) ^ (r & 7)) << 4);
  }
  auto tile_offsets = [&](int i) {
#pragma unroll
    for (int it = 0; it < 9; ++it) {
      const int ix = max(sring[(i % kIR) * kKT + (int)prow[it]], 0);
      offs[it] = (uint32_t)ix * row_bytes + pcol[it];
    }
  };
  const unsigned m0w = (unsigned)__builtin_amdgcn_readfirstlane((int)(ring_base + ow * 1024));
  auto issue_tile = [&](int i) {
#pragma unroll
    for (int it = 0; it < 9; ++it)
      asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(offs[it]), "s"(kv_seq),
                   "{m0}"(m0w + (unsigned)((i % kNBuf) * kTileB + it * 4096)));
  };
  // indices 8 ow .. + 7 of tile i into the index ring (lanes 0-7; clamped past the selection;
  // issued for every step, past the last tile too, into a slot no one reads any more)
  const int32_t* ibase = uniform_ptr(irow);
  auto issue_idx = [&](int i) {
    if (lane < 8) {
      const uint32_t off = (uint32_t)min(i * kKT + 8 * ow + lane, nkeys - 1) * 4u;
      asm volatile("global_load_lds_dword %0, %1" :: "v"(off), "s"(ibase),
                   "{m0}"((unsigned)__builtin_amdgcn_readfirstlane(
                       (int)(sring_base + (unsigned)(((i % kIR) * kKT + 8 * ow) * 4)))));
    }
  };
  tile_offsets(0);
  issue_tile(0);
  if (nt > 1) { tile_offsets(1); issue_tile(1); }
  if (nt > 2) tile_offsets(2);
  v4f acc[8][4];                                       // O^T
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = v4f{0.f, 0.f, 0.f, 0.f};
  // V^T of tile k is read at the end of step k (the tile landed at that step's barrier) and
  // multiplied at step k + 1, once P of tile k is published: the reads' latency runs under the
  // barrier.  Tile k's slot is refilled at step k + 2, after those reads were consumed.
  VFrag vnext;
  for (int k = 0; k <= nt; ++k) {
    // tile k landed: issued after it are (k >= 1) the index load of step k - 1 and tile k + 1
    if (k < nt) {
      if (k == 0) { if (nt > 1) wait_vm<9>(); else wait_vm<0>(); }
      else if (k + 1 < nt) wait_vm<10>();
      else wait_vm<1>();
    }
    lds_barrier();
    issue_idx(k + 5);                                  // the indices before the tile: see above
    if (k + 2 < nt) {                                  // into the slot of tile k - 2
      issue_tile(k + 2);
      if (k + 3 < nt) tile_offsets(k + 3);             // its indices came with tile k or earlier
    }
    if (k >= 1) value_mma<4>(acc, vnext, pbuf[(k - 1) & 1], abuf[(k - 1) & 1]);
    if (k < nt) vnext = value_read(ring + (k % kNBuf) * kTileB, ow);
  }
  wait_vm<0>();                                        // the index loads past the end
  lds_barrier();                                       // running max and sum published

  // ---- epilogue (FINAL): rows through ring slots 0-1 as in sfa_kernel, 64 heads
  constexpr int kOP = kDv * 2 + 16;
  static_assert(NH * kOP <= 2 * kTileB, "the output rows do not fit two ring slots");
  unsigned char* ot = ring;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int hl = 16 * nb + c16;
    const int h = h0 + hl;
    if (h >= a.Hq) continue;
    const float mh = fin[0][hl], lh = fin[1][hl];
    const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float M = fmaxf(mh, sk);
    const float f = mh == -INFINITY ? 0.f : exp2f(mh - M);
    const float den = lh * f + (sk == -INFINITY ? 0.f : exp2f(sk - M));
    const float inv = den > 0.f ? f / den : 0.f;
    unsigned char* orow = ot + hl * kOP + (128 * ow + 4 * g) * 2;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[mb][nb][0] * inv, acc[mb][nb][1] * inv);
      pk.y = pack_bf16x2(acc[mb][nb][2] * inv, acc[mb][nb][3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * mb) = pk;
    }
  }
  lds_barrier();
  // 64 rows x 64 pieces of 16 bytes over the 256 value-wave threads; row hl = piece / 64
  u16* obase = a.out + ((long)t * a.Hq + h0) * kDv;
  const int vt = tid - 256;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int piece = vt + 256 * i, hl = piece >> 6, c = piece & 63;
    if (h0 + hl < a.Hq)
      *reinterpret_cast<uint4*>(obase + (long)hl * kDv + c * 8) =
          *reinterpret_cast<const uint4*>(ot + hl * kOP + c * 16);
  }
}

// Merge split partials: with a_s = O_s / l_s (stored bf16), m_s, l_s (fp32) per split,
//   o = sum_s 2^(m_s - M) l_s a_s / (sum_s 2^(m_s - M) l_s + 2^(sink - M)),  M = max(m_s, sink).
// One wave per (token, head), lane = 8 value dims.  One memory round trip: the first kPre
// splits' partial outputs (addresses clamped to the last split, weighted 0 past it) and every
// split's (m, l), lane s holding split s (n_split <= 64); the maxima and weights then move across
// lanes with v_readlane (uniform loops over the splits, no LDS round trips).  Workgroups are
// ordered like the split kernel's (xcd_remap over token-major ids), so a token's partials are
// read on the XCD whose L2 received them.
__global__ void __launch_bounds__(256) sfa_combine(SfaArgs a) {
  constexpr int kPre = 8;                              // splits whose partials load up front
  const int lane = threadIdx.x & 63;
  const int th = xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (th >= a.T * a.Hq) return;                        // whole waves only; no barriers below
  const int t = th / a.Hq, h = th % a.Hq, ns = a.n_split;
  if (a.tk_hist2 && h == 0) {                          // read by this call's attention: clear it
    uint4* h2 = reinterpret_cast<uint4*>(a.tk_hist2 + (long)t * kHistBins);
#pragma unroll
    for (int i = 0; i < kHistBins / 4 / 64; ++i) h2[lane + 64 * i] = uint4{0u, 0u, 0u, 0u};
  }
  const u16* src = a.ws_o + (((long)t * ns) * a.Hq + h) * kDv + lane * 8;
  const long sstride = (long)a.Hq * kDv;
  uint4 pv[kPre];
#pragma unroll
  for (int sp = 0; sp < kPre; ++sp) pv[sp] = *reinterpret_cast<const uint4*>(src + min(sp, ns - 1) * sstride);
  const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (((long)t * ns + min(lane, ns - 1)) * a.Hq + h) * 2);
  const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  auto lane_f = [](float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
  };
  float M = sk;
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, lane_f(ml.x, sp));
  const float f = (lane < ns && ml.x != -INFINITY) ? exp2f(ml.x - M) * ml.y : 0.f;   // split weight
  float den = (sk == -INFINITY) ? 0.f : exp2f(sk - M);
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
  for (int sp = 0; sp < kPre; ++sp)
    if (sp < ns) { const float fs = lane_f(f, sp); den += fs; add(fs, pv[sp]); }
  for (int sp = kPre; sp < ns; ++sp) {
    const float fs = lane_f(f, sp);
    den += fs;
    add(fs, *reinterpret_cast<const uint4*>(src + sp * sstride));
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint4 pk;
  pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  pk.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  pk.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(a.out + ((long)t * a.Hq + h) * kDv + lane * 8) = pk;
}

struct SfaPlan { int n_hg, n_split, kps; bool h64; };

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
  p.h64 = false;
  return p;
}

// Prefill-sized batches on flat caches (one split per token, at least 256 workgroups of 64
// heads): sfa_kernel64.  DSA_SFA_H64=0 keeps sfa_kernel (testing).
static void plan_h64(SfaPlan& p, int T, int Hq, bool flat) {
  const char* e = getenv("DSA_SFA_H64");
  const bool off = e && !strcmp(e, "0");
  if (flat && !off && p.n_split == 1 && Hq % 64 == 0 && (long)T * (Hq / 64) >= 256) {
    p.h64 = true;
    p.n_hg = Hq / 64;
  }
}

}  // namespace dsa

using dsa_host::fail;
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn);

// Fixed scratch for the split partials of dsa_sparse_attn_decode_noalloc (callers that cannot
// allocate).  Each GPU holds its own copy until the process ends; host code uses the device
// address resolved per device below, never this name.
constexpr size_t kScratchBytes = (size_t)12 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};
}  // namespace

// The device address of `scratch` on the current device (resolved once per device).
static dsa_status scratch_address(void** out, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(DSA_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}
dsa_status dsa_check_batch_paged(const dsa_batch* bt, const char* fn);
dsa_status dsa_check_paging(const dsa_paging* pg, const dsa_batch* bt, double row_bytes,
                            const char* fn, int* bs_log2);

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
                              const char* fn, dsa::SfaArgs* args, dsa::SfaPlan* plan,
                              const dsa_paging* pg = nullptr, const dsa_host::SfaSel* sel = nullptr) {
  dsa_status st = pg ? dsa_check_batch_paged(bt, fn) : dsa_check_batch(bt, fn);
  if (st != DSA_OK) return st;
  int bs_log2 = 0;
  if (pg) {
    st = dsa_check_paging(pg, bt, 2.0 * (double)kv_row_stride, fn, &bs_log2);
    if (st != DSA_OK) return st;
    if (bt->num_q > 0 && pg->blocks_per_seq > dsa::kMaxBps)
      return fail(DSA_ERR_UNSUPPORTED, "%s: blocks_per_seq must be <= %d (got %d)", fn, dsa::kMaxBps, pg->blocks_per_seq);
  }
  if (Hq != 16 && Hq != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: Hq must be 16 or 128 (got %d)", fn, Hq);
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "%s: k must be in [1, 2048] (got %d)", fn, k);
  if (kv_row_stride < dsa::kDqk || kv_row_stride % 8) return fail(DSA_ERR_INVALID_ARG, "%s: kv_row_stride must be >= 576 and a multiple of 8", fn);
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(DSA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (bt->num_q == 0) return DSA_OK;
  if (!q || !kv || !(idx || sel) || !out) return fail(DSA_ERR_INVALID_ARG, "%s: a data pointer is NULL", fn);
  if (sel && (pg || !sel->scores || !sel->hist2 || sel->nch < 1 || sel->nch > 64))
    return fail(DSA_ERR_UNSUPPORTED, "%s: a pending selection needs flat caches and rows of at most 64 chunks", fn);
  if (((uintptr_t)q | (uintptr_t)kv | (uintptr_t)out) & 15) return fail(DSA_ERR_INVALID_ARG, "%s: q/kv/out must be 16-byte aligned", fn);
  dsa::SfaPlan p = dsa::plan(bt->num_q, Hq, k);
  dsa::plan_h64(p, bt->num_q, Hq, !pg && !sel);
  if (sel && p.n_split < 2)                              // the merge clears the second-digit histograms
    return fail(DSA_ERR_UNSUPPORTED, "%s: a pending selection needs split partials (k > 32)", fn);
  const size_t need = dsa_sparse_attn_workspace_size(bt->num_q, Hq, k);
  if (need && (!ws || ws_bytes < need)) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  if (need && ((uintptr_t)ws & 255)) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (!pg && (double)bt->max_kv_len * (double)kv_row_stride * 2.0 >= 4294967296.0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: a sequence's latent rows must span < 4 GiB", fn);
  const long nwg = (long)bt->num_q * p.n_hg * p.n_split;
  if (nwg > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "%s: too many workgroups", fn);
  dsa::SfaArgs a{};
  a.q_seq = bt->q_seq; a.kv_start = bt->kv_start; a.q = (const dsa::u16*)q;
  a.kv = (const dsa::u16*)kv; a.kv_stride = kv_row_stride; a.idx = idx; a.k = k; a.sink = sink;
  a.scale_log2 = scale * dsa::kLog2e; a.out = (dsa::u16*)out;
  a.T = bt->num_q; a.B = bt->num_seqs; a.Hq = Hq; a.n_hg = p.n_hg; a.n_split = p.n_split; a.kps = p.kps;
  if (pg) { a.bt = pg->block_table; a.bps = pg->blocks_per_seq; a.bs_log2 = bs_log2; }
  a.poison = dsa_host::debug_poison();
  if (sel) {
    a.idx = nullptr; a.q_pos = bt->q_pos; a.scores = sel->scores; a.ld = sel->ld;
    a.tk_bg = sel->bg; a.tk_cnt = sel->cnt; a.tk_bits = sel->bits; a.tk_slots = sel->slots;
    a.tk_hist = sel->hist; a.tk_hist2 = sel->hist2; a.tk_nch = sel->nch; a.idx_out = sel->idx;
  }
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
  if (a.poison && p.n_split > 1) {                       // split partials: written before merged
    const size_t n = (size_t)a.T * p.n_split * a.Hq;
    dsa_host::poison_fill(a.ws_o, n * dsa::kDv * 2, s);
    dsa_host::poison_fill(a.ws_ml, n * 2 * 4, s);
  }
  if (a.tk_bg)                                           // the kernel resolves its own slice
    hipLaunchKernelGGL((dsa::sfa_kernel<false, true>), grid, dim3(512), 0, s, a);   // n_split > 1
  else if (p.h64)                                        // n_split == 1, flat
    hipLaunchKernelGGL(dsa::sfa_kernel64, grid, dim3(512), 0, s, a);
  else if (p.n_split == 1)
    hipLaunchKernelGGL((dsa::sfa_kernel<true, false>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((dsa::sfa_kernel<false, false>), grid, dim3(512), 0, s, a);
}

static void sfa_launch_merge(const dsa::SfaArgs& a, const dsa::SfaPlan& p, hipStream_t s) {
  if (p.n_split > 1)
    hipLaunchKernelGGL(dsa::sfa_combine, dim3((unsigned)((a.T * a.Hq + 3) / 4)), dim3(256), 0, s, a);
}

// The attention half of dsa_indexer_attention (not exported): over the selection idx, or over a
// selection still pending in the top-k workspace (sel; the kernel resolves its own slice and
// writes sel->idx).  validate_only: check the arguments, launch nothing.
dsa_status dsa_sfa_internal(const dsa_batch* bt, int32_t Hq, const void* q, const void* kv,
                            int64_t kv_row_stride, const int32_t* idx, int32_t k, const float* sink,
                            float scale, void* out, void* ws, size_t ws_bytes,
                            const dsa_host::SfaSel* sel, void* stream, const char* fn,
                            bool validate_only) {
  dsa::SfaArgs a{};
  dsa::SfaPlan p{};
  const dsa_status st = sfa_prepare(bt, Hq, q, kv, kv_row_stride, idx, k, sink, scale, out, ws,
                                    ws_bytes, fn, &a, &p, nullptr, sel);
  if (st != DSA_OK || bt->num_q == 0 || validate_only) return st;
  sfa_launch_split(a, p, (hipStream_t)stream);
  sfa_launch_merge(a, p, (hipStream_t)stream);
  return DSA_OK;
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

extern "C" dsa_status dsa_sparse_attn_decode_paged(const dsa_batch* bt, const dsa_paging* paging,
                                                   int32_t Hq, const void* q, const void* kv,
                                                   int64_t kv_row_stride, const int32_t* idx,
                                                   int32_t k, const float* sink, float scale,
                                                   void* out, void* ws, size_t ws_bytes,
                                                   void* stream) {
  const char* fn = "dsa_sparse_attn_decode_paged";
  if (!paging) return fail(DSA_ERR_INVALID_ARG, "%s: paging is NULL", fn);
  dsa::SfaArgs a{};
  dsa::SfaPlan p{};
  const dsa_status st = sfa_prepare(bt, Hq, q, kv, kv_row_stride, idx, k, sink, scale, out, ws,
                                    ws_bytes, fn, &a, &p, paging);
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

// dsa_sparse_attn_decode with the split partials in the library's fixed per-GPU scratch (no
// workspace argument, no allocation).  Rejects calls whose partials exceed the scratch.
extern "C" dsa_status dsa_sparse_attn_decode_noalloc(const dsa_batch* bt, int32_t Hq, const void* q,
                                                     const void* kv, int64_t kv_row_stride,
                                                     const int32_t* idx, int32_t k, const float* sink,
                                                     float scale, void* out, void* stream) {
  const char* fn = "dsa_sparse_attn_decode_noalloc";
  if (!bt) return fail(DSA_ERR_INVALID_ARG, "%s: batch is NULL", fn);
  if (bt->num_q > 0 && Hq > 0 && k > 0) {
    const size_t need = dsa_sparse_attn_workspace_size(bt->num_q, Hq, k);
    if (need > kScratchBytes)
      return fail(DSA_ERR_UNSUPPORTED, "%s: split partials of %zu bytes exceed the fixed scratch of %zu bytes",
                  fn, need, kScratchBytes);
  }
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (bt->num_q > 0 && dsa_sparse_attn_workspace_size(bt->num_q, Hq, k) > 0) {
    const dsa_status st = scratch_address(&ws, fn);
    if (st != DSA_OK) return st;
    ws_bytes = kScratchBytes;
  }
  dsa::SfaArgs a{};
  dsa::SfaPlan p{};
  const dsa_status st = sfa_prepare(bt, Hq, q, kv, kv_row_stride, idx, k, sink, scale, out, ws,
                                    ws_bytes, fn, &a, &p);
  if (st != DSA_OK || bt->num_q == 0) return st;
  sfa_launch_split(a, p, (hipStream_t)stream);
  sfa_launch_merge(a, p, (hipStream_t)stream);
  return dsa_host::check_launch(fn);
}
