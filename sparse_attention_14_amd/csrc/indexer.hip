// Lightning Indexer scores on gfx950 (int8 MFMA; fp8 codes through exact bf16 MFMA).
//
// [LI] "Lightning Indexer" (jsqmd.com/news/787325): per query token, the quantized query of
// every indexer head is multiplied against the quantized key cache, followed by ReLU, a
// per-head weighting and a sum over heads; [PRO] gives the operands (per-token-head codes
// with fp16 dequant factors, fp16 head weights).
//
//   I[t,s] = k_scale[s] * sum_h (w * q_scale)[t,h] * max(D[t,h,s], 0),  D = q[t,h,:] . k[s,:]
//
// Work decomposition (decode and prefill shapes alike): a workgroup owns one sequence, a group
// of G of its query tokens and a chunk of CK = 512 cached keys.  Its waves split the chunk's
// 32-key blocks; a wave keeps one token's query codes (all heads) resident in VGPRs as the MFMA
// A operand and reads key rows from LDS as the B operand (the chunk moves HBM -> LDS once per
// token group with direct loads).  The head reduction is fused: the 32x32 accumulator puts 16
// heads of one key in a lane and the other 16 in lane l^32, so the weighted ReLU sum is 16
// FMAs per M-block plus a single cross-lane add.
//
// MFMA k-permutation: the contraction runs over all D dims, so A and B only need the same
// (lane, byte) -> d assignment.  Lane half hv = lane/32 owns dims [hv*D/2, hv*D/2 + D/2) of
// both the query row and the key row, so each lane reads D/2 contiguous bytes of its key row.
#include <cstdlib>
#include <cstring>

#include "common.h"

namespace dsa {

struct IdxArgs {
  const int32_t* q_start; const int32_t* q_pos; const int64_t* kv_start;
  const uint8_t* q_codes; const void* q_scale; const u16* w;
  const uint8_t* k_cache; const void* k_scale;
  float* scores; int32_t* dots; long ld;
  uint32_t* hist; int hist_k;            // optional top-k digit histogram [T][kHistShards][kHistBins]
  int poison;                            // debug: poison LDS before use
  int H; int ngrp; int scale_f16; int B; int T;
  const int32_t* bt; int bps; int bs_log2;   // paged caches: block table (NULL: flat rows)
};

constexpr int kCK = 512;     // keys per workgroup
constexpr int kBlk = 32;     // keys per MFMA column block

// Per-lane operand of one 32x32 block: this lane's D/2 code bytes.
//  int8: D/32 MFMAs v_mfma_i32_32x32x32_i8 (k = 32, 16 bytes per lane each), exact int32.
//  fp8 : the bytes are widened to bf16 in registers (every e4m3 value is exactly a bf16;
//        v_cvt_scalef32_pk_bf16_fp8 with unit scale converts two codes per instruction) and
//        contracted on v_mfma_f32_32x32x16_bf16 (k = 16): products are exact in fp32 and the
//        sums carry fp32 rounding only (measured: within 1e-7 of the row's largest dot, under
//        one fp32 ulp of sum |a b|).  Both fp8 MFMAs (32x32x64 f8f6f4 and 32x32x16 fp8) sum with
//        a narrower internal adder: up to 2.7e-5 of the row's largest dot on the same codes
//        (about 320 ulps), above the 1e-6 a head dot may carry under the top-k near-tie rule,
//        so they are not used here (dsa_e4m3_dots runs all three).
template <bool FP8, int D>
struct KFrag;
template <int D>
struct KFrag<false, D> { v4i v[D / 32]; };
template <int D>
struct KFrag<true, D> { v8bf v[D / 16]; };

template <int D>
__device__ __forceinline__ v8bf fp8x8_to_bf16(int lo, int hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool FP8, int D>
__device__ __forceinline__ void load_row_half(KFrag<FP8, D>& f, const uint8_t* p) {
  // p: 16-byte aligned start of this lane's D/2 bytes
  const v4i* q = reinterpret_cast<const v4i*>(p);
  if constexpr (!FP8) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) f.v[j] = q[j];
  } else {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const v4i w = q[j];
      f.v[2 * j] = fp8x8_to_bf16<D>(w[0], w[1]);
      f.v[2 * j + 1] = fp8x8_to_bf16<D>(w[2], w[3]);
    }
  }
}

template <bool FP8>
struct AccT;
template <> struct AccT<false> { typedef v16i type; };
template <> struct AccT<true> { typedef v16f type; };

template <bool FP8, int D>
__device__ __forceinline__ typename AccT<FP8>::type mma_block(const KFrag<FP8, D>& a,
                                                             const KFrag<FP8, D>& b) {
  typename AccT<FP8>::type c = {};
  if constexpr (!FP8) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a.v[j], b.v[j], c, 0, 0, 0);
  } else {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v[j], b.v[j], c, 0, 0, 0);
  }
  return c;
}

// Key chunk staging.  The chunk's key rows (CK x D bytes) and its key scales are moved
// HBM -> LDS with global_load_lds_dwordx4 issued from inline asm (each lane's 16 bytes land
// at M0 + 16 * lane), all at once, in four groups of 128 keys that are consumed as they land
// (explicit s_waitcnt vmcnt).  The compiler neither sees these loads (so it does not drain
// them at every LDS read) nor can sink them.  Inside the key loop no other vector-memory
// operation is issued -- scores go to LDS and are stored once at the end -- so the manual
// vmcnt values are exact.  Row r's 16-byte chunk c sits at chunk c ^ (r % CPR): 16-byte
// reads of one chunk column by 32 consecutive rows spread over all banks.
__device__ __forceinline__ void idx_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void idx_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// 16 bytes at base + off (base wave-uniform in SGPRs) into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void dma16(const void* base, uint32_t off, unsigned lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(base), "{m0}"(lds_addr));
}

constexpr int kGroups = 4;                    // 128-key groups per chunk

// G = query tokens per workgroup (1, 2, 4); NMB = 32-head M-blocks per token (ceil(H/32)).
// Waves per workgroup (four: each 32-key block of a 128-key group goes to one wave per token
// pair; eight waves were measured no faster, the kernel being bound by its memory phases).
template <int G>
struct IdxWaves { static constexpr int value = 4; };

template <int G, int NMB, int D, bool FP8, bool DOTS, bool SF16>
__global__ void __launch_bounds__(IdxWaves<G>::value * 64) indexer_kernel(IdxArgs a) {
  constexpr int NW = IdxWaves<G>::value;
  constexpr int NT = NW * 64;
  constexpr int NPH = NW / G;                // waves sharing one token
  constexpr int CPR = D / 16;                // 16-byte chunks per key row
  constexpr int KB = kCK * D;                // chunk bytes in LDS
  constexpr int INSTR = KB / 1024;           // DMA wave-instructions for the chunk
  constexpr int PER_GROUP = INSTR / NW / kGroups;  // per thread per group
  constexpr int HT = D == 128 ? 64 : 8;                  // indexer heads of the compiled shape
  constexpr int QB = G * HT * D;                         // the group's query codes (bytes)
  constexpr int GB = kCK / kGroups * D;                  // one key group in LDS (bytes)
  constexpr int QG = QB <= GB ? 1 : QB / GB;             // key groups whose LDS holds Q first
  // Decode shapes (Q of the group <= 16 KiB): Q gets an LDS region of its own, which the
  // chunk's scores reuse once Q sits in VGPRs (80 KiB in all: two workgroups per CU), and every
  // key group is issued together with Q -- one memory round trip for all operands.  Larger
  // groups (prefill) stage Q in the last key groups' LDS and issue those groups after Q moved.
  constexpr bool SEPQ = QB <= 16384;
  constexpr int QR = SEPQ ? (QB > G * kCK * 4 ? QB : G * kCK * 4) : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char kl[KB + QR];
  __shared__ float scl_s[(DOTS || SEPQ) ? 1 : G][kCK];
  if (a.poison) {
    poison_lds(&kl, sizeof(kl));
    poison_lds(&scl_s, sizeof(scl_s));
    __syncthreads();
  }
  float (*scl)[kCK] = SEPQ ? reinterpret_cast<float (*)[kCK]>(kl + KB) : scl_s;   // scores of the chunk

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hv = lane >> 5, col = lane & 31;
  const int b = blockIdx.y / a.ngrp, g = blockIdx.y % a.ngrp;
  const int chunk0 = blockIdx.x * kCK;
  const int ti = wave % G;                   // this wave's token
  const int phase = wave / G;
  // Batch metadata.  Small batches (B < 64, T <= 64) load q_start, q_pos and kv_start as
  // lane vectors in one memory round trip and pick entries by lane; larger ones chain loads.
  int q_lo, q_hi, maxp = -1, p;
  int pg[G];                                 // positions of the group's tokens (-1: none)
  long kv0;
  // Paged caches: the chunk's physical blocks as a lane vector (block j of the chunk in lane
  // j), loaded with the metadata; flat caches: the sequence's first row.
  int bt_l = 0;
  if (a.bt) bt_l = a.bt[(long)b * a.bps + min((chunk0 >> a.bs_log2) + lane, a.bps - 1)];
  if (a.B < 64 && a.T <= 64) {
    const int qs_l = a.q_start[min(lane, a.B)];
    const int qp_l = a.q_pos[min(lane, a.T - 1)];
    const long kv_l = a.bt ? 0 : a.kv_start[min(lane, a.B - 1)];
    q_lo = __builtin_amdgcn_readlane(qs_l, b) + g * G;
    q_hi = __builtin_amdgcn_readlane(qs_l, b + 1);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      pg[j] = q_lo + j < q_hi ? __builtin_amdgcn_readlane(qp_l, min(q_lo + j, a.T - 1)) : -1;
      maxp = max(maxp, pg[j]);
    }
    const int tt = min(q_lo + ti, a.T - 1);
    p = q_lo + ti < q_hi ? __builtin_amdgcn_readlane(qp_l, tt) : -1;
    kv0 = (long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kv_l >> 32), b) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)kv_l, b));
  } else {
    q_lo = a.q_start[b] + g * G;
    q_hi = a.q_start[b + 1];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      pg[j] = q_lo + j < q_hi ? a.q_pos[q_lo + j] : -1;
      maxp = max(maxp, pg[j]);
    }
    p = q_lo + ti < q_hi ? a.q_pos[q_lo + ti] : -1;
    kv0 = a.bt ? 0 : a.kv_start[b];
  }
  // cache row of chunk row r (0 <= r < kCK)
  auto cache_row = [&](int r) -> long {
    if (!a.bt) return kv0 + chunk0 + r;
    const int pos = chunk0 + r;
    const int blk = __shfl(bt_l, (pos >> a.bs_log2) - (chunk0 >> a.bs_log2), kWave);
    return ((long)blk << a.bs_log2) + (pos & ((1 << a.bs_log2) - 1));
  };
  retire(bt_l);            // landed with the metadata; later lane shuffles of it wait for nothing
  if (q_lo >= q_hi) return;
  if (chunk0 > maxp) return;
  const int t = q_lo + ti;
  const bool live = t < q_hi;
  const int H = a.H;

  // Loads below are unconditional (clamped indices, results selected afterwards): a load
  // behind a per-element branch is issued and waited for one at a time.
  const int tc = live ? t : q_hi - 1;
  const int nvalid = min(G, q_hi - q_lo);                // query tokens of this group
  constexpr int QI = (QB + NW * 1024 - 1) / (NW * 1024); // Q loads per wave (1 KiB each)
  constexpr int QJ = QB >= 1024 ? QB / 1024 : 1;         // Q loads in all
  // decode: every key group travels with Q; prefill: key group 0 travels with Q and groups
  // 1.. are issued once Q sits in VGPRs (the last QG of them overwrite Q's LDS); either way the
  // groups are consumed as they land
  constexpr int EARLY = SEPQ ? kGroups : 1;
  constexpr unsigned QOFF = SEPQ ? KB : (kGroups - QG) * GB;   // Q's LDS offset
  static_assert(SEPQ || EARLY + QG <= kGroups, "Q staging overlaps the first key group");
  static_assert((QB <= QG * GB && QB % 1024 == 0) || QB < 1024, "Q staging does not fit");
  // Rows past the chunk's last visible key are clamped (never stored).
  const int last_row = maxp - chunk0;
  float wq[NMB][16];                                     // set once the key stream is issued

  // Key scales of the chunk for the score stores (one per key, shared by the group's tokens;
  // rows past the last visible key clamped).  Issued ahead of the direct loads, they land with
  // the first key group and their first use (the stores) comes after the last one.
  constexpr int KPT = kCK / NT;                          // keys per thread
  uint32_t ksraw[DOTS ? 1 : KPT];
  if constexpr (!DOTS) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int r = min((int)threadIdx.x + i * NT, last_row);
      const long row = a.bt ? cache_row(r) : kv0 + chunk0 + r;
      ksraw[i] = SF16 ? (uint32_t)((const u16*)a.k_scale)[row] : ((const uint32_t*)a.k_scale)[row];
    }
  }

  // ---- DMA: the group's query codes (coalesced, rows of D bytes, swizzled like the key rows)
  // into their own LDS region (decode) or the LDS of the last QG key groups (prefill), then the
  // key groups: all of them (decode), or group 0 with the rest issued once Q sits in VGPRs.
  const unsigned kl_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)kl;
  // DMA base (SGPRs): the chunk's first row (flat) or the cache (paged; rows via the table,
  // the host checks that the cache spans < 4 GiB)
  const uint8_t* kchunk = uniform_ptr(a.bt ? a.k_cache : a.k_cache + (kv0 + chunk0) * D);
  auto chunk_off = [&](int rr) -> uint32_t { return (uint32_t)((a.bt ? cache_row(rr) : (long)rr) * D); };
  // A 1-KiB piece j of Q or of the chunk covers rows j * (1024 / D) + lane * 16 / D; as 1024 / D
  // is a multiple of the swizzle period, a lane's byte offset within its piece is the same for
  // every piece.  Whole groups of a flat cache with every row in range (all but the sequence's
  // last chunk) take that offset plus the piece's start; otherwise
  // rows are clamped (to the group's last token, the chunk's last visible key) or looked up in
  // the block table per piece.
  const int lrow = lane * 16 / D;
  const uint32_t lane_off = (uint32_t)(lrow * D + ((((lane * 16) % D) >> 4) ^ (lrow & (CPR - 1))) * 16);
  const bool fast_q = (QB >= 1024 && QB % 1024 == 0) && nvalid == G;
  const bool fast_k = !a.bt && last_row >= kCK - 1;
  {
    const uint8_t* qbase = uniform_ptr(a.q_codes + (long)q_lo * H * D);
    if (fast_q) {
#pragma unroll
      for (int it = 0; it < QI; ++it) {
        const int j = min(wave + NW * it, QJ - 1);
        dma16(qbase, lane_off + (uint32_t)(j * 1024), kl_base + QOFF + j * 1024);
      }
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int it = 0; it < QI; ++it) {
        const int j = min(wave + NW * it, QJ - 1);
        const int o = j * 1024 + ln * 16;
        const int r = o / D;                               // token * HT + head
        const int c = ((o % D) >> 4) ^ (r & (CPR - 1));
        const int tok = min(r / HT, nvalid - 1);
        dma16(qbase, (uint32_t)((tok * HT + r % HT) * D + c * 16), kl_base + QOFF + j * 1024);
      }
    }
  }
  auto issue_key_pieces = [&](int it0, int it1) {
    if (fast_k) {
#pragma unroll
      for (int it = it0; it < it1; ++it) {
        const int j = wave + NW * it;
        dma16(kchunk, lane_off + (uint32_t)(j * 1024), kl_base + j * 1024);
      }
    } else {
#pragma unroll
      for (int it = it0; it < it1; ++it) {
        const int j = wave + NW * it;
        const int o = j * 1024 + lane * 16;
        const int r = o / D;
        const int c = ((o % D) >> 4) ^ (r & (CPR - 1));
        const int rr = min(r, last_row);
        dma16(kchunk, chunk_off(rr) + (uint32_t)(c * 16), kl_base + j * 1024);
      }
    }
  };
  issue_key_pieces(0, EARLY * PER_GROUP);
  asm volatile("" ::: "memory");                        // the loads below stay behind the stream
  // (w * q_scale) for the 16 accumulator rows of each M-block held by this lane: rows
  // 8 j + 4 hv + e (e < 4) of block mb are heads 32 mb + 8 j + 4 hv + e.  The wave's token rows
  // of w and q_scale are read through the scalar unit (uniform addresses in the constant
  // address space): those reads are counted apart from the direct loads of Q and the keys, so
  // waiting for them never waits for the key stream.  The key scales are applied when the
  // scores are stored.
  if constexpr (!DOTS) {
    typedef const __attribute__((address_space(4))) uint32_t cu32;
    auto uni = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); };
    const int tcu = __builtin_amdgcn_readfirstlane(tc);
    cu32* wrow = (cu32*)(a.w + (long)tcu * H);                                  // f16 pairs
    cu32* srow = (cu32*)((const char*)a.q_scale + (long)tcu * H * (SF16 ? 2 : 4));
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hb = 32 * mb + 8 * j;                  // heads hb .. hb + 7 (hv picks a half)
        if (hb >= H) {                                   // uniform: rows past H weigh nothing
#pragma unroll
          for (int e = 0; e < 4; ++e) wq[mb][4 * j + e] = 0.f;
          continue;
        }
        // both halves are read (uniform, scalar) and the lane picks one: a per-lane choice of
        // address would turn these into vector loads
        const uint32_t w0 = uni(wrow[hb / 2]), w1 = uni(wrow[hb / 2 + 1]);
        const uint32_t w2 = uni(wrow[hb / 2 + 2]), w3 = uni(wrow[hb / 2 + 3]);
        const uint32_t wa = hv ? w2 : w0, wb = hv ? w3 : w1;
        float qs[4];
        if (SF16) {
          const uint32_t s0 = uni(srow[hb / 2]), s1 = uni(srow[hb / 2 + 1]);
          const uint32_t s2 = uni(srow[hb / 2 + 2]), s3 = uni(srow[hb / 2 + 3]);
          const uint32_t sa = hv ? s2 : s0, sb = hv ? s3 : s1;
          qs[0] = f16_bits_to_f32((u16)sa); qs[1] = f16_bits_to_f32((u16)(sa >> 16));
          qs[2] = f16_bits_to_f32((u16)sb); qs[3] = f16_bits_to_f32((u16)(sb >> 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = uni(srow[hb + e]), hi = uni(srow[hb + 4 + e]);
            qs[e] = __uint_as_float(hv ? hi : lo);
          }
        }
        wq[mb][4 * j + 0] = f16_bits_to_f32((u16)wa) * qs[0];
        wq[mb][4 * j + 1] = f16_bits_to_f32((u16)(wa >> 16)) * qs[1];
        wq[mb][4 * j + 2] = f16_bits_to_f32((u16)wb) * qs[2];
        wq[mb][4 * j + 3] = f16_bits_to_f32((u16)(wb >> 16)) * qs[3];
      }
  }

  idx_wait_vm<EARLY * PER_GROUP>();                      // Q landed (for this wave)
  idx_lds_barrier();                                     // ... and for every wave
  KFrag<FP8, D> qf[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = ti * HT + min(32 * mb + col, H - 1);
    const unsigned char* qrow = kl + QOFF + r * D;
#pragma unroll
    for (int q = 0; q < CPR / 2; ++q) {
      const int cc = hv * (CPR / 2) + q;
      const v4i w = *reinterpret_cast<const v4i*>(qrow + ((cc ^ (r & (CPR - 1))) << 4));
      if constexpr (!FP8) {
        qf[mb].v[q] = w;
      } else {
        qf[mb].v[2 * q] = fp8x8_to_bf16<D>(w[0], w[1]);
        qf[mb].v[2 * q + 1] = fp8x8_to_bf16<D>(w[2], w[3]);
      }
    }
    if (32 * mb + col >= H) {                            // rows past H are zero
#pragma unroll
      for (int j = 0; j < (FP8 ? D / 16 : D / 32); ++j) qf[mb].v[j] = {};
    }
  }
  // retire every compiler-visible load (the early key groups land with them), and let every
  // wave finish reading Q before the last groups (or the scores) overwrite its LDS
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int j = 0; j < (FP8 ? D / 16 : D / 32); ++j) retire(qf[mb].v[j]);
  idx_lds_barrier();
  issue_key_pieces(EARLY * PER_GROUP, INSTR / NW);

  // ---- consume the groups as they land
#pragma unroll
  for (int grp = 0; grp < kGroups; ++grp) {
    if (grp == 0) idx_wait_vm<PER_GROUP * 3>();
    else if (grp == 1) idx_wait_vm<PER_GROUP * 2>();
    else if (grp == 2) idx_wait_vm<PER_GROUP * 1>();
    else idx_wait_vm<0>();
    idx_lds_barrier();
    if (!live) continue;
#pragma unroll
    for (int kb = grp * (kCK / kBlk / kGroups) + phase; kb < (grp + 1) * (kCK / kBlk / kGroups); kb += NPH) {
      const int sl0 = kb * kBlk;             // key row in the chunk
      const int s = chunk0 + sl0 + col;
      if (chunk0 + sl0 > p) break;
      const int r = sl0 + col;
      KFrag<FP8, D> kf;
      {
        // this lane's D/2 bytes: logical chunks hv*CPR/2 .. +CPR/2 of row r
        v4i raw[CPR / 2];
#pragma unroll
        for (int q = 0; q < CPR / 2; ++q) {
          const int cc = hv * (CPR / 2) + q;
          raw[q] = *reinterpret_cast<const v4i*>(kl + r * D + ((cc ^ (r & (CPR - 1))) << 4));
        }
        if constexpr (!FP8) {
#pragma unroll
          for (int q = 0; q < CPR / 2; ++q) kf.v[q] = raw[q];
        } else {
#pragma unroll
          for (int q = 0; q < CPR / 2; ++q) {
            kf.v[2 * q] = fp8x8_to_bf16<D>(raw[q][0], raw[q][1]);
            kf.v[2 * q + 1] = fp8x8_to_bf16<D>(raw[q][2], raw[q][3]);
          }
        }
      }
      if constexpr (DOTS) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const auto acc = mma_block<FP8, D>(qf[mb], kf);
          if (s <= p) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int h = 32 * mb + 8 * (i >> 2) + 4 * hv + (i & 3);
              if (h < H) a.dots[((long)t * H + h) * a.ld + s] = (int32_t)acc[i];
            }
          }
        }
      } else {
        float sum = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const auto acc = mma_block<FP8, D>(qf[mb], kf);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float d;
            if constexpr (FP8) d = fmaxf(acc[i], 0.f);
            else d = (float)max(acc[i], 0);
            sum = fmaf(wq[mb][i], d, sum);
          }
        }
        sum += __shfl_xor(sum, 32, kWave);
        if (hv == 0) scl[ti][r] = sum;                   // times the key scale when stored
      }
    }
  }
  if constexpr (!DOTS) {
    __syncthreads();
    // coalesced score stores, times the key scales: token j of the group, keys chunk0 ..
    // min(chunk0 + kCK, p_j + 1)
    for (int j = 0; j < G; ++j) {
      const int tj = q_lo + j;
      if (tj >= q_hi) break;
      const int n = min(kCK, pg[j] + 1 - chunk0);
      float* dst = a.scores + (long)tj * a.ld + chunk0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int e = (int)threadIdx.x + i * NT;
        if (e < n) {
          const float ks = SF16 ? f16_bits_to_f32((u16)ksraw[i]) : __uint_as_float(ksraw[i]);
          dst[e] = scl[j][e] * ks;
        }
      }
    }
  }
}

template <int G, int NMB, int D, bool FP8, bool DOTS>
static void launch(const IdxArgs& a, dim3 grid, hipStream_t st) {
  const dim3 block(IdxWaves<G>::value * 64);
  if (a.scale_f16) hipLaunchKernelGGL((indexer_kernel<G, NMB, D, FP8, DOTS, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((indexer_kernel<G, NMB, D, FP8, DOTS, false>), grid, block, 0, st, a);
}

template <int NMB, int D, bool FP8, bool DOTS>
static void launch_g(int G, const IdxArgs& a, dim3 grid, hipStream_t st) {
  if (G == 1) launch<1, NMB, D, FP8, DOTS>(a, grid, st);
  else if (G == 2) launch<2, NMB, D, FP8, DOTS>(a, grid, st);
  else launch<4, NMB, D, FP8, DOTS>(a, grid, st);
}


// Sum of lane l and lane l ^ 32 (the two 16-head halves of an MFMA column), in every lane.
__device__ __forceinline__ float add_half_swap(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(x[0]) + __uint_as_float(x[1]);
}

// ---------------------------------------------------------------------------------------------
// Prefill kernel: many query tokens per sequence, int8 codes, 64 heads x 128 dims (flat or paged).
// [LI] "Lightning Indexer" (jsqmd.com/news/787325): at prefill the indexer is a dense int8 GEMM
// per head over the chunk's tokens and the cached keys, then ReLU and the head-weighted sum.
//
// Workgroup = (sequence, tile of kPT query tokens).  The tile's query codes and w * q_scale stay
// in LDS; its kPW waves split the keys the tile sees into kPG-key groups (wave w takes groups
// w, w + kPW, ...).  A wave holds one group's key codes in registers, loaded straight from memory,
// and runs every token of the tile against them:
// 16 v_mfma_i32_32x32x32_i8 per token (2 head blocks x 2 key blocks x 4 depth steps, query
// fragments from LDS), then the ReLU-weighted head sum (3 VALU ops per (token, head, key) --
// the kernel's bound) and the key scale.  Each key group is read once per kPT tokens (the
// decode-shaped tile kernel reads it once per 4).  Causality: a token skips the groups past its
// position (wave-uniform) and masks the keys past it inside the last one.
constexpr int kPT = 16;                        // query tokens per prefill workgroup
constexpr int kPG = 64;                        // keys per wave group
constexpr int kPW = 16;                        // waves per prefill workgroup (4 per SIMD)
constexpr int kQP = 144;                       // LDS bytes per staged query row (128 + 16)

__global__ void __launch_bounds__(kPW * 64) indexer_prefill_kernel(IdxArgs a) {
  constexpr int H = 64, D = 128;
  // one LDS block: w * q_scale first, then the query codes, so that every read below is a
  // per-lane base plus an immediate offset (the offset field reaches 64 KiB)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kPT * H * 4 + kPT * H * kQP];
  float (*wq)[H] = reinterpret_cast<float (*)[H]>(lds);
  uint8_t* qs = lds + kPT * H * 4;
  if (a.poison) {
    poison_lds(&lds, sizeof(lds));
    __syncthreads();
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hv = lane >> 5, col = lane & 31;
  const int b = blockIdx.y;
  const int q0 = a.q_start[b];
  const int nseq = a.q_start[b + 1] - q0;
  if ((int)blockIdx.x * kPT >= nseq) return;                 // whole workgroup, before any barrier
  const int t0 = q0 + blockIdx.x * kPT;
  const int nt = min(kPT, nseq - (int)blockIdx.x * kPT);
  // the tile's positions as a lane vector (token j in lane j), its largest position
  const int pl = lane < nt ? a.q_pos[t0 + lane] : -1;
  int maxp = pl;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) maxp = max(maxp, __shfl_xor(maxp, m, kWave));
  const long kv0 = a.bt ? 0 : a.kv_start[b];               // paged: rows through the block table
  // stage the tile's query codes (rows kQP = 144 bytes apart: the 32 rows one fragment read
  // touches start 36 banks apart and cover all 64 banks) and head weights
  for (int o = tid * 16; o < nt * H * D; o += kPW * 64 * 16) {
    const int r = o >> 7, c = (o >> 4) & 7;
    *reinterpret_cast<uint4*>(qs + r * kQP + (c << 4)) =
        *reinterpret_cast<const uint4*>(a.q_codes + (long)t0 * H * D + o);
  }
  for (int i = tid; i < nt * H; i += kPW * 64) {
    const long ti = (long)t0 * H + i;
    const float qsv = a.scale_f16 ? f16_bits_to_f32(((const u16*)a.q_scale)[ti]) : ((const float*)a.q_scale)[ti];
    wq[i / H][i % H] = f16_bits_to_f32(a.w[ti]) * qsv;
  }
  __syncthreads();

  const int ngroups = (maxp + 1 + kPG - 1) / kPG;
  auto load_group = [&](int g, v4i (&kf)[2][4], float (&ks)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int pos = min(g * kPG + 32 * kb + col, maxp);     // positions past maxp: masked below
      const long row = a.bt ? ((long)a.bt[(long)b * a.bps + (pos >> a.bs_log2)] << a.bs_log2) +
                                  (pos & ((1 << a.bs_log2) - 1))
                            : kv0 + pos;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        kf[kb][q] = *reinterpret_cast<const v4i*>(a.k_cache + row * D + 32 * q + 16 * hv);
      ks[kb] = a.scale_f16 ? f16_bits_to_f32(((const u16*)a.k_scale)[row]) : ((const float*)a.k_scale)[row];
    }
  };
  auto load_q = [&](int j, v4i (&qf)[2][4]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        qf[mb][q] = *reinterpret_cast<const v4i*>(qs + (j * H + 32 * mb + col) * kQP +
                                                  ((2 * q + hv) << 4));
  };
  // a wave loads its group at the group's start: the other three waves of its SIMD run their
  // tokens meanwhile (a register copy of the next group in flight would cost the fourth wave)
  v4i kf[2][4];
  float ks[2];
  for (int g = wave; g < ngroups; g += kPW) {
    load_group(g, kf, ks);
    const int key0 = g * kPG;
    for (int j = 0; j < nt; ++j) {
      const int p = __builtin_amdgcn_readlane(pl, j);
      if (key0 > p) continue;
      v4i qa[2][4];
      load_q(j, qa);
      float sum[2][2] = {{0.f, 0.f}, {0.f, 0.f}};           // two partial sums per key block
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        v16i acc0 = {}, acc1 = {};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[mb][q], kf[0][q], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[mb][q], kf[1][q], acc1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 w4 = *reinterpret_cast<const float4*>(&wq[j][32 * mb + 8 * i + 4 * hv]);
          const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sum[0][r & 1] = fmaf(wv[r], (float)max(acc0[4 * i + r], 0), sum[0][r & 1]);
            sum[1][r & 1] = fmaf(wv[r], (float)max(acc1[4 * i + r], 0), sum[1][r & 1]);
          }
        }
      }
      const float s0v = add_half_swap(sum[0][0] + sum[0][1]);
      const float s1v = add_half_swap(sum[1][0] + sum[1][1]);
      if (hv == 0) {
        float* dst = a.scores + (long)(t0 + j) * a.ld;
        const int k0 = key0 + col, k1 = key0 + 32 + col;
        if (k0 <= p) dst[k0] = s0v * ks[0];
        if (k1 <= p) dst[k1] = s1v * ks[1];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Prolog inside the streaming kernel (dsa_indexer_prolog_topk).  [PRO] "Indexer Prolog"
// (jsqmd.com/news/787325): the query and the new cache key are quantized per token-head after
// Hadamard(RoPE(.)); [AQ] "Activation Quantization" (mooersco.com/news/996258, section 4, steps
// 1-3): fp32 amax, scale = amax / qmax, rne(clamp(x / scale)).
//
// One row per D/8 lanes, 8 consecutive elements per lane (element i = 8 li + e), read from LDS.
// RoPE and the Hadamard run in fp64 (products of fp32 values are exact there; one rounding to fp32
// at the end), the quantizer in fp32.  The quotient x / scale is formed as
// fp32(fp64(x) * fp64(1 / scale)): the two fp64 roundings stay within 2^-51 relative, and the
// quotient of two fp32 values is never within 2^-49 (relative) of an fp32 rounding midpoint, so
// the result is the correctly rounded fp32 division -- the same codes as dsa_indexer_prolog.
struct ProArgs {
  const void* q_in; const void* k_in; const float* cs; const float* sn;   // tables [T][rope_dim/2]
  uint8_t* q_codes; void* q_scale; uint8_t* k_cache; void* k_scale;
  int in_bf16, rope_dim, rope_offset, rope_interleaved, hadamard, round_scale;
};

template <int D, bool FP8>
__device__ __forceinline__ uint2 pro_quant8(const ProArgs& p, const unsigned char* raw,
                                            const float* cs, const float* sn, float& scale) {
  constexpr int LPR = D / 8;                               // lanes per row
  const int lane = threadIdx.x & 63, li = lane % LPR;
  float f[8];
  if (p.in_bf16) {
    const uint4 v = *reinterpret_cast<const uint4*>(raw + li * 16);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_to_f32((u16)(wv[e] & 0xFFFFu));
      f[2 * e + 1] = bf16_to_f32((u16)(wv[e] >> 16));
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(raw + li * 32);
    const float4 b = *reinterpret_cast<const float4*>(raw + li * 32 + 16);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  if (p.rope_dim > 0 || p.hadamard) {
    double x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (double)f[e];
    if (p.rope_dim > 0) {
      // partner of element i: i ^ 1 (interleaved, same lane) or i +- rope_dim / 2 (lane +- half / 8;
      // the host requires rope_offset % 8 == 0 and rope_dim % 16 == 0 for this form)
      const int half = p.rope_dim >> 1;
      const int rel0 = li * 8 - p.rope_offset;
      const bool lane_in = rel0 >= 0 && rel0 < p.rope_dim;
      double pv[8];
      if (p.rope_interleaved) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = x[e ^ 1];
      } else {
        const int src = lane_in ? lane + (rel0 < half ? half / 8 : -(half / 8)) : lane;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = __shfl(x[e], src, kWave);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rel = rel0 + e;
        if (rel >= 0 && rel < p.rope_dim) {
          bool first;
          int pair;
          if (p.rope_interleaved) { first = (rel & 1) == 0; pair = rel >> 1; }
          else { first = rel < half; pair = first ? rel : rel - half; }
          const double c = (double)cs[pair], sn_ = (double)sn[pair];
          // first of the pair: x1 c - x2 s ; second: x2 c + x1 s
          x[e] = first ? x[e] * c - pv[e] * sn_ : x[e] * c + pv[e] * sn_;
        }
      }
    }
    if (p.hadamard) {
      // natural (Sylvester) order: for stride h, (a, b) -> (a + b, a - b), a = the element whose
      // index has bit h clear; strides 1, 2, 4 inside the lane, 8 .. D/2 across lanes
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if ((e & h) == 0) {
            const double u = x[e], v = x[e + h];
            x[e] = u + v; x[e + h] = u - v;
          }
        }
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) {
        const bool hi = (li & m) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double o = __shfl_xor(x[e], m, kWave);
          x[e] = hi ? o - x[e] : x[e] + o;
        }
      }
      const double norm = D == 128 ? 0.088388347648318440550 : 0.125;   // 1/sqrt(128), 1/sqrt(64)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= norm;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)x[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  const float qmax = FP8 ? 448.0f : 127.0f;
  float s = amax / qmax;                                   // IEEE-rounded division
  if (p.round_scale && s > 0.f) {
    int ex;
    const float m = frexpf(s, &ex);                        // s = m * 2^ex, m in [0.5, 1)
    s = m == 0.5f ? s : ldexpf(1.0f, ex);
  }
  const double rs = s > 0.f ? 1.0 / (double)s : 0.0;
  uint32_t code[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float y = s > 0.f ? (float)((double)f[e] * rs) : 0.f;
    y = fminf(fmaxf(y, -qmax), qmax);
    if constexpr (FP8) code[e] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
    else code[e] = (uint32_t)(uint8_t)(int8_t)__float2int_rn(y);
  }
  scale = s;
  return uint2{code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
               code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24};
}

// ---------------------------------------------------------------------------------------------
// Streaming decode kernel (at most four query tokens per sequence).
//
// A workgroup of eight waves owns one sequence and a long span of its keys (SPAN keys, chosen on
// the host so that about one workgroup per CU covers the batch).  Every wave is its own pipeline:
// it takes every 8th (G <= 2) or 4th (G = 4, two token pairs) 32-key block of the span, streams
// those blocks HBM -> LDS by direct loads through a private ring of NB slots (NB - 1 blocks in
// flight), waits for them with its own vmcnt and never for another wave, and contracts each
// block against the query codes of its tokens (the block is read once per CU whatever G is).
// No barrier stands in the block loop, so the waves sharing a SIMD drift apart and one's
// ReLU-weighted head sum (VALU) runs under the other's MFMAs.  The query codes, the head weights
// and the query scales are staged once per workgroup (w * q_scale as a small LDS table).
// Scores stay in LDS until the span is done; a final coalesced pass multiplies them by the key
// scales (loaded before the stream, waited for only there), stores them and feeds the top-k
// histogram.
constexpr int kSNW = 8;                        // waves per workgroup
// G x SPAN scores held in LDS (with the ring and the query codes: at most 160 KiB)
__host__ __device__ constexpr int stream_scl(int G) { return G == 1 ? 8192 : 4096; }

template <int G, int D>
struct SShape {
  static constexpr int HT = D == 128 ? 64 : 8;              // heads of the compiled shape
  static constexpr int NMB = (HT + 31) / 32;                // 32-head M-blocks
  static constexpr int CPR = D / 16;                        // 16-byte chunks per key row
  static constexpr int NTW = G < 2 ? G : 2;                 // tokens per wave
  static constexpr int BSTR = kSNW / (G / NTW);             // block stride of a wave
  static constexpr int BB = 32 * D;                         // block bytes
  static constexpr int NPB = BB / 1024;                     // 1-KiB DMA pieces per block
  static constexpr int NB = D == 128 ? 3 : 6;               // ring slots per wave
  static constexpr int SCL = stream_scl(G);
  static constexpr int QB = G * HT * D;                     // query codes of the group
  static constexpr int QR = (QB + 1023) / 1024 * 1024;      // their LDS region
  static constexpr int KPT = SCL / G / (kSNW * 64);         // key scales per thread (max)
  static_assert(NB >= 3 && NB - 2 <= 6, "ring depth");
  static_assert(G * kHistBins * 4 <= kSNW * NB * BB, "histogram does not fit the ring");
};

// s_waitcnt vmcnt(P * n) for a runtime n in [0, 6]
template <int P>
__device__ __forceinline__ void wait_blocks_after(int n) {
  switch (n) {
    case 0: idx_wait_vm<0>(); break;
    case 1: idx_wait_vm<P * 1>(); break;
    case 2: idx_wait_vm<P * 2>(); break;
    case 3: idx_wait_vm<P * 3>(); break;
    case 4: idx_wait_vm<P * 4>(); break;
    case 5: idx_wait_vm<P * 5>(); break;
    default: idx_wait_vm<P * 6>(); break;
  }
}
// 4 bytes at base + off (base wave-uniform in SGPRs) into LDS at lds_addr + 4 * lane
__device__ __forceinline__ void dma4(const void* base, uint32_t off, unsigned lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" :: "v"(off), "s"(base), "{m0}"(lds_addr));
}

struct StreamArgs {
  IdxArgs a;
  int span;              // keys per workgroup (a multiple of 32 * kSNW)
  ProArgs pro;           // PRO: the prolog's inputs and outputs
};

// PRO (dsa_indexer_prolog_topk): the workgroup quantizes its group's query rows itself instead of
// loading codes.  Their raw rows (and the rotary tables, and the raw new-key rows of the group)
// move into LDS by direct loads -- into the ring slots 1 .. NB-1 of every wave, free until the
// stream's second block is issued -- together with the stream's first block; every wave then
// quantizes rows (one per D/8 lanes) into the query-code region, the last wave also the group's
// new key rows whose positions fall in this span.  The wave that consumes the block holding such
// a key copies its fresh codes over the row the stream read, the final pass uses its fresh scale,
// and the workgroup writes the new key rows (and, workgroup 0 of the sequence, the query codes
// and scales) at its end.
template <int G, int D> struct ProStage {
  static constexpr int SRB = (SShape<G, D>::NB - 1) * SShape<G, D>::BB;   // staging bytes per wave
  static constexpr int CAP = kSNW * SRB;                                   // raw query bytes that fit
};

template <int G, int D, bool FP8, bool DOTS, bool SF16, bool PRO>
__global__ void __launch_bounds__(kSNW * 64) indexer_stream_kernel(StreamArgs sa) {
  typedef SShape<G, D> S;
  constexpr int NT = kSNW * 64;
  constexpr int NTW = S::NTW;
  const IdxArgs& a = sa.a;
  const int SPAN = sa.span;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSNW * S::NB * S::BB];
  __shared__ __attribute__((aligned(1024))) unsigned char qsm[S::QR];
  __shared__ __attribute__((aligned(16))) float scl[DOTS ? 1 : S::SCL];
  __shared__ __attribute__((aligned(16))) uint32_t wraw[G * S::HT / 2 > 64 ? G * S::HT / 2 : 64];
  __shared__ __attribute__((aligned(16))) uint32_t sraw[G * S::HT * (SF16 ? 1 : 2) / 2 > 64 ? G * S::HT * (SF16 ? 1 : 2) / 2 : 64];
  __shared__ __attribute__((aligned(16))) float wqt[G][S::HT];
  __shared__ int sbt[S::SCL / G / 16 + 1];                    // paged: the span's block entries
  constexpr int PG = PRO ? G : 1;
  __shared__ __attribute__((aligned(16))) float qsc[PG][PRO ? S::HT : 1];        // query scales
  __shared__ __attribute__((aligned(16))) unsigned char newk[PG][PRO ? D : 16];  // new key codes
  __shared__ float newks[PG];                                                    // ... and scales
  __shared__ __attribute__((aligned(16))) float ptab[PRO ? 2 * G * 64 : 4];      // cos, sin rows
  __shared__ __attribute__((aligned(16))) unsigned char nkraw[PRO ? G * D * 4 : 16];   // raw new keys
  if (sa.a.poison) {
    poison_lds(&ring, sizeof(ring));
    poison_lds(&qsm, sizeof(qsm));
    poison_lds(&scl, sizeof(scl));
    poison_lds(&wraw, sizeof(wraw));
    poison_lds(&sraw, sizeof(sraw));
    poison_lds(&wqt, sizeof(wqt));
    poison_lds(&sbt, sizeof(sbt));
    poison_lds(&qsc, sizeof(qsc));
    poison_lds(&newk, sizeof(newk));
    poison_lds(&newks, sizeof(newks));
    poison_lds(&ptab, sizeof(ptab));
    poison_lds(&nkraw, sizeof(nkraw));
    __syncthreads();
  }

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hv = lane >> 5, col = lane & 31;
  const int b = blockIdx.y;
  // span sx of sequence b, rotated by b: workgroup ids go round-robin to the XCDs, and the
  // first spans of every sequence (the ones short sequences have) then spread over all of them
  const int sx = (int)((blockIdx.x + gridDim.x - blockIdx.y % gridDim.x) % gridDim.x);
  const int span0 = sx * SPAN;
  const int tw0 = (wave / S::BSTR) * NTW;                     // this wave's first token
  const int blk0 = wave % S::BSTR;                             // ... and first block

  // ---- batch metadata in one round trip (lane vectors, picked by lane) for small batches
  int t0, nq, pg[G], maxp = -1;
  long kv0;
  if (a.B < 64 && a.T <= 64) {
    const int qs_l = a.q_start[min(lane, a.B)];
    const int qp_l = a.q_pos[min(lane, a.T - 1)];
    const long kv_l = a.bt ? 0 : a.kv_start[min(lane, a.B - 1)];
    t0 = __builtin_amdgcn_readlane(qs_l, b);
    nq = min(__builtin_amdgcn_readlane(qs_l, b + 1) - t0, G);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      pg[j] = j < nq ? __builtin_amdgcn_readlane(qp_l, min(t0 + j, a.T - 1)) : -1;
      maxp = max(maxp, pg[j]);
    }
    kv0 = (long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kv_l >> 32), b) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)kv_l, b));
  } else {
    t0 = a.q_start[b];
    nq = min(a.q_start[b + 1] - t0, G);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      pg[j] = j < nq ? a.q_pos[t0 + j] : -1;
      maxp = max(maxp, pg[j]);
    }
    kv0 = a.bt ? 0 : a.kv_start[b];
  }
  if (nq <= 0 || span0 > maxp) return;
  const int nkeys = min(SPAN, maxp + 1 - span0);               // keys of the span in use
  const int last_row = nkeys - 1;                              // span-relative clamp for loads
  const int nblk = (nkeys + 31) / 32;                          // 32-key blocks of the span
  const int nbw = blk0 < nblk ? (nblk - 1 - blk0) / S::BSTR + 1 : 0;   // this wave's blocks
  const int H = a.H;

  // paged: the span's block-table entries into LDS (blocks of >= 16 keys)
  if (a.bt) {
    const int nbe = (nkeys - 1 + (span0 & ((1 << a.bs_log2) - 1))) / (1 << a.bs_log2) + 1;
    for (int i = tid; i < nbe; i += NT) sbt[i] = a.bt[(long)b * a.bps + (span0 >> a.bs_log2) + i];
    __syncthreads();
  }
  auto cache_row = [&](int r) -> long {                        // r: span-relative key
    if (!a.bt) return kv0 + span0 + r;
    const int pos = span0 + r;
    return ((long)sbt[(pos >> a.bs_log2) - (span0 >> a.bs_log2)] << a.bs_log2) + (pos & ((1 << a.bs_log2) - 1));
  };

  // ---- key scales of the span (waited for in the final pass only)
  uint32_t ksraw[DOTS ? 1 : S::KPT];
  if constexpr (!DOTS) {
#pragma unroll
    for (int i = 0; i < S::KPT; ++i) {
      const long row = cache_row(min(tid + i * NT, last_row));
      ksraw[i] = SF16 ? (uint32_t)((const u16*)a.k_scale)[row] : ((const uint32_t*)a.k_scale)[row];
    }
  }
  asm volatile("" ::: "memory");

  // ---- DMA: query codes, head weights and query scales, then this wave's first NB - 1 blocks
  const unsigned q_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)qsm;
  const unsigned ring_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)ring;
  // PRO: does a new key of the group fall in this span?
  bool has_new = false;
#pragma unroll
  for (int j = 0; j < G; ++j) has_new |= j < nq && pg[j] >= span0 && pg[j] < span0 + nkeys;
  const int insz = sa.pro.in_bf16 ? 2 : 4;
  const int rhalf = sa.pro.rope_dim >> 1;
  {
    if constexpr (!PRO) {
      const uint8_t* qsrc = uniform_ptr(a.q_codes + (long)t0 * H * D);
      const int qbytes = nq * H * D;                             // tokens past nq: clamped copies
      if constexpr (S::QB >= 1024) {
        for (int j = wave; j < S::QB / 1024; j += kSNW)
          dma16(qsrc, (uint32_t)min(j * 1024 + lane * 16, qbytes - 16), q_base + j * 1024);
      } else {
        for (int j = wave; j < (S::QB + 255) / 256; j += kSNW)
          dma4(qsrc, (uint32_t)min(j * 256 + lane * 4, qbytes - 4), q_base + j * 256);
      }
    } else {
      // raw query rows -> staging: byte o at wave (o / SRB)'s slots 1 .. NB-1, offset o % SRB
      typedef ProStage<G, D> P;
      const unsigned char* rsrc = uniform_ptr((const unsigned char*)sa.pro.q_in + (long)t0 * H * D * insz);
      const int rbytes = nq * H * D * insz;                      // <= P::CAP (host check)
      for (int j = wave; j * 1024 < rbytes; j += kSNW)
        dma16(rsrc, (uint32_t)min(j * 1024 + lane * 16, rbytes - 16),
              ring_base + (unsigned)((j * 1024 / P::SRB) * (S::NB * S::BB) + S::BB + (j * 1024) % P::SRB));
      if (wave == kSNW - 2) {
        const unsigned tab_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float*)ptab;
        if (rhalf > 0) {
          const int tbytes = nq * rhalf * 4;
          const unsigned char* csrc = uniform_ptr((const unsigned char*)sa.pro.cs + (long)t0 * rhalf * 4);
          const unsigned char* ssrc = uniform_ptr((const unsigned char*)sa.pro.sn + (long)t0 * rhalf * 4);
          for (int j = 0; j * 256 < tbytes; ++j) {
            dma4(csrc, (uint32_t)min(j * 256 + lane * 4, tbytes - 4), tab_base + j * 256);
            dma4(ssrc, (uint32_t)min(j * 256 + lane * 4, tbytes - 4), tab_base + G * 64 * 4 + j * 256);
          }
        }
        if (has_new) {
          const int kbytes = nq * D * insz;
          const unsigned char* ksrc = uniform_ptr((const unsigned char*)sa.pro.k_in + (long)t0 * D * insz);
          const unsigned nk_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)nkraw;
          if (kbytes >= 1024) {
            for (int j = 0; j * 1024 < kbytes; ++j)
              dma16(ksrc, (uint32_t)min(j * 1024 + lane * 16, kbytes - 16), nk_base + j * 1024);
          } else {
            for (int j = 0; j * 256 < kbytes; ++j)
              dma4(ksrc, (uint32_t)min(j * 256 + lane * 4, kbytes - 4), nk_base + j * 256);
          }
        }
      }
    }
    if constexpr (!DOTS) {
      if (wave == kSNW - 1) {
        const int wbytes = nq * H * 2;
        const unsigned char* wsrc = uniform_ptr((const unsigned char*)a.w + (long)t0 * H * 2);
        for (int j = 0; j < (G * S::HT * 2 + 255) / 256; ++j)
          dma4(wsrc, (uint32_t)min(j * 256 + lane * 4, wbytes - 4),
               (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)wraw + j * 256);
      }
      if (wave == kSNW - 1 && !PRO) {
        const int sb = SF16 ? 2 : 4;
        const int sbytes = nq * H * sb;
        const unsigned char* ssrc = uniform_ptr((const unsigned char*)a.q_scale + (long)t0 * H * sb);
        for (int j = 0; j < (G * S::HT * sb + 255) / 256; ++j)
          dma4(ssrc, (uint32_t)min(j * 256 + lane * 4, sbytes - 4),
               (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)sraw + j * 256);
      }
    }
  }
  // Block i of this wave is span block blk0 + BSTR * i in ring slot i % NB.  Piece j of a block
  // holds rows j * (1024 / D) + lrow; the lane's 16 bytes are chunk c of that row, stored at
  // chunk c ^ (row % CPR) (the swizzle period divides 1024 / D, so the lane offset is the same in
  // every piece and every block).
  const int lrow = lane * 16 / D;
  const int lchunk = (((lane * 16) % D) >> 4) ^ (lrow & (S::CPR - 1));
  const uint32_t lane_off = (uint32_t)(lrow * D + lchunk * 16);
  const unsigned wring = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)ring +
                         (unsigned)(wave * S::NB * S::BB);
  const uint8_t* kbase = uniform_ptr(a.bt ? a.k_cache : a.k_cache + (kv0 + span0) * D);
  auto issue_block = [&](int i) {
    const unsigned slot = wring + (unsigned)((i % S::NB) * S::BB);
    const int r0 = (blk0 + S::BSTR * i) * 32;
    if (!a.bt && r0 + 31 <= last_row) {
#pragma unroll
      for (int j = 0; j < S::NPB; ++j) dma16(kbase, (uint32_t)(r0 * D + j * 1024) + lane_off, slot + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < S::NPB; ++j) {
        const int rr = min(r0 + j * (1024 / D) + lrow, last_row);
        dma16(kbase, (uint32_t)((a.bt ? cache_row(rr) : (long)rr) * D + lchunk * 16), slot + j * 1024);
      }
    }
  };
  if constexpr (!PRO) {
    for (int i = 0; i < S::NB - 1 && i < nbw; ++i) issue_block(i);
  } else {
    // the first block, then the prolog while it is in flight
    if (nbw > 0) issue_block(0);
    wait_blocks_after<S::NPB>(nbw > 0 ? 1 : 0);               // raw rows, tables, weights landed
    idx_lds_barrier();
    typedef ProStage<G, D> P;
    constexpr int LPR = D / 8, RPW = 64 / LPR;
    const int li = lane % LPR, rp = lane / LPR;
    const int R = nq * H;
    for (int ps = wave; ps * RPW < R; ps += kSNW) {          // wave-uniform bound
      const int r = min(ps * RPW + rp, R - 1);
      const int j = r / H, h = r % H;
      const int o = r * D * insz;
      float sc;
      const uint2 c = pro_quant8<D, FP8>(sa.pro, ring + (o / P::SRB) * (S::NB * S::BB) + S::BB + o % P::SRB,
                                         ptab + j * rhalf, ptab + G * 64 + j * rhalf, sc);
      if (ps * RPW + rp < R) {
        *reinterpret_cast<uint2*>(qsm + (j * S::HT + h) * D + li * 8) = c;
        if (li == 0) qsc[j][h] = SF16 ? f16_bits_to_f32(f32_to_f16_bits(sc)) : sc;
      }
    }
    if (wave == kSNW - 1 && has_new) {
      const int j = min(rp, nq - 1);
      float sc;
      const uint2 c = pro_quant8<D, FP8>(sa.pro, nkraw + j * D * insz, ptab + j * rhalf,
                                         ptab + G * 64 + j * rhalf, sc);
      int pj = pg[0];
#pragma unroll
      for (int jj = 1; jj < G; ++jj) if (jj == j) pj = pg[jj];
      if (rp < nq && pj >= span0 && pj < span0 + nkeys) {
        *reinterpret_cast<uint2*>(&newk[j][li * 8]) = c;
        if (li == 0) newks[j] = SF16 ? f16_bits_to_f32(f32_to_f16_bits(sc)) : sc;
      }
    }
    idx_lds_barrier();                                         // codes visible; staging free
    for (int i = 1; i < S::NB - 1 && i < nbw; ++i) issue_block(i);
  }

  // ---- staging: wait for the query, weights and scales (issued before the blocks), build
  // w * q_scale, then move this wave's operands into registers
  wait_blocks_after<S::NPB>(min(S::NB - 1, nbw));
  idx_lds_barrier();
  if constexpr (!DOTS) {
    if (tid < G * S::HT) {
      const int j = tid / S::HT, h = tid % S::HT;
      const int jj = min(j, nq - 1);
      const u16 wv = ((const u16*)wraw)[jj * H + h];
      const float qsv = PRO ? qsc[PRO ? jj : 0][PRO ? h : 0]
                            : SF16 ? f16_bits_to_f32(((const u16*)sraw)[jj * H + h])
                                   : __uint_as_float(sraw[jj * H + h]);
      wqt[j][h] = f16_bits_to_f32(wv) * qsv;
    }
    idx_lds_barrier();
  }
  KFrag<FP8, D> qf[NTW][S::NMB];
  float wq[DOTS ? 1 : NTW][S::NMB][16];
  int pt[NTW];
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int ti = tw0 + u;
    pt[u] = ti < nq ? pg[ti] : -1;
#pragma unroll
    for (int mb = 0; mb < S::NMB; ++mb) {
      const int hr = min(32 * mb + col, S::HT - 1);
      const unsigned char* qrow = qsm + (ti * S::HT + hr) * D;
#pragma unroll
      for (int q = 0; q < S::CPR / 2; ++q) {
        const v4i w = *reinterpret_cast<const v4i*>(qrow + (hv * (S::CPR / 2) + q) * 16);
        if constexpr (!FP8) {
          qf[u][mb].v[q] = w;
        } else {
          qf[u][mb].v[2 * q] = fp8x8_to_bf16<D>(w[0], w[1]);
          qf[u][mb].v[2 * q + 1] = fp8x8_to_bf16<D>(w[2], w[3]);
        }
      }
      if (32 * mb + col >= S::HT) {
#pragma unroll
        for (int j = 0; j < (FP8 ? D / 16 : D / 32); ++j) qf[u][mb].v[j] = {};
      }
      if constexpr (!DOTS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (32 * mb + 8 * j >= S::HT) {
#pragma unroll
            for (int e = 0; e < 4; ++e) wq[u][mb][4 * j + e] = 0.f;
          } else {
            const float4 v = *reinterpret_cast<const float4*>(&wqt[ti][32 * mb + 8 * j + 4 * hv]);
            wq[u][mb][4 * j + 0] = v.x; wq[u][mb][4 * j + 1] = v.y;
            wq[u][mb][4 * j + 2] = v.z; wq[u][mb][4 * j + 3] = v.w;
          }
        }
      }
    }
  }

  // ---- the block loop: no barrier, each wave waits for its own loads only
  for (int i = 0; i < nbw; ++i) {
    wait_blocks_after<S::NPB>(min(S::NB - 2, nbw - 1 - i));   // block i landed
    if (i + S::NB - 1 < nbw) issue_block(i + S::NB - 1);       // into the slot of block i - 1
    const int key0 = (blk0 + S::BSTR * i) * 32;                // span-relative first key
    if (span0 + key0 > maxp) break;                            // wave-uniform (never, by nbw)
    unsigned char* tile = ring + wave * S::NB * S::BB + (i % S::NB) * S::BB;
    if constexpr (PRO) {
      // a new key of the group in this block: its fresh codes replace the row the stream read
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const int r = pg[jj] - span0 - key0;
        if (jj < nq && r >= 0 && r < 32 && lane < D / 16)
          *reinterpret_cast<uint4*>(tile + r * D + ((lane ^ (r & (S::CPR - 1))) << 4)) =
              *reinterpret_cast<const uint4*>(&newk[jj][lane * 16]);
      }
      asm volatile("" ::: "memory");
    }
    KFrag<FP8, D> kf;
    {
      v4i raw[S::CPR / 2];
#pragma unroll
      for (int q = 0; q < S::CPR / 2; ++q) {
        const int cc = hv * (S::CPR / 2) + q;
        raw[q] = *reinterpret_cast<const v4i*>(tile + col * D + ((cc ^ (col & (S::CPR - 1))) << 4));
      }
      if constexpr (!FP8) {
#pragma unroll
        for (int q = 0; q < S::CPR / 2; ++q) kf.v[q] = raw[q];
      } else {
#pragma unroll
        for (int q = 0; q < S::CPR / 2; ++q) {
          kf.v[2 * q] = fp8x8_to_bf16<D>(raw[q][0], raw[q][1]);
          kf.v[2 * q + 1] = fp8x8_to_bf16<D>(raw[q][2], raw[q][3]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int ti = tw0 + u;
      if (span0 + key0 > pt[u]) continue;                      // wave-uniform (pt = -1: no token)
      if constexpr (DOTS) {
        const int s = span0 + key0 + col;
#pragma unroll
        for (int mb = 0; mb < S::NMB; ++mb) {
          const auto acc = mma_block<FP8, D>(qf[u][mb], kf);
          if (s <= pt[u]) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int h = 32 * mb + 8 * (e >> 2) + 4 * hv + (e & 3);
              if (8 * (e >> 2) + 32 * mb < S::HT && h < H)
                a.dots[((long)(t0 + ti) * H + h) * a.ld + s] = (int32_t)acc[e];
            }
          }
        }
      } else {
        float sum = 0.f;
#pragma unroll
        for (int mb = 0; mb < S::NMB; ++mb) {
          const auto acc = mma_block<FP8, D>(qf[u][mb], kf);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            if (32 * mb + 8 * (e >> 2) >= S::HT) continue;      // compile-time: rows past H
            float d;
            if constexpr (FP8) d = fmaxf(acc[e], 0.f);
            else d = (float)max(acc[e], 0);
            sum = fmaf(wq[u][mb][e], d, sum);
          }
        }
        sum = add_half_swap(sum);
        if (hv == 0) scl[ti * SPAN + key0 + col] = sum;         // times the key scale when stored
      }
    }
  }
  if constexpr (!DOTS) {
    __syncthreads();                                             // every stream has landed
    // With the top-k's first radix pass fused (a.hist): a histogram of the top 11 key bits of
    // the span's scores per token in LDS (the ring is free), its non-zero bins then added to
    // one of the token's histogram shards.  Rows with at most hist_k valid keys get none.
    uint32_t* hl = reinterpret_cast<uint32_t*>(ring);
    if (a.hist) {
      for (int i = tid * 4; i < G * kHistBins; i += NT * 4)
        *reinterpret_cast<uint4*>(hl + i) = uint4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    for (int j = 0; j < G; ++j) {
      if (j >= nq) break;
      const int n = min(nkeys, pg[j] + 1 - span0);
      const bool hj = a.hist && pg[j] + 1 > a.hist_k;
      float* dst = a.scores + (long)(t0 + j) * a.ld + span0;
#pragma unroll
      for (int i = 0; i < S::KPT; ++i) {
        const int e = tid + i * NT;
        if (e < n) {
          float ks = SF16 ? f16_bits_to_f32((u16)ksraw[i]) : __uint_as_float(ksraw[i]);
          if constexpr (PRO) {
#pragma unroll
            for (int jj = 0; jj < G; ++jj)
              if (jj < nq && span0 + e == pg[jj]) ks = newks[jj];
          }
          const float v = scl[j * SPAN + e] * ks;
          dst[e] = v;
          if (hj) atomicAdd(&hl[j * kHistBins + (order_key(v) >> 21)], 1u);
        }
      }
    }
    if constexpr (PRO) {
      // the prolog's outputs: the group's query codes and scales (span 0 of the sequence),
      // the new key rows of this span
      if (sx == 0) {
        const int qb = nq * H * D;                               // H == HT (compiled shapes)
        for (int o = tid * 16; o < qb; o += NT * 16)
          *reinterpret_cast<uint4*>(sa.pro.q_codes + (long)t0 * H * D + o) = *reinterpret_cast<const uint4*>(qsm + o);
        for (int i = tid; i < nq * H; i += NT) {
          const float v = qsc[i / H][i % H];
          if (SF16) ((u16*)sa.pro.q_scale)[(long)t0 * H + i] = f32_to_f16_bits(v);
          else ((float*)sa.pro.q_scale)[(long)t0 * H + i] = v;
        }
      }
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        if (jj < nq && pg[jj] >= span0 && pg[jj] < span0 + nkeys) {
          const long row = kv0 + pg[jj];
          if (tid < D / 16)
            *reinterpret_cast<uint4*>(sa.pro.k_cache + row * D + tid * 16) = *reinterpret_cast<const uint4*>(&newk[jj][tid * 16]);
          if (tid == 0) {
            if (SF16) ((u16*)sa.pro.k_scale)[row] = f32_to_f16_bits(newks[jj]);
            else ((float*)sa.pro.k_scale)[row] = newks[jj];
          }
        }
      }
    }
    if (a.hist) {
      __syncthreads();
      uint32_t* gh = a.hist + (long)blockIdx.x % kHistShards * kHistBins;
      for (int i = tid; i < G * kHistBins; i += NT) {
        const int j = i / kHistBins;
        const uint32_t c = hl[i];
        if (c && j < nq)
          atomicAdd(gh + (long)(t0 + j) * kHistShards * kHistBins + (i % kHistBins), c);
      }
    }
  }
}

template <int G, int D, bool FP8, bool DOTS, bool PRO>
static void launch_stream(const StreamArgs& sa, dim3 grid, hipStream_t st) {
  if (sa.a.scale_f16) hipLaunchKernelGGL((indexer_stream_kernel<G, D, FP8, DOTS, true, PRO>), grid, dim3(kSNW * 64), 0, st, sa);
  else hipLaunchKernelGGL((indexer_stream_kernel<G, D, FP8, DOTS, false, PRO>), grid, dim3(kSNW * 64), 0, st, sa);
}

template <int D, bool FP8, bool DOTS, bool PRO = false>
static void launch_stream_g(int G, const StreamArgs& sa, dim3 grid, hipStream_t st) {
  if (G == 1) launch_stream<1, D, FP8, DOTS, PRO>(sa, grid, st);
  else if (G == 2) launch_stream<2, D, FP8, DOTS, PRO>(sa, grid, st);
  else launch_stream<4, D, FP8, DOTS, PRO>(sa, grid, st);
}
// raw query bytes the PRO kernel can stage for a group of G tokens
static int pro_capacity(int G, int D) {
  if (D == 128) return G == 1 ? ProStage<1, 128>::CAP : G == 2 ? ProStage<2, 128>::CAP : ProStage<4, 128>::CAP;
  return G == 1 ? ProStage<1, 64>::CAP : G == 2 ? ProStage<2, 64>::CAP : ProStage<4, 64>::CAP;
}

}  // namespace dsa

using dsa_host::fail;

static dsa_status check_batch(const dsa_batch* bt, const char* fn, bool need_kv = true) {
  if (!bt) return fail(DSA_ERR_INVALID_ARG, "%s: batch is NULL", fn);
  if (bt->num_seqs < 0 || bt->num_q < 0) return fail(DSA_ERR_INVALID_ARG, "%s: negative batch size", fn);
  if (bt->num_q > 0) {
    if (bt->num_seqs < 1) return fail(DSA_ERR_INVALID_ARG, "%s: tokens without sequences", fn);
    if (!bt->q_start || !bt->q_seq || !bt->q_pos || (need_kv && !bt->kv_start))
      return fail(DSA_ERR_INVALID_ARG, "%s: a batch array is NULL", fn);
    if (bt->max_q_per_seq < 1 || bt->max_q_per_seq > bt->num_q)
      return fail(DSA_ERR_INVALID_ARG, "%s: max_q_per_seq out of range (%d)", fn, bt->max_q_per_seq);
    if (bt->max_kv_len < 1) return fail(DSA_ERR_INVALID_ARG, "%s: max_kv_len must be >= 1", fn);
  }
  return DSA_OK;
}

// exported for the other translation units
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn) { return check_batch(bt, fn); }
dsa_status dsa_check_batch_paged(const dsa_batch* bt, const char* fn) { return check_batch(bt, fn, false); }

// A paged layout for batch bt: table present, block size a power of two in [16, 1024], enough
// blocks per sequence, and num_blocks * block_size rows of row_bytes spanning < 4 GiB.
// Returns the block size's log2 through bs_log2.
dsa_status dsa_check_paging(const dsa_paging* pg, const dsa_batch* bt, double row_bytes,
                            const char* fn, int* bs_log2) {
  if (!pg) return fail(DSA_ERR_INVALID_ARG, "%s: paging is NULL", fn);
  const int bs = pg->block_size;
  if (bs < 16 || bs > 1024 || (bs & (bs - 1)))
    return fail(DSA_ERR_INVALID_ARG, "%s: block_size must be a power of two in [16, 1024] (got %d)", fn, bs);
  int l = 0;
  while ((1 << l) < bs) ++l;
  *bs_log2 = l;
  if (bt->num_q == 0) return DSA_OK;
  if (!pg->block_table) return fail(DSA_ERR_INVALID_ARG, "%s: block_table is NULL", fn);
  if (pg->num_blocks < 1) return fail(DSA_ERR_INVALID_ARG, "%s: num_blocks must be >= 1", fn);
  if ((long)pg->blocks_per_seq * bs < bt->max_kv_len)
    return fail(DSA_ERR_INVALID_ARG, "%s: blocks_per_seq * block_size (%ld) < max_kv_len (%d)", fn,
                (long)pg->blocks_per_seq * bs, bt->max_kv_len);
  if ((double)pg->num_blocks * bs * row_bytes >= 4294967296.0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: the paged cache must span < 4 GiB", fn);
  return DSA_OK;
}

static dsa_status indexer_common(const dsa_batch* bt, int H, int D, dsa_dtype code, dsa_dtype sdt,
                                 const void* q, const void* qs, const void* w, const void* k,
                                 const void* ks, float* scores, int32_t* dots, bool want_dots,
                                 long ld, uint32_t* hist, int hist_k, void* stream, const char* fn,
                                 const dsa_paging* pg = nullptr, const dsa::ProArgs* pro = nullptr,
                                 bool validate_only = false) {
  dsa_status st = check_batch(bt, fn, pg == nullptr);
  if (st != DSA_OK) return st;
  int bs_log2 = 0;
  if (pg) {
    st = dsa_check_paging(pg, bt, (double)D, fn, &bs_log2);
    if (st != DSA_OK) return st;
  }
  if (!((H == 64 && D == 128) || (H == 8 && D == 64)))
    return fail(DSA_ERR_UNSUPPORTED, "%s: (H, D) = (%d, %d) not compiled; supported (64,128), (8,64)", fn, H, D);
  if (code != DSA_I8 && code != DSA_FP8_E4M3) return fail(DSA_ERR_UNSUPPORTED, "%s: code dtype must be I8 or FP8_E4M3", fn);
  if (!want_dots && sdt != DSA_F16 && sdt != DSA_F32) return fail(DSA_ERR_UNSUPPORTED, "%s: scale dtype must be F16 or F32", fn);
  if (bt->num_q == 0) return DSA_OK;
  if (!q || !k || (want_dots ? !dots : (!qs || !w || !ks || !scores)))
    return fail(DSA_ERR_INVALID_ARG, "%s: a data pointer is NULL", fn);
  if (ld < bt->max_kv_len) return fail(DSA_ERR_INVALID_ARG, "%s: ld (%ld) < max_kv_len (%d)", fn, ld, bt->max_kv_len);
  if (!want_dots && (ld % 4)) return fail(DSA_ERR_INVALID_ARG, "%s: ld must be a multiple of 4", fn);
  if (((uintptr_t)q | (uintptr_t)k) & 15) return fail(DSA_ERR_INVALID_ARG, "%s: q/k codes must be 16-byte aligned", fn);
  // the token rows of w and q_scale are read as whole dwords
  if (!want_dots && (((uintptr_t)qs | (uintptr_t)w) & 15))
    return fail(DSA_ERR_INVALID_ARG, "%s: q_scale and w must be 16-byte aligned", fn);

  dsa::IdxArgs a{};
  a.q_start = bt->q_start; a.q_pos = bt->q_pos; a.kv_start = bt->kv_start;
  a.q_codes = (const uint8_t*)q; a.q_scale = qs; a.w = (const dsa::u16*)w;
  a.k_cache = (const uint8_t*)k; a.k_scale = ks; a.scores = scores; a.dots = dots; a.ld = ld;
  a.hist = hist; a.hist_k = hist_k;
  a.poison = dsa_host::debug_poison();
  a.H = H; a.scale_f16 = sdt == DSA_F16; a.B = bt->num_seqs; a.T = bt->num_q;
  if (pg) { a.bt = pg->block_table; a.bps = pg->blocks_per_seq; a.bs_log2 = bs_log2; }
  const int G = bt->max_q_per_seq >= 3 ? 4 : bt->max_q_per_seq;
  a.ngrp = (bt->max_q_per_seq + G - 1) / G;
  const long gy = (long)bt->num_seqs * a.ngrp;
  if (gy > 65535L) return fail(DSA_ERR_INVALID_ARG, "%s: too many token groups", fn);
  // only the streaming kernel accumulates the top-k's histogram (decode groups)
  if (hist && a.ngrp != 1) return fail(DSA_ERR_UNSUPPORTED, "%s: fused histogram needs at most 4 tokens per sequence", fn);
  if (pro) {
    if (a.ngrp != 1 || pg)
      return fail(DSA_ERR_UNSUPPORTED, "%s: decode batches (at most 4 query tokens per sequence) on a flat cache only", fn);
    const long rbytes = (long)G * H * D * (pro->in_bf16 ? 2 : 4);
    if (rbytes > dsa::pro_capacity(G, D))
      return fail(DSA_ERR_UNSUPPORTED, "%s: %d query tokens per sequence of %s rows exceed the in-kernel staging (%ld > %d bytes)",
                  fn, bt->max_q_per_seq, pro->in_bf16 ? "bf16" : "fp32", rbytes, dsa::pro_capacity(G, D));
  }
  if (validate_only) return DSA_OK;
  hipStream_t s = (hipStream_t)stream;
  const bool fp8 = code == DSA_FP8_E4M3;
  if (a.ngrp == 1) {
    // decode: the streaming kernel, spans (multiples of 256 keys) sized for about one
    // workgroup per CU
    const int gk = 32 * dsa::kSNW;
    const long groups = (long)(bt->max_kv_len + gk - 1) / gk;
    long sg = (groups * bt->num_seqs + 255) / 256;
    const long sg_max = dsa::stream_scl(G) / G / gk;
    if (sg < 1) sg = 1;
    if (sg > sg_max) sg = sg_max;
    dsa::StreamArgs sa{a, (int)(sg * gk), pro ? *pro : dsa::ProArgs{}};
    const dim3 grid((unsigned)((bt->max_kv_len + sa.span - 1) / sa.span), (unsigned)bt->num_seqs);
    if (pro) {
      if (D == 128) {
        if (fp8) dsa::launch_stream_g<128, true, false, true>(G, sa, grid, s);
        else dsa::launch_stream_g<128, false, false, true>(G, sa, grid, s);
      } else {
        if (fp8) dsa::launch_stream_g<64, true, false, true>(G, sa, grid, s);
        else dsa::launch_stream_g<64, false, false, true>(G, sa, grid, s);
      }
    } else if (D == 128) {
      if (want_dots) { if (fp8) return fail(DSA_ERR_UNSUPPORTED, "%s: int8 only", fn); dsa::launch_stream_g<128, false, true>(G, sa, grid, s); }
      else if (fp8) dsa::launch_stream_g<128, true, false>(G, sa, grid, s);
      else dsa::launch_stream_g<128, false, false>(G, sa, grid, s);
    } else {
      if (want_dots) { if (fp8) return fail(DSA_ERR_UNSUPPORTED, "%s: int8 only", fn); dsa::launch_stream_g<64, false, true>(G, sa, grid, s); }
      else if (fp8) dsa::launch_stream_g<64, true, false>(G, sa, grid, s);
      else dsa::launch_stream_g<64, false, false>(G, sa, grid, s);
    }
    return dsa_host::check_launch(fn);
  }
  if (!want_dots && !fp8 && !hist && H == 64 && D == 128) {
    // many tokens per sequence, no fused histogram (the top-k's row workgroups build their own):
    // the prefill kernel, one workgroup per (sequence, tile of kPT tokens)
    const dim3 pgrid((unsigned)((bt->max_q_per_seq + dsa::kPT - 1) / dsa::kPT), (unsigned)bt->num_seqs);
    hipLaunchKernelGGL(dsa::indexer_prefill_kernel, pgrid, dim3(dsa::kPW * 64), 0, s, a);
    return dsa_host::check_launch(fn);
  }
  const dim3 grid((unsigned)((bt->max_kv_len + dsa::kCK - 1) / dsa::kCK), (unsigned)gy);
  if (D == 128) {
    if (want_dots) { if (fp8) return fail(DSA_ERR_UNSUPPORTED, "%s: int8 only", fn); dsa::launch_g<2, 128, false, true>(G, a, grid, s); }
    else if (fp8) dsa::launch_g<2, 128, true, false>(G, a, grid, s);
    else dsa::launch_g<2, 128, false, false>(G, a, grid, s);
  } else {
    if (want_dots) { if (fp8) return fail(DSA_ERR_UNSUPPORTED, "%s: int8 only", fn); dsa::launch_g<1, 64, false, true>(G, a, grid, s); }
    else if (fp8) dsa::launch_g<1, 64, true, false>(G, a, grid, s);
    else dsa::launch_g<1, 64, false, false>(G, a, grid, s);
  }
  return dsa_host::check_launch(fn);
}

extern "C" dsa_status dsa_indexer_scores(const dsa_batch* batch, int32_t H, int32_t D,
                                         dsa_dtype code_dtype, dsa_dtype scale_dtype,
                                         const void* q_codes, const void* q_scale, const void* w,
                                         const void* k_cache, const void* k_scale, float* scores,
                                         int64_t ld, void* stream) {
  return indexer_common(batch, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                        k_scale, scores, nullptr, false, ld, nullptr, 0, stream, "dsa_indexer_scores");
}

extern "C" dsa_status dsa_indexer_scores_paged(const dsa_batch* batch, const dsa_paging* paging,
                                               int32_t H, int32_t D, dsa_dtype code_dtype,
                                               dsa_dtype scale_dtype, const void* q_codes,
                                               const void* q_scale, const void* w,
                                               const void* k_cache, const void* k_scale,
                                               float* scores, int64_t ld, void* stream) {
  const char* fn = "dsa_indexer_scores_paged";
  if (!paging) return fail(DSA_ERR_INVALID_ARG, "%s: paging is NULL", fn);
  return indexer_common(batch, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                        k_scale, scores, nullptr, false, ld, nullptr, 0, stream, fn, paging);
}

// Scores plus the fused first radix pass of the top-k (used by dsa_indexer_topk[_paged]).
dsa_status dsa_indexer_scores_hist(const dsa_batch* batch, int32_t H, int32_t D, dsa_dtype code_dtype,
                                   dsa_dtype scale_dtype, const void* q_codes, const void* q_scale,
                                   const void* w, const void* k_cache, const void* k_scale,
                                   float* scores, int64_t ld, uint32_t* hist, int32_t k,
                                   void* stream, const char* fn, const dsa_paging* paging,
                                   bool validate_only) {
  return indexer_common(batch, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                        k_scale, scores, nullptr, false, ld, hist, k, stream, fn, paging, nullptr,
                        validate_only);
}

dsa_status dsa_prolog_own_keys(const dsa_prolog_cfg* cfg, const dsa_batch* bt, const void* q_in,
                               const float* q_cos, const float* q_sin, void* q_codes, void* q_scale,
                               const void* k_in, void* k_cache, void* k_scale, void* stream);

// Schedules of dsa_indexer_prolog_topk.  The in-kernel prolog repeats the group's query
// quantization in every span workgroup of the sequence (measured on the part: about 3.4 us per
// workgroup for 2 tokens x 64 heads of fp32 rows, against 2-5 us for a separate prolog launch),
// so it is taken only where a sequence has few spans; the decision depends on the shapes alone.
constexpr int kFusedMaxSpans = 16;

// The indexer half of dsa_indexer_prolog_topk: the prolog (inside the streaming kernel, or as its
// own launch), then the scores and the top-k's first radix pass.  cfg has been validated.
dsa_status dsa_indexer_prolog_scores_hist(const dsa_prolog_cfg* cfg, const dsa_batch* batch,
                                          const void* q_in, const float* q_cos, const float* q_sin,
                                          const void* k_in, const void* w, void* q_codes, void* q_scale,
                                          void* k_cache, void* k_scale, float* scores, int64_t ld,
                                          uint32_t* hist, int32_t k, void* stream, const char* fn,
                                          bool validate_only) {
  dsa_status st = check_batch(batch, fn);
  if (st != DSA_OK || batch->num_q == 0) return st;
  if (!q_in || !k_in || !q_codes || !q_scale || !k_cache || !k_scale)
    return fail(DSA_ERR_INVALID_ARG, "%s: a prolog pointer is NULL", fn);
  if (cfg->rope_dim > 0 && (!q_cos || !q_sin)) return fail(DSA_ERR_INVALID_ARG, "%s: q_cos/q_sin is NULL", fn);
  if (((uintptr_t)q_in | (uintptr_t)k_in) & 15) return fail(DSA_ERR_INVALID_ARG, "%s: q_in/k_in must be 16-byte aligned", fn);
  if (((uintptr_t)q_cos | (uintptr_t)q_sin) & 3) return fail(DSA_ERR_INVALID_ARG, "%s: q_cos/q_sin must be 4-byte aligned", fn);
  if (!((cfg->H == 64 && cfg->D == 128) || (cfg->H == 8 && cfg->D == 64)))
    return fail(DSA_ERR_UNSUPPORTED, "%s: (H, D) = (%d, %d) not compiled; supported (64,128), (8,64)", fn, cfg->H, cfg->D);
  // the in-kernel form: decode groups whose raw query rows fit the staging, rope pairs inside a
  // lane's 8 elements or 8-lane apart, and few spans per sequence
  const int G = batch->max_q_per_seq >= 3 ? 4 : batch->max_q_per_seq;
  const long rbytes = (long)G * cfg->H * cfg->D * (cfg->in_dtype == DSA_BF16 ? 2 : 4);
  const int gk = 32 * dsa::kSNW;
  long sg = ((long)(batch->max_kv_len + gk - 1) / gk * batch->num_seqs + 255) / 256;
  sg = sg < 1 ? 1 : (sg > dsa::stream_scl(G) / G / gk ? dsa::stream_scl(G) / G / gk : sg);
  const long spans = (batch->max_kv_len + sg * gk - 1) / (sg * gk);
  bool in_kernel = batch->max_q_per_seq <= 4 && rbytes <= dsa::pro_capacity(G, cfg->D) &&
                   (cfg->rope_dim == 0 || (cfg->rope_offset % 8 == 0 && cfg->rope_dim % 16 == 0)) &&
                   spans <= kFusedMaxSpans;
  if (const char* e = getenv("DSA_PROLOG_SCHEDULE")) {      // testing: force a schedule where legal
    if (!strcmp(e, "separate")) in_kernel = false;
    else if (!strcmp(e, "fused") && batch->max_q_per_seq <= 4 && rbytes <= dsa::pro_capacity(G, cfg->D) &&
             (cfg->rope_dim == 0 || (cfg->rope_offset % 8 == 0 && cfg->rope_dim % 16 == 0)))
      in_kernel = true;
  }
  if (!in_kernel) {
    st = indexer_common(batch, cfg->H, cfg->D, cfg->code_dtype, cfg->scale_dtype, q_codes, q_scale, w,
                        k_cache, k_scale, scores, nullptr, false, ld, hist, k, nullptr, fn, nullptr,
                        nullptr, /*validate_only=*/true);
    if (st != DSA_OK || validate_only) return st;
    st = dsa_prolog_own_keys(cfg, batch, q_in, q_cos, q_sin, q_codes, q_scale, k_in, k_cache, k_scale, stream);
    if (st != DSA_OK) return st;
    return indexer_common(batch, cfg->H, cfg->D, cfg->code_dtype, cfg->scale_dtype, q_codes, q_scale, w,
                          k_cache, k_scale, scores, nullptr, false, ld, hist, k, stream, fn);
  }
  dsa::ProArgs p{};
  p.q_in = q_in; p.k_in = k_in; p.cs = q_cos; p.sn = q_sin;
  p.q_codes = (uint8_t*)q_codes; p.q_scale = q_scale; p.k_cache = (uint8_t*)k_cache; p.k_scale = k_scale;
  p.in_bf16 = cfg->in_dtype == DSA_BF16; p.rope_dim = cfg->rope_dim; p.rope_offset = cfg->rope_offset;
  p.rope_interleaved = cfg->rope_interleaved; p.hadamard = cfg->hadamard; p.round_scale = cfg->round_scale;
  return indexer_common(batch, cfg->H, cfg->D, cfg->code_dtype, cfg->scale_dtype, q_codes, q_scale, w,
                        k_cache, k_scale, scores, nullptr, false, ld, hist, k, stream, fn, nullptr, &p,
                        validate_only);
}

extern "C" dsa_status dsa_indexer_dots_i32(const dsa_batch* batch, int32_t H, int32_t D,
                                           const int8_t* q_codes, const int8_t* k_cache,
                                           int32_t* dots, int64_t ld, void* stream) {
  return indexer_common(batch, H, D, DSA_I8, DSA_F32, q_codes, nullptr, nullptr, k_cache, nullptr,
                        nullptr, dots, true, ld, nullptr, 0, stream, "dsa_indexer_dots_i32");
}

// ---------------------------------------------------------------------------------------------
// Test hook for the choice of the fp8 indexer contraction: C = A B^T over e4m3 codes on one of
// three matrix-core paths.  One wave per 32 x 32 block of C; per 16-deep step the lane holding
// row (or column) l % 32 supplies the 8 codes at depth 8 (l / 32) of that step, for A and B
// alike, so every path forms the same products and differs only in how it sums them.
namespace dsa {
__global__ void __launch_bounds__(64) e4m3_dots_kernel(const uint8_t* A, const uint8_t* B, int n,
                                                       int d, int path, float* C) {
  const int lane = threadIdx.x;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const uint8_t* ar = A + (long)(i0 + (lane & 31)) * d + 8 * (lane >> 5);
  const uint8_t* br = B + (long)(j0 + (lane & 31)) * d + 8 * (lane >> 5);
  v16f acc = {};
  if (path == DSA_CONTRACT_FP8_K64) {
    // v_mfma_scale_f32_32x32x64_f8f6f4, both operands e4m3 (format 0), unit E8M0 scales (127)
    for (int k0 = 0; k0 < d; k0 += 64) {
      v8i a8, b8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint2 av = *reinterpret_cast<const uint2*>(ar + k0 + 16 * s);
        const uint2 bv = *reinterpret_cast<const uint2*>(br + k0 + 16 * s);
        a8[2 * s] = (int)av.x; a8[2 * s + 1] = (int)av.y;
        b8[2 * s] = (int)bv.x; b8[2 * s + 1] = (int)bv.y;
      }
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc, 0, 0, 0, 127, 0, 127);
    }
  } else if (path == DSA_CONTRACT_FP8_K16) {
    for (int k0 = 0; k0 < d; k0 += 16) {
      const long av = *reinterpret_cast<const long*>(ar + k0);
      const long bv = *reinterpret_cast<const long*>(br + k0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av, bv, acc, 0, 0, 0);
    }
  } else {
    // the fp8 indexer's own contraction: codes widened to bf16, v_mfma_f32_32x32x16_bf16
    for (int k0 = 0; k0 < d; k0 += 16) {
      const uint2 av = *reinterpret_cast<const uint2*>(ar + k0);
      const uint2 bv = *reinterpret_cast<const uint2*>(br + k0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16<0>((int)av.x, (int)av.y),
                                                    fp8x8_to_bf16<0>((int)bv.x, (int)bv.y), acc, 0, 0, 0);
    }
  }
  // 32 x 32 accumulator: register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    C[(long)i * n + j0 + (lane & 31)] = acc[r];
  }
}
}  // namespace dsa

extern "C" dsa_status dsa_e4m3_dots(const uint8_t* a, int32_t m, const uint8_t* b, int32_t n,
                                    int32_t d, int32_t contraction, float* c, void* stream) {
  const char* fn = "dsa_e4m3_dots";
  if (contraction != DSA_CONTRACT_BF16 && contraction != DSA_CONTRACT_FP8_K64 &&
      contraction != DSA_CONTRACT_FP8_K16)
    return fail(DSA_ERR_INVALID_ARG, "%s: unknown contraction %d", fn, contraction);
  if (m < 0 || n < 0 || m % 32 || n % 32) return fail(DSA_ERR_INVALID_ARG, "%s: m and n must be multiples of 32", fn);
  if (d <= 0 || d % 64 || d > 4096) return fail(DSA_ERR_INVALID_ARG, "%s: d must be a multiple of 64 in [64, 4096]", fn);
  if (m == 0 || n == 0) return DSA_OK;
  if (!a || !b || !c) return fail(DSA_ERR_INVALID_ARG, "%s: a data pointer is NULL", fn);
  if (((uintptr_t)a | (uintptr_t)b) & 15) return fail(DSA_ERR_INVALID_ARG, "%s: a and b must be 16-byte aligned", fn);
  if ((uintptr_t)c & 3) return fail(DSA_ERR_INVALID_ARG, "%s: c must be 4-byte aligned", fn);
  if ((long)m / 32 > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: m must be < 2097152", fn);
  hipLaunchKernelGGL(dsa::e4m3_dots_kernel, dim3((unsigned)(n / 32), (unsigned)(m / 32)), dim3(64), 0,
                     (hipStream_t)stream, a, b, n, d, (int)contraction, c);
  return dsa_host::check_launch(fn);
}
