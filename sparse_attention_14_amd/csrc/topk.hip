// Top-k token selection on gfx950: exact radix select over order-preserving fp32 keys.
//
// [LI] "Lightning Indexer" (jsqmd.com/news/787325): the indexer ends in a TopK; the page
// points at its single-core sort-and-merge tail at batch 4 and proposes sorting inside the
// preceding vector stage and merging at the end.  Here every stage spreads a row over many
// workgroups, so a decode batch of 8 rows still occupies the whole chip:
//
//   hist    : the top 11 bits of every key, per row, in a 2048-bin histogram (its own pass,
//             or, for decode batches, fused into the streaming indexer by dsa_indexer_topk)
//   select  : one workgroup per 4096-score chunk derives the digit b1 that holds the k-th
//             largest key; positions above b1 go into the chunk's position bitmap, positions
//             with digit b1 (candidates, 1-3 % of a Gaussian-like row) into the chunk's
//             candidate list
//   finalize: again one workgroup per chunk.  Each one loads every candidate of its row and
//             resolves the exact k-th key K* with two more digits (the same answer in every
//             workgroup), counts what the earlier chunks contribute to the selection, and
//             writes its own chunk's selected positions at that offset: ascending output with
//             no sort and no cross-workgroup exchange, ties to the lower position.
// A workgroup's work is a short instruction stream after one memory round trip; the
// alternatives (one workgroup per row, or device-scope fences between workgroups) cost
// several microseconds of issue time or L2 write-back on this part.  Rows whose candidate
// lists overflow (near-constant scores, massive ties) resolve K* by streaming the row again.
//
// [SFA] step 2: slots past the selection are -1.  Keys: fp32 bits, sign-flipped so that
// unsigned order equals numeric order; -0.0 is mapped to +0.0 first.
#include <algorithm>
#include <stdlib.h>
#include <string.h>

#include "common.h"

namespace dsa {

constexpr int kBins = kHistBins;     // 11-bit digits
constexpr int kShards = kHistShards; // copies of each row histogram (spread atomic traffic)
constexpr int kNT = 1024;            // threads per workgroup
constexpr int kChunk = kTkChunk;     // scores per chunk: one float4 per thread
static_assert(kChunk == 4 * kNT, "a select workgroup reads one float4 per thread");
constexpr int kCW = kTkCW;           // bitmap words per chunk
constexpr int kMaxLen = 64 * kChunk; // longest row
constexpr int kCap = kTkCap;         // candidate slots per chunk
constexpr int kLoadC = kTkLoad / kNT; // candidate entries per finalize thread (first trip)
constexpr int kLoad2 = 2 * kLoadC;   // second trip: every slot of a row of up to 16 chunks
static_assert(kLoad2 * kNT == 16 * kCap, "the second trip covers 16 chunks of kCap slots");
constexpr int kStreamC = 4;          // chunks whose scores are in flight at once (streamed rows)
constexpr int kRNT = 512;            // threads of a row workgroup (many-row batches)
constexpr int kRNW = kRNT / 64;      // its waves
constexpr int kRJ = 32;              // float4 slots per thread per segment
constexpr int kQJ = 8;               // slots per ordered-prefix pass
constexpr int kSeg = 4 * kRJ * kRNT; // scores per segment (65536)
constexpr int kLc = 12288;           // compacted entries held in LDS
constexpr int kRowMinT = 256;        // batches of at least this many rows take one workgroup per row

// Workspace (zero-filled before the first call; every call leaves the histograms zero-filled
// again, and the rest is written before it is read):
//   hist  [T][kShards][kBins] u32   row histogram of the top digit
//   bg    [T][2] u32                the row's threshold digit b1 and the count above it
//   cnt   [T][nch] u32              per chunk: n_above | n_cand << 16
//   bits  [T][nch][kCW] u32         per chunk: positions above b1
//   slots [T][nch][kCap] u64        per chunk: candidates, key << 32 | position
struct TkArgs {
  const int32_t* q_pos; const float* scores; long ld; int k; int T; int nch;
  int32_t* idx; uint32_t* hist; uint32_t* bg; uint32_t* cnt; uint32_t* bits; uint64_t* slots;
  uint32_t* hist2;                   // optional [T][kBins]: the candidates' second digits (select)
  int poison;                        // debug: poison LDS before use
};

// Keeps the loads issued above it in place: the compiler would otherwise sink loads that only
// the non-returning path uses below an early-exit branch, which costs a second memory round
// trip (the branch waits for q_pos first).  No wait is implied.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// This thread's four scores of chunk ch (positions ch * kChunk + 4 tid .. +3); every address
// lies inside the row's ld columns, positions past p are masked by the caller.
__device__ __forceinline__ float4 load4(const float* row, long ld, int ch) {
  const long e0 = min((long)ch * kChunk + 4 * threadIdx.x, (ld & ~3L) - 4);
  return *reinterpret_cast<const float4*>(row + e0);
}

// First pass (when the indexer did not accumulate it): histogram of the top 11 key bits of a
// chunk in LDS; non-zero bins are added to shard (chunk % kShards) of the row's.
__global__ void __launch_bounds__(kNT) topk_hist(TkArgs a) {
  __shared__ uint32_t h[kBins];
  if (a.poison) {
    poison_lds(&h, sizeof(h));
    __syncthreads();
  }
  const int t = blockIdx.y, ch = blockIdx.x;
  const int p = a.q_pos[t];
  const float4 v = load4(a.scores + (long)t * a.ld, a.ld, ch);
  issue_fence();
  if (p + 1 <= a.k || ch * kChunk > p) return;
  for (int i = threadIdx.x; i < kBins; i += kNT) h[i] = 0u;
  __syncthreads();
  const int e0 = ch * kChunk + 4 * threadIdx.x;
  const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (e0 + q <= p) atomicAdd(&h[order_key(f[q]) >> 21], 1u);
  __syncthreads();
  uint32_t* gh = a.hist + ((long)t * kShards + ch % kShards) * kBins;
  for (int i = threadIdx.x; i < kBins; i += kNT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Select: one workgroup per chunk.  One memory round trip (q_pos, the row histogram and the
// chunk's scores), the threshold digit b1 from the histogram, then the chunk's bitmap of
// positions above b1 and its candidates (digit == b1) in position order (block scan).
__global__ void __launch_bounds__(kNT) topk_select(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[kNT / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t bw[kCW];
  if (a.poison) {
    poison_lds(&h, sizeof(h));
    poison_lds(&sh, sizeof(sh));
    poison_lds(&res, sizeof(res));
    poison_lds(&bw, sizeof(bw));
    __syncthreads();
  }
  const int t = blockIdx.y, ch = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = a.q_pos[t];
  const float4 v = load4(a.scores + (long)t * a.ld, a.ld, ch);
  // the upper half of every shard first (digits 1024..2047: keys of scores >= +0); the k-th
  // largest score of a row is positive in practice, and the lower half is loaded only when
  // the upper half holds fewer than k keys
  static_assert(kBins == 2 * kNT, "one digit of each half per thread");
  const uint32_t* gh = a.hist + (long)t * kShards * kBins;
  uint32_t hv[kShards];
#pragma unroll
  for (int sd = 0; sd < kShards; ++sd) hv[sd] = gh[sd * kBins + kNT + tid];
  issue_fence();
  const int k = a.k;
  if (p + 1 <= k || ch * kChunk > p) return;             // short rows: finalize writes them
  uint32_t x = 0;
#pragma unroll
  for (int sd = 0; sd < kShards; ++sd) x += hv[sd];
  h[kNT + tid] = x;
  h[tid] = 0u;
  if (tid < kCW) bw[tid] = 0u;
  if (tid == 0) res[0] = 0xFFFFFFFFu;
  {
    // thread tid holds digit kNT + tid, so the digits above it are the threads above it: one
    // block scan over the registers finds the digit of the k-th largest key in the upper half
    // (the LDS copy serves the rare lower-half search below)
    uint32_t all;
    const uint32_t pre = block_excl_scan<kNT>(x, sh, all);
    const uint32_t above = all - pre - x;
    if (above < (uint32_t)k && (uint32_t)k <= above + x) { res[0] = kNT + tid; res[1] = above; }
    __syncthreads();
  }
  if (res[0] == 0xFFFFFFFFu) {                            // block-uniform: the lower half too
    uint32_t y = 0;
#pragma unroll
    for (int sd = 0; sd < kShards; ++sd) y += gh[sd * kBins + tid];
    h[tid] = y;
    __syncthreads();
    find_digit_desc<kNT>(h, (uint32_t)k, sh, res);
  }
  const uint32_t b1 = res[0];
  const int e0 = ch * kChunk + 4 * tid;
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t keys[4];
  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    keys[q] = order_key(f[q]);
    const bool ok = e0 + q <= p;
    const uint32_t d = keys[q] >> 21;
    gtm |= (uint32_t)(ok && d > b1) << q;
    eqm |= (uint32_t)(ok && d == b1) << q;
  }
  if (gtm) atomicOr(&bw[tid >> 3], gtm << (4 * (tid & 7)));
  if (a.hist2 && eqm) {                                  // the row's second-digit histogram
    uint32_t* h2 = a.hist2 + (long)t * kBins;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if ((eqm >> q) & 1u) atomicAdd(&h2[(keys[q] >> 10) & 0x7FFu], 1u);
  }
  const uint32_t mine = (uint32_t)__popc(gtm) | ((uint32_t)__popc(eqm) << 16);
  uint32_t tot;
  const uint32_t before = block_excl_scan<kNT>(mine, sh, tot);   // also publishes bw
  uint32_t o = before >> 16;                                      // candidates before this thread
  uint64_t* slot = a.slots + ((long)t * a.nch + ch) * kCap;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if ((eqm >> q) & 1u) {
      if (o < (uint32_t)kCap) slot[o] = ((uint64_t)keys[q] << 32) | (uint32_t)(e0 + q);
      ++o;
    }
  if (tid < kCW) a.bits[((long)t * a.nch + ch) * kCW + tid] = bw[tid];
  if (tid == 0) {
    a.cnt[(long)t * a.nch + ch] = tot;
    if (ch == 0) { a.bg[2 * t] = b1; a.bg[2 * t + 1] = res[1]; }
  }
}

// Finalize: one workgroup per chunk again.
//  * One memory round trip: q_pos, b1 and G (the count above b1), every chunk's counts, the
//    first entries of every chunk's candidate list (kLoadC per thread) and this chunk's bitmap
//    words.
//  * The second radix digit (11 bits) b2 over the row's candidates, then the third (10 bits)
//    give the exact k-th key K*; take_eq is how many keys equal to K* to keep (the lowest
//    positions).  Every workgroup of the row computes the same values.
//  * The selection before this chunk: the earlier chunks' counts above b1, plus their
//    candidates above K*, plus the ties at K* they keep.  This chunk's own selection (bitmap
//    words, its candidates above K*, its kept ties) is written from there in position order.
// Rows whose candidate lists are longer than the first trip loads take a second trip over
// every slot when the row has at most 16 chunks and no chunk overflowed its slots (a short row
// with a crowded digit); otherwise (massive ties, near-constant scores) they take their
// candidates from the row's scores, kStreamC chunks in flight at a time.  Chunk 0 writes short
// rows and zeroes the row's histogram shards for the next call.
__global__ void __launch_bounds__(kNT) topk_finalize(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[kNT / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t scnt[64];
  __shared__ uint32_t flag;
  __shared__ uint32_t bw[kCW];
  __shared__ uint32_t tw[kCW];
  __shared__ uint32_t red[4];
  if (a.poison) {
    poison_lds(&h, sizeof(h));
    poison_lds(&sh, sizeof(sh));
    poison_lds(&res, sizeof(res));
    poison_lds(&scnt, sizeof(scnt));
    poison_lds(&flag, sizeof(flag));
    poison_lds(&bw, sizeof(bw));
    poison_lds(&tw, sizeof(tw));
    poison_lds(&red, sizeof(red));
    __syncthreads();
  }
  const int t = blockIdx.y, ch = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch_m = a.nch;
  const float* row = a.scores + (long)t * a.ld;
  // ---- one round trip
  const int p = a.q_pos[t];
  const uint32_t b1 = a.bg[2 * t], G = a.bg[2 * t + 1];
  const uint32_t my_cnt = a.cnt[(long)t * nch_m + min(tid, nch_m - 1)];     // masked below
  const uint32_t gw = a.bits[((long)t * nch_m + ch) * kCW + min(tid, kCW - 1)];
  // first-trip candidate entries: entry f of the row's lists is chunk f >> sl, slot f & (2^sl - 1)
  int sl = 31 - __clz((kLoadC * kNT) / nch_m);
  sl = min(sl, 9);                                        // kCap = 512
  const uint64_t* srow = a.slots + (long)t * nch_m * kCap;
  uint64_t ev[kLoad2];                                    // [kLoadC, kLoad2): second trip only
#pragma unroll
  for (int u = 0; u < kLoadC; ++u) {
    const int f = tid + u * kNT;
    ev[u] = srow[(long)min(f >> sl, nch_m - 1) * kCap + (f & ((1 << sl) - 1))];
  }
  issue_fence();
  const int k = a.k;
  int32_t* out = a.idx + (long)t * k;
  if (p + 1 <= k) {                                       // short row: everything, then -1
    if (ch == 0)
      for (int j = tid; j < k; j += kNT) out[j] = j <= p ? j : -1;
    return;
  }
  if (ch * kChunk > p) return;
  if (ch == 0) {                                          // nothing below reads the histogram
    uint32_t* gh = a.hist + (long)t * kShards * kBins;
    for (int i = tid; i < kShards * kBins; i += kNT) gh[i] = 0u;
  }
  const int nch = p / kChunk + 1;                         // chunks of this row
  for (int i = tid; i < kBins; i += kNT) h[i] = 0u;
  if (tid < 64) scnt[tid] = tid < nch ? my_cnt : 0u;     // tid < nch <= nch_m
  if (tid == 0) flag = 0u;
  if (tid < kCW) { bw[tid] = gw; tw[tid] = 0u; }
  if (tid < 4) red[tid] = 0u;
  __syncthreads();
  // bit 0: a chunk holds more candidates than the first trip read; bit 1: more than its slots
  if (tid < nch && (my_cnt >> 16) > (1u << sl)) atomicOr(&flag, (my_cnt >> 16) > (uint32_t)kCap ? 3u : 1u);
  // candidate validity without branches: every count read first (chunk f >> sl <= 63, as
  // 2^sl >= 64 for rows of at most 64 chunks; chunks past the row read 0)
  uint32_t cn[kLoadC];
#pragma unroll
  for (int u = 0; u < kLoadC; ++u) cn[u] = scnt[(tid + u * kNT) >> sl];
  uint32_t cvalid = 0;
#pragma unroll
  for (int u = 0; u < kLoadC; ++u)
    cvalid |= (uint32_t)((uint32_t)((tid + u * kNT) & ((1 << sl) - 1)) < (cn[u] >> 16)) << u;
  __syncthreads();                                        // flag
  const uint32_t fl = flag;
  // Rows of at most 16 chunks whose lists fit their slots but not the first trip's share (a
  // short row with a crowded digit) read every slot in a second trip; the rest stream the row.
  const bool streamed = (fl & 2u) != 0u || (fl != 0u && nch * kCap > kLoad2 * kNT);
  if (fl != 0u && !streamed) {                            // block-uniform
#pragma unroll
    for (int u = 0; u < kLoad2; ++u) {
      const int f = tid + u * kNT;                        // chunk f >> 9 < 16, slot f & 511
      ev[u] = srow[(long)min(f >> 9, nch_m - 1) * kCap + (f & (kCap - 1))];
    }
    cvalid = 0;
#pragma unroll
    for (int u = 0; u < kLoad2; ++u) {
      const int f = tid + u * kNT;
      cvalid |= (uint32_t)((uint32_t)(f & (kCap - 1)) < (scnt[f >> 9] >> 16)) << u;
    }
  }
  const uint32_t need = (uint32_t)k - G;                  // 1 <= need <= #candidates
  // every candidate of the row: from the first trip, or from the row's scores
  auto each_cand = [&](auto&& fn) {
    if (!streamed) {
#pragma unroll
      for (int u = 0; u < kLoad2; ++u)
        if ((cvalid >> u) & 1u) fn((uint32_t)(ev[u] >> 32), (uint32_t)ev[u]);
    } else {
      for (int c0 = 0; c0 < nch; c0 += kStreamC) {      // kStreamC chunks' loads in flight
        float4 x[kStreamC];
#pragma unroll
        for (int j = 0; j < kStreamC; ++j) x[j] = load4(row, a.ld, min(c0 + j, nch - 1));
#pragma unroll
        for (int j = 0; j < kStreamC; ++j) {
          if (c0 + j >= nch) break;
          const float ff[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
          const int e0 = (c0 + j) * kChunk + 4 * tid;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t key = order_key(ff[q]);
            if (e0 + q <= p && (key >> 21) == b1) fn(key, (uint32_t)(e0 + q));
          }
        }
      }
    }
  };
  each_cand([&](uint32_t key, uint32_t) { atomicAdd(&h[(key >> 10) & 0x7FFu], 1u); });
  __syncthreads();
  find_digit_desc<kNT>(h, need, sh, res);
  const uint32_t b2 = res[0];
  const uint32_t need2 = need - res[1];                   // >= 1, among the b2 bin
  __syncthreads();
  for (int i = tid; i < kBins; i += kNT) h[i] = 0u;
  __syncthreads();
  each_cand([&](uint32_t key, uint32_t) {
    if (((key >> 10) & 0x7FFu) == b2) atomicAdd(&h[key & 0x3FFu], 1u);
  });
  __syncthreads();
  find_digit_desc<kNT>(h, need2, sh, res);
  const uint32_t kstar = (b1 << 21) | (b2 << 10) | res[0];
  const uint32_t n_eq = h[res[0]];
  const uint32_t take_eq = need2 - res[1];                // >= 1
  const bool all_ties = n_eq == take_eq;
  // earlier chunks: their candidates above K* and their ties at K*; this chunk's own
  // candidates above K* (bitmap) and its ties (tie bitmap)
  const uint32_t c0 = (uint32_t)ch * kChunk, c1 = c0 + kChunk;
  uint32_t gt_before = 0, eq_before = 0;
  each_cand([&](uint32_t key, uint32_t pos) {
    if (pos < c0) {
      gt_before += key > kstar;
      eq_before += key == kstar;
    } else if (pos < c1) {
      if (key > kstar) atomicOr(&bw[(pos - c0) >> 5], 1u << (pos & 31));
      else if (key == kstar) atomicOr(&tw[(pos - c0) >> 5], 1u << (pos & 31));
    }
  });
  uint32_t above_b1 = 0;                                  // earlier chunks' counts above b1
  for (int c = 0; c < ch; ++c) above_b1 += scnt[c] & 0xFFFFu;
  gt_before += __shfl_xor(gt_before, 1, kWave); gt_before += __shfl_xor(gt_before, 2, kWave);
  gt_before += __shfl_xor(gt_before, 4, kWave); gt_before += __shfl_xor(gt_before, 8, kWave);
  gt_before += __shfl_xor(gt_before, 16, kWave); gt_before += __shfl_xor(gt_before, 32, kWave);
  eq_before += __shfl_xor(eq_before, 1, kWave); eq_before += __shfl_xor(eq_before, 2, kWave);
  eq_before += __shfl_xor(eq_before, 4, kWave); eq_before += __shfl_xor(eq_before, 8, kWave);
  eq_before += __shfl_xor(eq_before, 16, kWave); eq_before += __shfl_xor(eq_before, 32, kWave);
  if ((tid & 63) == 0) {
    if (gt_before) atomicAdd(&red[0], gt_before);
    if (eq_before) atomicAdd(&red[1], eq_before);
  }
  __syncthreads();
  const uint32_t ties_before = red[1];
  const uint32_t ties_left = ties_before >= take_eq ? 0u : take_eq - ties_before;   // for this chunk
  const uint32_t start = above_b1 + red[0] + min(ties_before, take_eq);
  // this chunk's words: bitmap | kept ties; thread w < kCW owns word w (position order)
  uint32_t word = 0, tie = 0;
  if (tid < kCW) { word = bw[tid]; tie = tw[tid]; }
  uint32_t ntie = (uint32_t)__popc(tie);
  uint32_t tot;
  uint32_t r = block_excl_scan<kNT>(ntie, sh, tot);       // ties before this word, in the chunk
  if (all_ties) {
    word |= tie;
  } else {
    uint32_t m = tie;
    while (m && r < ties_left) { const uint32_t lb = m & (0u - m); word |= lb; m ^= lb; ++r; }
  }
  const uint32_t nb = (uint32_t)__popc(word);
  __syncthreads();                                        // sh reuse
  uint32_t o = start + block_excl_scan<kNT>(nb, sh, tot);
  const int base = (int)c0 + tid * 32;
  while (word) {
    const int bit = __ffs(word) - 1;
    word &= word - 1;
    if (o < (uint32_t)k) out[o] = base + bit;
    ++o;
  }
}

// Ordered exclusive prefix over (slot j, thread) of per-thread counts c[j], j < NJ: the element
// of slot j of thread t comes after every element of slots < j and after slot j of threads < t.
// tbl: LDS [NJ * kRNW + 1]; ends with a barrier after which tbl may be reused.
template <int NJ>
__device__ __forceinline__ void prefix2d(const uint32_t (&c)[NJ], uint32_t (&off)[NJ],
                                         uint32_t& total, uint32_t* tbl) {
  static_assert(NJ * kRNW % 64 == 0 && NJ * kRNW <= 256, "one wave scans the table");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    inc[j] = wave_incl_scan(c[j]);
    if (lane == 63) tbl[j * kRNW + w] = inc[j];
  }
  __syncthreads();
  if (threadIdx.x < 64) {                     // NJ x kRNW wave totals in (slot, wave) order
    constexpr int Q = NJ * kRNW / 64;
    uint32_t x[Q], sum = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) { x[q] = tbl[lane * Q + q]; sum += x[q]; }
    const uint32_t incl = wave_incl_scan(sum);
    uint32_t run = incl - sum;
#pragma unroll
    for (int q = 0; q < Q; ++q) { tbl[lane * Q + q] = run; run += x[q]; }
    if (lane == 63) tbl[NJ * kRNW] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NJ; ++j) off[j] = tbl[j * kRNW + w] + inc[j] - c[j];
  total = tbl[NJ * kRNW];
  __syncthreads();
}

// This thread's float4 slots of segment s (positions s * kSeg + 4 * (tid + kRNT * j) .. + 3);
// addresses are clamped into the row's ld columns, positions past p are masked by the caller.
__device__ __forceinline__ void load_seg(float4 (&v)[kRJ], const float* row, long ld, int s) {
#pragma unroll
  for (int j = 0; j < kRJ; ++j) {
    const long e0 = min((long)s * kSeg + 4 * ((long)threadIdx.x + (long)kRNT * j), (ld & ~3L) - 4);
    v[j] = *reinterpret_cast<const float4*>(row + e0);
  }
}

__device__ __forceinline__ float f4get(const float4& v, int r) {
  return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}

__device__ __forceinline__ void issue_fence_row() { asm volatile("" ::: "memory"); }

// Many-row batches (a prefill chunk: thousands of rows): one workgroup per row finishes the
// selection on its own, with no second launch.  One memory round trip brings the row's first
// 65536 scores (registers), from which the workgroup builds the row's first-digit histogram in
// LDS (later segments are streamed again); every key with digit >= b1 is compacted into
// LDS in position order (an ordered prefix over (float4 slot, thread)); two more digits over the
// candidates give K*; the selection is one ordered pass over the compacted list.  Rows with more
// entries than LDS holds re-read the row for each pass.  On a decode batch of a few rows this
// is slower than spreading each row over its chunks (one CU's ALUs order 65536 keys in ~15 us),
// which is why it serves many-row batches only.
__global__ void __launch_bounds__(kRNT) topk_row(TkArgs a) {
  __shared__ __attribute__((aligned(16))) uint64_t lst[kLc];       // compacted (key << 32 | pos)
  __shared__ __attribute__((aligned(16))) uint32_t h[kBins];
  __shared__ uint32_t tbl[kQJ * kRNW + 1];
  __shared__ uint32_t sh[kRNT / 64];
  __shared__ uint32_t res[2];
  if (a.poison) {
    poison_lds(&lst, sizeof(lst));
    poison_lds(&h, sizeof(h));
    poison_lds(&tbl, sizeof(tbl));
    poison_lds(&sh, sizeof(sh));
    poison_lds(&res, sizeof(res));
    __syncthreads();
  }
  const int t = blockIdx.x, tid = threadIdx.x;
  const int k = a.k;
  const float* row = a.scores + (long)t * a.ld;
  // ---- one round trip: q_pos and the first segment
  const int p = a.q_pos[t];
  float4 v[kRJ];
  load_seg(v, row, a.ld, 0);
  issue_fence_row();
  int32_t* out = a.idx + (long)t * k;
  if (p + 1 <= k) {                                  // a short row: everything, then -1
    for (int j = tid; j < k; j += kRNT) out[j] = j <= p ? j : -1;
    return;
  }
  const int L = p + 1;
  const int nseg = (L + kSeg - 1) / kSeg;
  // ---- the first digit's histogram over the row
  {
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q * kRNT + tid] = 0u;
    __syncthreads();
    // segment 0 from the registers, later segments through a small buffer (the registers keep
    // segment 0 for the compaction)
#pragma unroll
    for (int j = 0; j < kRJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * (tid + kRNT * j) + r < L) atomicAdd(&h[order_key(f4get(v[j], r)) >> 21], 1u);
    for (int s = 1; s < nseg; ++s)
      for (int j0 = 0; j0 < kRJ; j0 += kQJ) {
        float4 w[kQJ];
#pragma unroll
        for (int j = 0; j < kQJ; ++j) {
          const long e0 = min((long)s * kSeg + 4 * ((long)tid + (long)kRNT * (j0 + j)), (a.ld & ~3L) - 4);
          w[j] = *reinterpret_cast<const float4*>(row + e0);
        }
#pragma unroll
        for (int j = 0; j < kQJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (s * kSeg + 4 * (tid + kRNT * (j0 + j)) + r < L)
              atomicAdd(&h[order_key(f4get(w[j], r)) >> 21], 1u);
      }
  }
  if (tid == 0) { res[0] = 0u; res[1] = 0u; }
  __syncthreads();
  find_digit_desc<kRNT>(h, (uint32_t)k, sh, res);
  const uint32_t b1 = res[0];
  const uint32_t need = (uint32_t)k - res[1];        // >= 1 keys of digit b1 are taken
  // ---- keys with digit >= b1, compacted in position order
  // (slots are position-major, so each group of kQJ slots is compacted on its own)
  constexpr int HJ = kQJ;
  uint32_t n_list = 0;
  for (int s = 0; s < nseg; ++s) {
    if (s > 0) load_seg(v, row, a.ld, s);
#pragma unroll
    for (int hh = 0; hh < kRJ / kQJ; ++hh) {
      uint32_t c[HJ], off[HJ], tot;
#pragma unroll
      for (int jj = 0; jj < HJ; ++jj) {
        const int j = hh * HJ + jj;
        c[jj] = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = s * kSeg + 4 * (tid + kRNT * j) + r;
          c[jj] += pos < L && (order_key(f4get(v[j], r)) >> 21) >= b1;
        }
      }
      prefix2d<HJ>(c, off, tot, tbl);
#pragma unroll
      for (int jj = 0; jj < HJ; ++jj) {
        const int j = hh * HJ + jj;
        uint32_t o = n_list + off[jj];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = s * kSeg + 4 * (tid + kRNT * j) + r;
          const uint32_t key = order_key(f4get(v[j], r));
          if (pos < L && (key >> 21) >= b1) {
            if (o < (uint32_t)kLc) lst[o] = ((uint64_t)key << 32) | (uint32_t)pos;
            ++o;
          }
        }
      }
      n_list += tot;
    }
  }
  __syncthreads();
  const bool listed = n_list <= (uint32_t)kLc;
  // every key of digit b1, from the list or (rows too long for it) from the scores
  auto each_cand = [&](auto&& fn) {
    if (listed) {
      for (uint32_t f = tid; f < n_list; f += kRNT) {
        const uint64_t e = lst[f];
        const uint32_t key = (uint32_t)(e >> 32);
        if ((key >> 21) == b1) fn(key);
      }
    } else {
      for (int s = 0; s < nseg; ++s) {
        load_seg(v, row, a.ld, s);
#pragma unroll
        for (int j = 0; j < kRJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t key = order_key(f4get(v[j], r));
            if (s * kSeg + 4 * (tid + kRNT * j) + r < L && (key >> 21) == b1) fn(key);
          }
      }
    }
  };
  // ---- two more digits: the exact k-th key K*
#pragma unroll
  for (int q = 0; q < 4; ++q) h[q * kRNT + tid] = 0u;
  if (tid == 0) { res[0] = 0u; res[1] = 0u; }
  __syncthreads();
  each_cand([&](uint32_t key) { atomicAdd(&h[(key >> 10) & 0x7FFu], 1u); });
  __syncthreads();
  find_digit_desc<kRNT>(h, need, sh, res);
  const uint32_t b2 = res[0];
  const uint32_t need2 = need - res[1];
#pragma unroll
  for (int q = 0; q < 4; ++q) h[q * kRNT + tid] = 0u;
  if (tid == 0) { res[0] = 0u; res[1] = 0u; }
  __syncthreads();
  each_cand([&](uint32_t key) {
    if (((key >> 10) & 0x7FFu) == b2) atomicAdd(&h[key & 0x3FFu], 1u);
  });
  __syncthreads();
  find_digit_desc<kRNT>(h, need2, sh, res);
  const uint32_t kstar = (b1 << 21) | (b2 << 10) | res[0];
  const uint32_t take_eq = need2 - res[1];          // >= 1 keys equal to K* are taken
  // ---- the selection, in position order: keys above K*, and the first take_eq keys equal to K*
  if (listed) {
    constexpr int PER = (kLc + kRNT - 1) / kRNT;     // list entries per thread (a contiguous run)
    const uint32_t e0 = (uint32_t)tid * PER;
    uint32_t keys[PER];
    uint32_t nt = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      keys[u] = e0 + u < n_list ? (uint32_t)(lst[e0 + u] >> 32) : 0u;
      nt += e0 + u < n_list && keys[u] == kstar;
    }
    uint32_t tt;
    uint32_t rank = block_excl_scan<kRNT>(nt, sh, tt);   // equal keys before this run
    uint32_t nsel = 0, selm = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      bool sel = false;
      if (e0 + u < n_list) {
        if (keys[u] > kstar) sel = true;
        else if (keys[u] == kstar) { sel = rank < take_eq; ++rank; }
      }
      selm |= (uint32_t)sel << u;
      nsel += sel;
    }
    __syncthreads();
    uint32_t st;
    uint32_t o = block_excl_scan<kRNT>(nsel, sh, st);
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if ((selm >> u) & 1u) {
        if (o < (uint32_t)k) out[o] = (int32_t)(uint32_t)lst[e0 + u];
        ++o;
      }
  } else {
    uint32_t o_base = 0, t_base = 0;
    for (int s = 0; s < nseg; ++s) {
      load_seg(v, row, a.ld, s);
#pragma unroll
      for (int hh = 0; hh < kRJ / kQJ; ++hh) {
        uint32_t c[HJ], off[HJ], tot;
#pragma unroll
        for (int jj = 0; jj < HJ; ++jj) {
          const int j = hh * HJ + jj;
          c[jj] = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            c[jj] += s * kSeg + 4 * (tid + kRNT * j) + r < L && order_key(f4get(v[j], r)) == kstar;
        }
        prefix2d<HJ>(c, off, tot, tbl);              // equal keys before each slot
        uint32_t sc[HJ], soff[HJ], stot;
#pragma unroll
        for (int jj = 0; jj < HJ; ++jj) {
          const int j = hh * HJ + jj;
          sc[jj] = 0;
          uint32_t rank = t_base + off[jj];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t key = order_key(f4get(v[j], r));
            if (s * kSeg + 4 * (tid + kRNT * j) + r < L) {
              if (key > kstar) ++sc[jj];
              else if (key == kstar) { sc[jj] += rank < take_eq; ++rank; }
            }
          }
        }
        prefix2d<HJ>(sc, soff, stot, tbl);
#pragma unroll
        for (int jj = 0; jj < HJ; ++jj) {
          const int j = hh * HJ + jj;
          uint32_t o = o_base + soff[jj];
          uint32_t rank = t_base + off[jj];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int pos = s * kSeg + 4 * (tid + kRNT * j) + r;
            const uint32_t key = order_key(f4get(v[j], r));
            if (pos < L) {
              bool sel = key > kstar;
              if (key == kstar) { sel = rank < take_eq; ++rank; }
              if (sel) { if (o < (uint32_t)k) out[o] = pos; ++o; }
            }
          }
        }
        o_base += stot;
        t_base += tot;
      }
    }
  }
}

}  // namespace dsa

using dsa_host::fail;
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn);
dsa_status dsa_check_batch_paged(const dsa_batch* bt, const char* fn);

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static int tk_nch(int32_t max_kv_len) { return (max_kv_len + dsa::kChunk - 1) / dsa::kChunk; }

// Workspace: the row histograms at the start (the only part that must stay zero between
// calls), the other regions (written before they are read) packed against the end of the
// caller's buffer.  A buffer sized for the largest num_q and max_kv_len of a series of calls
// then never lets one call's lists land on another call's histogram rows.
struct TkLayout { size_t hist, bg, cnt, bits, slots, others; };
static TkLayout tk_layout(int32_t T, int32_t max_kv_len) {
  TkLayout L{};
  const int nch = tk_nch(max_kv_len);
  L.hist = align256((size_t)T * dsa::kShards * dsa::kBins * 4);
  L.bg = 0;                                              // offsets within the other regions
  L.cnt = L.bg + align256((size_t)T * 2 * 4);
  L.bits = L.cnt + align256((size_t)T * nch * 4);
  L.slots = L.bits + align256((size_t)T * nch * dsa::kCW * 4);
  L.others = L.slots + align256((size_t)T * nch * dsa::kCap * 8);
  return L;
}

extern "C" size_t dsa_topk_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k) {
  (void)k;
  if (num_q <= 0 || max_kv_len <= 0) return 0;
  const TkLayout L = tk_layout(num_q, max_kv_len);
  return L.hist + L.others;
}

// Validates a top-k call and fills the kernel arguments (no launch).
static dsa_status topk_prepare(const dsa_batch* bt, const float* scores, int64_t ld, int32_t k,
                               int32_t* idx, void* ws, size_t ws_bytes, const char* fn,
                               dsa::TkArgs* out, bool paged = false) {
  // the top-k reads positions only: a paged batch needs no kv_start
  dsa_status st = paged ? dsa_check_batch_paged(bt, fn) : dsa_check_batch(bt, fn);
  if (st != DSA_OK) return st;
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "%s: k must be in [1, 2048] (got %d)", fn, k);
  if (bt->num_q == 0) return DSA_OK;
  if (!scores || !idx) return fail(DSA_ERR_INVALID_ARG, "%s: scores/idx is NULL", fn);
  if (ld < bt->max_kv_len || ld % 4) return fail(DSA_ERR_INVALID_ARG, "%s: ld must be >= max_kv_len and a multiple of 4", fn);
  if ((uintptr_t)scores & 15) return fail(DSA_ERR_INVALID_ARG, "%s: scores must be 16-byte aligned", fn);
  if (bt->max_kv_len > dsa::kMaxLen) return fail(DSA_ERR_UNSUPPORTED, "%s: max_kv_len above %d", fn, dsa::kMaxLen);
  if (bt->num_q > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: more than 65535 query tokens", fn);
  const TkLayout L = tk_layout(bt->num_q, bt->max_kv_len);
  if (!ws || ws_bytes < L.hist + L.others) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, L.hist + L.others);
  if ((uintptr_t)ws & 255) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  dsa::TkArgs a{};
  a.q_pos = bt->q_pos; a.scores = scores; a.ld = ld; a.k = k; a.T = bt->num_q; a.idx = idx;
  a.nch = tk_nch(bt->max_kv_len);
  a.poison = dsa_host::debug_poison();
  char* w = (char*)ws;
  char* o = w + ((ws_bytes - L.others) & ~(size_t)255);   // >= w + L.hist
  a.hist = (uint32_t*)w;
  a.bg = (uint32_t*)(o + L.bg);
  a.cnt = (uint32_t*)(o + L.cnt);
  a.bits = (uint32_t*)(o + L.bits);
  a.slots = (uint64_t*)(o + L.slots);
  *out = a;
  return DSA_OK;
}

// Select + finalize (the row histograms are already in the workspace).
static void topk_tail(const dsa::TkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.nch, (unsigned)a.T);
  if (a.poison)                                          // written by select before finalize reads
    dsa_host::poison_fill(a.bg, (size_t)((const char*)(a.slots + (size_t)a.T * a.nch * dsa::kCap) - (const char*)a.bg), s);
  hipLaunchKernelGGL(dsa::topk_select, grid, dim3(dsa::kNT), 0, s, a);
  hipLaunchKernelGGL(dsa::topk_finalize, grid, dim3(dsa::kNT), 0, s, a);
}

// The top-k after the scores: one workgroup per row for many-row batches (it builds its own
// histogram), else (histogram pass unless the indexer accumulated it) select + finalize.
static void topk_after_scores(dsa::TkArgs& a, bool rows, bool hist_done, hipStream_t s) {
  if (rows) {
    hipLaunchKernelGGL(dsa::topk_row, dim3((unsigned)a.T), dim3(dsa::kRNT), 0, s, a);
    return;
  }
  if (!hist_done)
    hipLaunchKernelGGL(dsa::topk_hist, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kNT), 0, s, a);
  topk_tail(a, s);
}

extern "C" dsa_status dsa_topk(const dsa_batch* bt, const float* scores, int64_t ld, int32_t k,
                               int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_topk";
  dsa::TkArgs a{};
  const dsa_status st = topk_prepare(bt, scores, ld, k, idx, ws, ws_bytes, fn, &a);
  if (st != DSA_OK || bt->num_q == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  if (a.T >= dsa::kRowMinT) {                            // the row workgroups build their histograms
    hipLaunchKernelGGL(dsa::topk_row, dim3((unsigned)a.T), dim3(dsa::kRNT), 0, s, a);
    return dsa_host::check_launch(fn);
  }
  hipLaunchKernelGGL(dsa::topk_hist, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kNT), 0, s, a);
  topk_tail(a, s);
  return dsa_host::check_launch(fn);
}

dsa_status dsa_indexer_scores_hist(const dsa_batch* batch, int32_t H, int32_t D, dsa_dtype code_dtype,
                                   dsa_dtype scale_dtype, const void* q_codes, const void* q_scale,
                                   const void* w, const void* k_cache, const void* k_scale,
                                   float* scores, int64_t ld, uint32_t* hist, int32_t k,
                                   void* stream, const char* fn, const dsa_paging* paging,
                                   bool validate_only = false);

static dsa_status indexer_topk(const dsa_batch* bt, const dsa_paging* pg, int32_t H, int32_t D,
                               dsa_dtype code_dtype, dsa_dtype scale_dtype, const void* q_codes,
                               const void* q_scale, const void* w, const void* k_cache,
                               const void* k_scale, float* scores, int64_t ld, int32_t k,
                               int32_t* idx, void* ws, size_t ws_bytes, void* stream, const char* fn) {
  dsa::TkArgs a{};
  dsa_status st = topk_prepare(bt, scores, ld, k, idx, ws, ws_bytes, fn, &a, pg != nullptr);
  if (st != DSA_OK) return st;
  // the indexer validates its own operands; with no tokens it is a no-op as well.  Batches of
  // many rows take one workgroup per row, which builds its row's histogram itself: there the
  // indexer's many small workgroups would each flush thousands of bins with global atomics
  // (measured on the prefill chunk: ~0.7 ms of atomics against ~0.1 ms for the row workgroups).
  // Only the streaming (decode) indexer accumulates the histogram; batches with more than 4
  // tokens per sequence get it from their own pass.
  const bool rows = bt->num_q >= dsa::kRowMinT;
  const bool fused_hist = !rows && bt->max_q_per_seq <= 4;
  st = dsa_indexer_scores_hist(bt, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                               k_scale, scores, ld, bt->num_q && fused_hist ? a.hist : nullptr, k,
                               stream, fn, pg);
  if (st != DSA_OK || bt->num_q == 0) return st;
  topk_after_scores(a, rows, fused_hist, (hipStream_t)stream);
  return dsa_host::check_launch(fn);
}

extern "C" dsa_status dsa_indexer_topk(const dsa_batch* bt, int32_t H, int32_t D,
                                       dsa_dtype code_dtype, dsa_dtype scale_dtype,
                                       const void* q_codes, const void* q_scale, const void* w,
                                       const void* k_cache, const void* k_scale, float* scores,
                                       int64_t ld, int32_t k, int32_t* idx, void* ws,
                                       size_t ws_bytes, void* stream) {
  return indexer_topk(bt, nullptr, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                      k_scale, scores, ld, k, idx, ws, ws_bytes, stream, "dsa_indexer_topk");
}

dsa_status dsa_check_prolog_cfg(const dsa_prolog_cfg* cfg, const char* fn);
dsa_status dsa_indexer_prolog_scores_hist(const dsa_prolog_cfg* cfg, const dsa_batch* batch,
                                          const void* q_in, const float* q_cos, const float* q_sin,
                                          const void* k_in, const void* w, void* q_codes, void* q_scale,
                                          void* k_cache, void* k_scale, float* scores, int64_t ld,
                                          uint32_t* hist, int32_t k, void* stream, const char* fn,
                                          bool validate_only = false);

// dsa_indexer_prolog followed by dsa_indexer_topk; where the shapes suit it the prolog runs inside
// the indexer kernel (each indexer workgroup quantizes its sequence's query rows itself and the
// workgroup whose key span holds a token's own position quantizes that token's new key row).
extern "C" dsa_status dsa_indexer_prolog_topk(const dsa_prolog_cfg* cfg, const dsa_batch* bt,
                                              const void* q_in, const float* q_cos,
                                              const float* q_sin, const void* k_in, const void* w,
                                              void* q_codes, void* q_scale, void* k_cache,
                                              void* k_scale, int32_t k, float* scores, int64_t ld,
                                              int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_indexer_prolog_topk";
  dsa_status st = dsa_check_prolog_cfg(cfg, fn);
  if (st != DSA_OK) return st;
  dsa::TkArgs a{};
  st = topk_prepare(bt, scores, ld, k, idx, ws, ws_bytes, fn, &a);
  if (st != DSA_OK) return st;
  const bool rows = bt->num_q >= dsa::kRowMinT;     // one workgroup per row: own histogram
  const bool fused_hist = !rows && bt->max_q_per_seq <= 4;
  st = dsa_indexer_prolog_scores_hist(cfg, bt, q_in, q_cos, q_sin, k_in, w, q_codes, q_scale, k_cache,
                                      k_scale, scores, ld, bt->num_q && fused_hist ? a.hist : nullptr,
                                      k, stream, fn);
  if (st != DSA_OK || bt->num_q == 0) return st;
  topk_after_scores(a, rows, fused_hist, (hipStream_t)stream);
  return dsa_host::check_launch(fn);
}

extern "C" dsa_status dsa_indexer_topk_paged(const dsa_batch* bt, const dsa_paging* paging,
                                             int32_t H, int32_t D, dsa_dtype code_dtype,
                                             dsa_dtype scale_dtype, const void* q_codes,
                                             const void* q_scale, const void* w,
                                             const void* k_cache, const void* k_scale,
                                             float* scores, int64_t ld, int32_t k, int32_t* idx,
                                             void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_indexer_topk_paged";
  if (!paging) return fail(DSA_ERR_INVALID_ARG, "%s: paging is NULL", fn);
  return indexer_topk(bt, paging, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                      k_scale, scores, ld, k, idx, ws, ws_bytes, stream, fn);
}

// ---------------------------------------------------------------------------------------------
// Deepseek Indexer Attention in one call.
dsa_status dsa_sfa_internal(const dsa_batch* bt, int32_t Hq, const void* q, const void* kv,
                            int64_t kv_row_stride, const int32_t* idx, int32_t k, const float* sink,
                            float scale, void* out, void* ws, size_t ws_bytes,
                            const dsa_host::SfaSel* sel, void* stream, const char* fn,
                            bool validate_only);

// An upper bound of dsa_sparse_attn_workspace_size(t, Hq, k) over every t <= T that grows with
// T (the attention's partials are not monotone in t): t * n_split * Hq rows of 512 bf16 values
// plus (max, sum), with t * n_split < 256 / n_hg + t, and no partials once t * n_hg >= 256.
static size_t sfa_ws_bound(int32_t T, int32_t Hq) {
  const long n_hg = (Hq + 31) / 32;
  const long rows = std::min(256 / n_hg + (long)T, 512 / n_hg) * (long)Hq;
  return align256((size_t)rows * 512 * 2) + align256((size_t)rows * 2 * 4);
}

// The second-digit histograms of the slice schedule (zero at rest, after the first-digit ones).
static size_t hist2_bytes(int32_t T) { return align256((size_t)T * dsa::kBins * 4); }

extern "C" size_t dsa_indexer_attention_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k,
                                                       int32_t Hq) {
  if (num_q <= 0 || max_kv_len <= 0 || Hq <= 0) return 0;
  return dsa_topk_workspace_size(num_q, max_kv_len, k) + hist2_bytes(num_q) + sfa_ws_bound(num_q, Hq);
}

// Workspace: the top-k's row histograms at the start, then the second-digit histograms of the
// slice schedule (both zero between calls; a later call's first-digit rows may cover an earlier
// call's second-digit rows, zero as well); the top-k's other regions against the end of the
// buffer, the attention's split partials just before them.  A buffer sized for the largest
// num_q and max_kv_len keeps every call's end-packed regions past every call's histograms (the
// partials' bound grows with num_q).
extern "C" dsa_status dsa_indexer_attention(const dsa_batch* bt, const dsa_dia* d, void* ws,
                                            size_t ws_bytes, void* stream) {
  const char* fn = "dsa_indexer_attention";
  if (!bt || !d) return fail(DSA_ERR_INVALID_ARG, "%s: batch/args is NULL", fn);
  dsa_status st = dsa_check_batch(bt, fn);
  if (st != DSA_OK) return st;
  if (d->prolog) {
    st = dsa_check_prolog_cfg(d->prolog, fn);
    if (st != DSA_OK) return st;
    const dsa_prolog_cfg* c = d->prolog;
    if (c->H != d->H || c->D != d->D || c->code_dtype != d->code_dtype || c->scale_dtype != d->scale_dtype)
      return fail(DSA_ERR_INVALID_ARG, "%s: H, D, code_dtype and scale_dtype must equal the prolog's", fn);
  }
  if (bt->num_q == 0) return DSA_OK;
  const size_t need = dsa_indexer_attention_workspace_size(bt->num_q, bt->max_kv_len, d->k, d->Hq);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  dsa::TkArgs a{};
  st = topk_prepare(bt, d->scores, d->ld, d->k, d->idx, ws, ws_bytes, fn, &a);
  if (st != DSA_OK) return st;
  // the attention's partials end where the top-k's end-packed regions begin (at or past
  // ws + histograms + sfa_ws_bound, by the size check above)
  const size_t sfa_bytes = align256(dsa_sparse_attn_workspace_size(bt->num_q, d->Hq, d->k));
  char* sfa_ws = (char*)a.bg - sfa_bytes;
  const bool rows = bt->num_q >= dsa::kRowMinT;          // one workgroup per row: own histogram
  const bool fused_hist = !rows && bt->max_q_per_seq <= 4;
  // The attention resolves its own slices where that measured faster than the finalize launch
  // it replaces: at most 32 query tokens on rows of at most 131072 positions (every attention
  // workgroup of a token repeats the row's k-th key search, whose cost grows with the row,
  // while the finalize spreads it over the row's chunks; measured: faster for 8 tokens of 65536
  // and 32 ragged ones of 6K-65K positions, equal for 8 of 131072).  DSA_DIA_SCHEDULE=
  // slice|finalize forces one form (testing).
  // (The merge pass clears the second-digit histograms for the next call: the slice schedule
  // needs split partials, i.e. k > 32.)
  const bool splits = dsa_sparse_attn_workspace_size(bt->num_q, d->Hq, d->k) > 0;
  bool slice = !rows && splits && bt->num_q <= 32 && bt->max_kv_len <= 131072;
  if (const char* e = getenv("DSA_DIA_SCHEDULE")) {
    if (!strcmp(e, "slice")) slice = !rows && splits;
    else if (!strcmp(e, "finalize")) slice = false;
  }
  uint32_t* hist2 = (uint32_t*)((char*)ws + align256((size_t)bt->num_q * dsa::kShards * dsa::kBins * 4));
  if (slice) a.hist2 = hist2;
  dsa_host::SfaSel sel{d->scores, d->ld, a.bg, a.cnt, a.bits, a.slots, a.hist, hist2, a.nch, d->idx};
  // every argument first
  uint32_t* hist = fused_hist ? a.hist : nullptr;
  if (d->prolog)
    st = dsa_indexer_prolog_scores_hist(d->prolog, bt, d->q_in, d->q_cos, d->q_sin, d->k_in, d->w,
                                        d->q_codes, d->q_scale, d->k_cache, d->k_scale, d->scores,
                                        d->ld, hist, d->k, stream, fn, /*validate_only=*/true);
  else
    st = dsa_indexer_scores_hist(bt, d->H, d->D, d->code_dtype, d->scale_dtype, d->q_codes,
                                 d->q_scale, d->w, d->k_cache, d->k_scale, d->scores, d->ld, hist,
                                 d->k, stream, fn, nullptr, /*validate_only=*/true);
  if (st != DSA_OK) return st;
  st = dsa_sfa_internal(bt, d->Hq, d->q, d->kv, d->kv_row_stride, d->idx, d->k, d->sink, d->scale,
                        d->out, sfa_ws, sfa_bytes, slice ? &sel : nullptr, stream, fn, true);
  if (st != DSA_OK) return st;
  // then the launches: indexer (+ prolog, + first-digit histogram), the top-k's select pass,
  // the attention resolving its own slices, the merge; or the finalize pass before the
  // attention; or, for many-row batches, the indexer, the row top-k and the attention
  if (d->prolog)
    st = dsa_indexer_prolog_scores_hist(d->prolog, bt, d->q_in, d->q_cos, d->q_sin, d->k_in, d->w,
                                        d->q_codes, d->q_scale, d->k_cache, d->k_scale, d->scores,
                                        d->ld, hist, d->k, stream, fn);
  else
    st = dsa_indexer_scores_hist(bt, d->H, d->D, d->code_dtype, d->scale_dtype, d->q_codes,
                                 d->q_scale, d->w, d->k_cache, d->k_scale, d->scores, d->ld, hist,
                                 d->k, stream, fn, nullptr);
  if (st != DSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (rows) {
    hipLaunchKernelGGL(dsa::topk_row, dim3((unsigned)a.T), dim3(dsa::kRNT), 0, s, a);
  } else {
    if (!fused_hist)
      hipLaunchKernelGGL(dsa::topk_hist, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kNT), 0, s, a);
    if (a.poison)                                        // written by select before it is read
      dsa_host::poison_fill(a.bg, (size_t)((const char*)(a.slots + (size_t)a.T * a.nch * dsa::kCap) - (const char*)a.bg), s);
    hipLaunchKernelGGL(dsa::topk_select, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kNT), 0, s, a);
    if (!slice)
      hipLaunchKernelGGL(dsa::topk_finalize, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kNT), 0, s, a);
  }
  st = dsa_sfa_internal(bt, d->Hq, d->q, d->kv, d->kv_row_stride, d->idx, d->k, d->sink, d->scale,
                        d->out, sfa_ws, sfa_bytes, slice ? &sel : nullptr, stream, fn, false);
  if (st != DSA_OK) return st;
  return dsa_host::check_launch(fn);
}
