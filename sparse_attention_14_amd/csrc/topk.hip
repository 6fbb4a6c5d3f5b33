// Top-k token selection on gfx950: exact radix select over order-preserving fp32 keys.
//
// [LI] "Lightning Indexer" (jsqmd.com/news/787325): the indexer ends in a TopK; the page
// points at its single-core sort-and-merge tail at batch 4 and proposes sorting inside the
// preceding vector stage and merging at the end.  Here a row is split across many
// workgroups instead, so a decode batch of 8 rows still spreads over the whole chip:
//
//   hist    : the top 11 bits of every key, per row, in a 2048-bin histogram (its own pass,
//             or fused into the indexer workgroups by dsa_indexer_topk)
//   select  : one workgroup per 4096-score chunk re-derives the digit b1 that holds the k-th
//             largest key; positions above b1 go into the row's position bitmap, positions
//             with digit b1 (candidates) into the row's candidate list
//   finalize: one workgroup per row resolves the exact k-th key K* with two more digits over
//             the candidates, adds the candidates above K* (and the lowest-position ties at
//             K*) to the bitmap and writes its set positions in order: ascending output with
//             no sort, ties to the lower position.  (A last-workgroup-finalizes scheme inside
//             the select pass needs a device-scope release per workgroup, which writes back
//             the L2 and costs more than the extra launch.)
//
// [SFA] step 2: slots past the selection are -1.  Keys: fp32 bits, sign-flipped so that
// unsigned order equals numeric order; -0.0 is mapped to +0.0 first.
#include <algorithm>

#include "common.h"

namespace dsa {

constexpr int kBins = kHistBins;     // 11-bit digits
constexpr int kShards = kHistShards; // copies of each row histogram (spread atomic traffic)
constexpr int kTkChunk = 4096;       // scores per select workgroup
constexpr int kTkNT = 256;           // threads per select workgroup
constexpr int kPerThr = kTkChunk / kTkNT;
constexpr int kSlotCap = 256;        // entries per (chunk, wave) slot

// Workspace (zero-filled before the first call; every call leaves the histograms zero-filled
// again, and the rest is written before it is read):
//   hist  [T][kShards][kBins] u32          row histogram of the top digit, in shards
//   cnt   [T][nch][4] u32                  per (chunk, wave): n_above | n_cand << 16
//   b1    [T] u32                          the row's threshold digit
//   bits  [T][bw] u32                      per row: bitmap of the positions above b1
//   slots [T][nch][4][kSlotCap] u64        per (chunk, wave): candidates, key << 32 | position
struct TkArgs {
  const int32_t* q_pos; const float* scores; long ld; int k; int T; int nch;
  int32_t* idx; uint32_t* hist; uint32_t* cnt; uint32_t* b1; uint32_t* bits; long bw;
  uint64_t* slots;
};

// Inclusive prefix sum over the 64 lanes of a wave: four row shifts within each 16-lane row,
// then the row broadcasts of lanes 15 and 31 (DPP, no LDS round trip).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

// Exclusive prefix sum over the NT threads of the block (one barrier); `total` gets the sum.
// sh holds NT/64 words; consecutive uses of one sh must be separated by a barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t x = sh[i];
    before += i < w ? x : 0u;
    tot += x;
  }
  total = tot;
  return before + inc - v;
}

// The digit holding the need-th largest element of an LDS histogram over kBins digits:
// res[0] = digit, res[1] = elements in larger digits.  Ends with a barrier.
template <int NT>
__device__ void find_digit_desc(const uint32_t* hist, uint32_t need, uint32_t* sh, uint32_t* res) {
  constexpr int PER = kBins / NT;
  const int tid = threadIdx.x;
  uint32_t loc[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { loc[j] = hist[kBins - 1 - (tid * PER + j)]; tot += loc[j]; }
  uint32_t all;
  uint32_t before = block_excl_scan<NT>(tot, sh, all);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (before < need && need <= before + loc[j]) { res[0] = kBins - 1 - (tid * PER + j); res[1] = before; }
    before += loc[j];
  }
  __syncthreads();
}

// First pass (when the indexer did not accumulate it): histogram of the top 11 key bits of a
// 4096-score chunk in LDS; non-zero bins are added to shard (chunk % kShards) of the row's.
__global__ void __launch_bounds__(kTkNT) topk_hist(TkArgs a) {
  __shared__ uint32_t h[kBins];
  const int t = blockIdx.y;
  const int p = a.q_pos[t];
  if (p + 1 <= a.k) return;
  const long s0 = (long)blockIdx.x * kTkChunk;
  if (s0 > p) return;
  for (int i = threadIdx.x; i < kBins; i += kTkNT) h[i] = 0u;
  __syncthreads();
  const float* row = a.scores + (long)t * a.ld + s0;
  const int n = (int)min((long)kTkChunk, (long)p + 1 - s0);
  float4 vv[kPerThr / 4];                                 // all loads first (in-bounds; masked)
#pragma unroll
  for (int j = 0; j < kPerThr / 4; ++j) {
    const int e0 = min(threadIdx.x * 4 + j * kTkNT * 4, (int)(((a.ld - s0) & ~3L) - 4));
    vv[j] = *reinterpret_cast<const float4*>(row + e0);
  }
#pragma unroll
  for (int j = 0; j < kPerThr / 4; ++j) {
    const int e0 = threadIdx.x * 4 + j * kTkNT * 4;
    const float e[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (e0 + q < n) atomicAdd(&h[order_key(e[q]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + ((long)t * kShards + blockIdx.x % kShards) * kBins;
  for (int i = threadIdx.x; i < kBins; i += kTkNT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Select pass: one workgroup per 4096-score chunk.  From the row histogram it re-derives the
// top digit b1 that holds the k-th largest key.  Positions with digit > b1 are certainly
// selected: each thread stores the 16-bit mask of its 16 positions into the row's position
// bitmap (every call rewrites the chunk's bits, so the bitmap needs no clearing).  Positions
// with digit == b1 are candidates: each wave writes them (key, position) to its own slot (wave
// prefix sum, no atomics).
__global__ void __launch_bounds__(kTkNT) topk_select(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[kTkNT / 64];
  __shared__ uint32_t res[2];
  const int t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ch = blockIdx.x;
  const long s0 = (long)ch * kTkChunk;                    // < ld: the grid covers max_kv_len
  const float* row = a.scores + (long)t * a.ld + s0;
  // the chunk's scores, the row histogram and q_pos are loaded together (one memory round
  // trip; every address is in bounds whatever the row's length)
  const int p = a.q_pos[t];
  float4 vv[kPerThr / 4];
#pragma unroll
  for (int j = 0; j < kPerThr / 4; ++j) {                // thread owns 16 consecutive scores
    const int e0 = min(tid * kPerThr + 4 * j, (int)(((a.ld - s0) & ~3L) - 4));
    vv[j] = *reinterpret_cast<const float4*>(row + e0);   // in-bounds; masked below
  }
  const uint32_t* gh = a.hist + (long)t * kShards * kBins;
  uint32_t hv[kShards][kBins / kTkNT];
#pragma unroll
  for (int sd = 0; sd < kShards; ++sd)
#pragma unroll
    for (int j = 0; j < kBins / kTkNT; ++j) hv[sd][j] = gh[sd * kBins + tid + j * kTkNT];
#pragma unroll
  for (int j = 0; j < kBins / kTkNT; ++j) {
    uint32_t v = 0;
#pragma unroll
    for (int sd = 0; sd < kShards; ++sd) v += hv[sd][j];
    h[tid + j * kTkNT] = v;
  }
  const int k = a.k;
  if (p + 1 <= k) return;                                 // short rows: finalize writes them
  const int nch = (p + kTkChunk) / kTkChunk;              // chunks covering 0 .. p
  if (ch >= nch) return;
  const int n = (int)min((long)kTkChunk, (long)p + 1 - s0);
  __syncthreads();
  find_digit_desc<kTkNT>(h, (uint32_t)k, sh, res);
  const uint32_t b1 = res[0];
  const int nv = min(max(n - tid * kPerThr, 0), kPerThr);          // valid positions of the thread
  const uint32_t vmask = nv == kPerThr ? 0xFFFFu : ((1u << nv) - 1u);
  uint32_t gtm = 0, eqm = 0;                              // bit e: position s0 + 16 tid + e
  uint32_t keys[kPerThr];
#pragma unroll
  for (int j = 0; j < kPerThr / 4; ++j) {
    const float f[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * j + q;
      keys[e] = order_key(f[q]);
      const uint32_t d = keys[e] >> 21;
      gtm |= (uint32_t)(d > b1) << e;
      eqm |= (uint32_t)(d == b1) << e;
    }
  }
  gtm &= vmask;
  eqm &= vmask;
  reinterpret_cast<uint16_t*>(a.bits + (long)t * a.bw)[(s0 >> 4) + tid] = (uint16_t)gtm;
  const uint32_t mine = (uint32_t)__popc(gtm) | ((uint32_t)__popc(eqm) << 16);
  const uint32_t inc = wave_incl_scan(mine);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  uint32_t o = (inc - mine) >> 16;                        // candidates of the lanes before
  uint64_t* slot = a.slots + (((long)t * a.nch + ch) * 4 + wave) * kSlotCap;
  const uint32_t pos0 = (uint32_t)(s0 + tid * kPerThr);
  if (eqm) {
#pragma unroll
    for (int e = 0; e < kPerThr; ++e)
      if ((eqm >> e) & 1u) {
        if (o < (uint32_t)kSlotCap) slot[o] = ((uint64_t)keys[e] << 32) | (pos0 + e);
        ++o;
      }
  }
  if (lane == 0) a.cnt[((long)t * a.nch + ch) * 4 + wave] = wtot;
  if (ch == 0 && tid == 0) a.b1[t] = b1;
}

// Finalize: one workgroup per row.
//  * One memory round trip (sized by the batch maxima, so that nothing waits for q_pos) loads
//    the row's position bitmap (positions above b1), the slot counts and the first entries of
//    every candidate slot into registers; the candidates' second-digit histogram follows.
//  * The second radix digit (11 bits) b2 splits the candidates; when few candidates share b2
//    (the usual case) the exact k-th key K* comes from their pairwise ranks, else from a third
//    digit (10 bits).  take_eq is how many keys equal to K* to keep.
//  * Candidates above K* join the bitmap, and so do the keys equal to K*: all of them when they
//    are exactly take_eq, else the take_eq lowest positions (ranked by a block scan over a tie
//    bitmap).
//  * The output is the bitmap's set positions in ascending order (block scan of per-thread
//    popcounts), staged in LDS and stored coalesced: no sort.
// Rows with a candidate slot longer than the first trip (crowded digits, massive ties) take
// their candidates from the row's scores instead.  The row's histogram shards are zeroed for
// the next call.  Slot indexing uses shifts (no integer division).
constexpr int kFinNT = 512;
constexpr int kFinW = kFinNT / 64;                        // waves
constexpr int kMaxWords = 262144 / 32;                    // bitmap words of the longest row
constexpr int kWPT = kMaxWords / kFinNT;                  // bitmap words per thread (max)
constexpr int kSpecPT = 8;                                // first-trip slot loads per thread
constexpr int kSmall = 64;                                // pairwise ranking of the b2 bin

__global__ void __launch_bounds__(kFinNT) topk_finalize(TkArgs a) {
  __shared__ uint32_t h2[kBins], h3[kBins];
  __shared__ uint32_t sh[kFinW];
  __shared__ uint32_t res[2];
  __shared__ uint32_t scnt[kFinNT];
  __shared__ uint32_t flags[2];        // [0]: a slot longer than the first trip, [1]: small count
  __shared__ uint32_t wsum[kFinW];
  __shared__ uint32_t small[kSmall];
  __shared__ uint32_t bm[kMaxWords];   // selected positions
  __shared__ uint32_t tb[kMaxWords];   // ties at K* (rare path)
  __shared__ int32_t ostage[2048];     // output, staged for coalesced stores
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- one round trip, sized by the batch maxima
  const int nsub_m = a.nch * 4;                           // <= 256
  const int wpt_m = (int)((a.bw + kFinNT - 1) / kFinNT);  // <= kWPT
  int sl = 31 - __clz((kSpecPT * kFinNT) / nsub_m);       // first-trip entries per slot: 2^sl
  sl = min(sl, 8);                                        // kSlotCap = 256
  const uint64_t* srow = a.slots + (long)t * nsub_m * kSlotCap;
  const uint32_t* gbits = a.bits + (long)t * a.bw;
  const int p = a.q_pos[t];
  uint32_t wv[kWPT];
#pragma unroll
  for (int j = 0; j < kWPT; ++j) {
    const long w = (long)tid * wpt_m + j;
    wv[j] = (j < wpt_m && w < a.bw) ? gbits[w] : 0u;
  }
  const uint32_t my_cnt = tid < nsub_m ? a.cnt[(long)t * nsub_m + tid] : 0u;
  uint64_t ev[kSpecPT];
#pragma unroll
  for (int u = 0; u < kSpecPT; ++u) {
    const int f = tid + u * kFinNT;
    ev[u] = srow[(long)min(f >> sl, nsub_m - 1) * kSlotCap + (f & ((1 << sl) - 1))];
  }
  const uint32_t b1 = a.b1[t];
  {                                                       // nothing below reads the histogram
    uint32_t* gh = a.hist + (long)t * kShards * kBins;
    for (int i = tid; i < kShards * kBins; i += kFinNT) gh[i] = 0u;
  }
  const int k = a.k;
  int32_t* out = a.idx + (long)t * k;
  if (p + 1 <= k) {                                       // short row: everything, then -1
    for (int j = tid; j < k; j += kFinNT) out[j] = j <= p ? j : -1;
    return;
  }
  const int nch = (p + kTkChunk) / kTkChunk;
  const int nsub = nch * 4;
  const int nw = (p + 1 + 31) >> 5;                       // bitmap words of this row
  for (int i = tid; i < kBins; i += kFinNT) { h2[i] = 0u; h3[i] = 0u; }
#pragma unroll
  for (int j = 0; j < kWPT; ++j) {
    const int w = tid * wpt_m + j;
    if (j < wpt_m) { bm[w] = w < nw ? wv[j] : 0u; tb[w] = 0u; }
  }
  if (tid < 2) flags[tid] = 0u;
  scnt[tid] = tid < nsub ? my_cnt : 0u;
  {
    uint32_t s = wave_incl_scan(tid < nsub ? (my_cnt & 0xFFFFu) : 0u);
    s = (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
    if (lane == 0) wsum[wave] = s;
  }
  __syncthreads();
  uint32_t G = 0;                                         // positions above b1 (< k)
#pragma unroll
  for (int i = 0; i < kFinW; ++i) G += wsum[i];
  if (tid < nsub && (my_cnt >> 16) > (1u << sl)) flags[0] = 1u;
  // this thread's first-trip candidates
  uint32_t cvalid = 0;
#pragma unroll
  for (int u = 0; u < kSpecPT; ++u) {
    const int f = tid + u * kFinNT, sidx = f >> sl;       // sidx < kFinNT
    cvalid |= (uint32_t)(sidx < nsub && (uint32_t)(f & ((1 << sl) - 1)) < (scnt[sidx] >> 16)) << u;
  }
  __syncthreads();                                        // flags
  const bool streamed = flags[0] != 0u;
  const uint32_t need = (uint32_t)k - G;                  // 1 <= need <= #candidates
  const float* row = a.scores + (long)t * a.ld;
  auto each_cand = [&](auto&& fn) {
    if (!streamed) {
#pragma unroll
      for (int u = 0; u < kSpecPT; ++u)
        if ((cvalid >> u) & 1u) fn((uint32_t)(ev[u] >> 32), (uint32_t)ev[u]);
    } else {
      for (int s = tid; s <= p; s += kFinNT) {
        const uint32_t key = order_key(row[s]);
        if ((key >> 21) == b1) fn(key, (uint32_t)s);
      }
    }
  };
  each_cand([&](uint32_t key, uint32_t) { atomicAdd(&h2[(key >> 10) & 0x7FFu], 1u); });
  __syncthreads();
  find_digit_desc<kFinNT>(h2, need, sh, res);
  const uint32_t b2 = res[0];
  uint32_t above = res[1];
  const uint32_t need2 = need - above;                    // >= 1, among the b2 bin
  const uint32_t c2 = h2[b2];
  uint32_t kstar, n_eq;
  if (c2 <= (uint32_t)kSmall) {                           // pairwise ranks within the b2 bin
    if (tid == 0) flags[1] = 0u;
    __syncthreads();
    each_cand([&](uint32_t key, uint32_t) {
      if (((key >> 10) & 0x7FFu) == b2) small[atomicAdd(&flags[1], 1u)] = key;
    });
    __syncthreads();
    if (tid < (int)c2) {
      const uint32_t mine = small[tid];
      uint32_t gt = 0, eq = 0;
      for (uint32_t j = 0; j < c2; ++j) { const uint32_t x = small[j]; gt += x > mine; eq += x == mine; }
      if (gt < need2 && need2 <= gt + eq) { res[0] = mine; res[1] = gt; sh[0] = eq; }
    }
    __syncthreads();
    kstar = res[0];
    above += res[1];
    n_eq = sh[0];
    __syncthreads();                                      // sh is reused below
  } else {                                                // third digit
    each_cand([&](uint32_t key, uint32_t) {
      if (((key >> 10) & 0x7FFu) == b2) atomicAdd(&h3[key & 0x3FFu], 1u);
    });
    __syncthreads();
    find_digit_desc<kFinNT>(h3, need2, sh, res);
    kstar = (b1 << 21) | (b2 << 10) | res[0];
    above += res[1];
    n_eq = h3[res[0]];
  }
  const uint32_t take_eq = need - above;                 // >= 1
  const bool all_ties = n_eq == take_eq;
  each_cand([&](uint32_t key, uint32_t pos) {
    if (key > kstar || (key == kstar && all_ties)) atomicOr(&bm[pos >> 5], 1u << (pos & 31));
    else if (key == kstar) atomicOr(&tb[pos >> 5], 1u << (pos & 31));
  });
  __syncthreads();
  if (!all_ties) {                                        // keep the take_eq lowest tie positions
    uint32_t nt = 0;
    for (int j = 0; j < wpt_m; ++j) nt += (uint32_t)__popc(tb[tid * wpt_m + j]);
    uint32_t tot;
    uint32_t r = block_excl_scan<kFinNT>(nt, sh, tot);     // ties before this thread's words
    for (int j = 0; j < wpt_m; ++j) {
      uint32_t m = tb[tid * wpt_m + j], keep = 0;
      while (m && r < take_eq) { const uint32_t lb = m & (0u - m); keep |= lb; m ^= lb; ++r; }
      r += (uint32_t)__popc(m);
      if (keep) bm[tid * wpt_m + j] |= keep;              // own words only
    }
    __syncthreads();
  }
  // ascending output: per-thread popcounts of its contiguous words, one block scan
  uint32_t nb = 0;
#pragma unroll
  for (int j = 0; j < kWPT; ++j) {
    wv[j] = j < wpt_m ? bm[tid * wpt_m + j] : 0u;
    nb += (uint32_t)__popc(wv[j]);
  }
  uint32_t tot;
  uint32_t o = block_excl_scan<kFinNT>(nb, sh, tot);
#pragma unroll
  for (int j = 0; j < kWPT; ++j) {
    uint32_t m = wv[j];
    const int base = (tid * wpt_m + j) * 32;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (o < (uint32_t)k) ostage[o] = base + bit;
      ++o;
    }
  }
  __syncthreads();
  for (int j = tid; j < k; j += kFinNT) out[j] = ostage[j];
}

}  // namespace dsa

using dsa_host::fail;
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn);
dsa_status dsa_check_batch_paged(const dsa_batch* bt, const char* fn);

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static int tk_nch(int32_t max_kv_len) { return (max_kv_len + dsa::kTkChunk - 1) / dsa::kTkChunk; }

struct TkLayout { size_t hist, cnt, b1, bits, slots, total; long bw; };
static TkLayout tk_layout(int32_t T, int32_t max_kv_len) {
  TkLayout L{};
  const int nch = tk_nch(max_kv_len);
  L.bw = (long)nch * (dsa::kTkChunk / 32);                // whole chunks of bits
  L.hist = 0;
  L.cnt = align256((size_t)T * dsa::kShards * dsa::kBins * 4);
  L.b1 = L.cnt + align256((size_t)T * nch * 4 * 4);
  L.bits = L.b1 + align256((size_t)T * 4);
  L.slots = L.bits + align256((size_t)T * L.bw * 4);
  L.total = L.slots + align256((size_t)T * nch * 4 * dsa::kSlotCap * 8);
  return L;
}

extern "C" size_t dsa_topk_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k) {
  (void)k;
  if (num_q <= 0 || max_kv_len <= 0) return 0;
  return tk_layout(num_q, max_kv_len).total;
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
  if (bt->max_kv_len > 64 * dsa::kTkChunk) return fail(DSA_ERR_UNSUPPORTED, "%s: max_kv_len above %d", fn, 64 * dsa::kTkChunk);
  const TkLayout L = tk_layout(bt->num_q, bt->max_kv_len);
  if (!ws || ws_bytes < L.total) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, L.total);
  if ((uintptr_t)ws & 255) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (bt->num_q > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: more than 65535 query tokens", fn);
  dsa::TkArgs a{};
  a.q_pos = bt->q_pos; a.scores = scores; a.ld = ld; a.k = k; a.T = bt->num_q; a.idx = idx;
  a.nch = tk_nch(bt->max_kv_len);
  char* w = (char*)ws;
  a.hist = (uint32_t*)(w + L.hist);
  a.cnt = (uint32_t*)(w + L.cnt);
  a.b1 = (uint32_t*)(w + L.b1);
  a.bits = (uint32_t*)(w + L.bits);
  a.bw = L.bw;
  a.slots = (uint64_t*)(w + L.slots);
  *out = a;
  return DSA_OK;
}

// Select + finalize (the row histograms are already in the workspace).
static void topk_tail(const dsa::TkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dsa::topk_select, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kTkNT), 0, s, a);
  hipLaunchKernelGGL(dsa::topk_finalize, dim3((unsigned)a.T), dim3(dsa::kFinNT), 0, s, a);
}

extern "C" dsa_status dsa_topk(const dsa_batch* bt, const float* scores, int64_t ld, int32_t k,
                               int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_topk";
  dsa::TkArgs a{};
  const dsa_status st = topk_prepare(bt, scores, ld, k, idx, ws, ws_bytes, fn, &a);
  if (st != DSA_OK || bt->num_q == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(dsa::topk_hist, dim3((unsigned)a.nch, (unsigned)a.T), dim3(dsa::kTkNT), 0, s, a);
  topk_tail(a, s);
  return dsa_host::check_launch(fn);
}

dsa_status dsa_indexer_scores_hist(const dsa_batch* batch, int32_t H, int32_t D, dsa_dtype code_dtype,
                                   dsa_dtype scale_dtype, const void* q_codes, const void* q_scale,
                                   const void* w, const void* k_cache, const void* k_scale,
                                   float* scores, int64_t ld, uint32_t* hist, int32_t k,
                                   void* stream, const char* fn, const dsa_paging* paging);

static dsa_status indexer_topk(const dsa_batch* bt, const dsa_paging* pg, int32_t H, int32_t D,
                               dsa_dtype code_dtype, dsa_dtype scale_dtype, const void* q_codes,
                               const void* q_scale, const void* w, const void* k_cache,
                               const void* k_scale, float* scores, int64_t ld, int32_t k,
                               int32_t* idx, void* ws, size_t ws_bytes, void* stream, const char* fn) {
  dsa::TkArgs a{};
  dsa_status st = topk_prepare(bt, scores, ld, k, idx, ws, ws_bytes, fn, &a, pg != nullptr);
  if (st != DSA_OK) return st;
  // the indexer validates its own operands; with no tokens it is a no-op as well
  st = dsa_indexer_scores_hist(bt, H, D, code_dtype, scale_dtype, q_codes, q_scale, w, k_cache,
                               k_scale, scores, ld, bt->num_q ? a.hist : nullptr, k, stream, fn, pg);
  if (st != DSA_OK || bt->num_q == 0) return st;
  topk_tail(a, (hipStream_t)stream);
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
