// Top-k token selection on gfx950: exact radix select over order-preserving fp32 keys.
//
// [LI] "Lightning Indexer" (jsqmd.com/news/787325): the indexer ends in a TopK; the page
// points at its single-core sort-and-merge tail at batch 4 and proposes sorting inside the
// preceding vector stage and merging at the end.  Here a row is split across many
// workgroups instead, so a decode batch of 8 rows still spreads over the whole chip:
//
//   clear   : zero the per-row histograms and counters in the workspace
//   hist    : each workgroup histograms the top 11 bits of its chunk in LDS, then adds the
//             non-zero bins to the row's global histogram
//   select  : every workgroup re-derives the threshold bin b* from the row histogram (the bin
//             holding the k-th largest key), writes positions above b* straight into idx
//             (unordered, wave-aggregated atomics) and appends b*'s elements to a
//             candidate list
//   finalize: one workgroup per row resolves the candidates with two more radix digits (the
//             exact k-th key T*), breaks ties at T* by lowest position (a radix select over
//             positions), then sorts the row's k positions ascending in LDS and pads with -1.
//
// [SFA] step 2: slots past the selection are -1.  Keys: fp32 bits, sign-flipped so that
// unsigned order equals numeric order; -0.0 is mapped to +0.0 first.
#include <algorithm>

#include "common.h"

namespace dsa {

constexpr int kBins = 2048;          // 11-bit digits
constexpr int kTkChunk = 4096;       // scores per workgroup in the hist/select passes

struct TkArgs {
  const int32_t* q_pos; const float* scores; long ld; int k; int T;
  int32_t* idx; uint32_t* hist; uint32_t* cnt; uint64_t* cand; long cap;
};
// cnt[t*4 + 0] = positions written above the threshold bin, [1] = candidates

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                              // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Wave-aggregated slot allocation; every lane of the wave must call it.
__device__ __forceinline__ uint32_t wave_alloc(uint32_t* ctr, bool pred) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return 0;
  const int leader = __ffsll((long long)m) - 1;
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
  base = __shfl(base, leader, kWave);
  return base + (uint32_t)__popcll(m & ((1ull << lane_id()) - 1ull));
}

// Inclusive block scan of one value per thread (NT threads, NT/64 <= 64 waves).
template <int NT>
__device__ uint32_t block_incl_scan(uint32_t v, uint32_t* sh) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  if (w == 0) {
    uint32_t tv = lane < NT / 64 ? sh[lane] : 0u;
#pragma unroll
    for (int o = 1; o < NT / 64; o <<= 1) {
      const uint32_t y = __shfl_up(tv, o, kWave);
      if (lane >= o) tv += y;
    }
    if (lane < NT / 64) sh[lane] = tv;
  }
  __syncthreads();
  if (w > 0) v += sh[w - 1];
  __syncthreads();
  return v;
}

// Given an LDS histogram over kBins digits, find the digit holding the `need`-th element
// counted from the top (descending=true) or from the bottom (descending=false).
// Writes res[0] = digit, res[1] = number of elements strictly before it in that order.
template <int NT>
__device__ void find_digit(const uint32_t* hist, uint32_t need, bool descending, uint32_t* sh,
                           uint32_t* res) {
  constexpr int PER = kBins / NT;
  const int tid = threadIdx.x;
  uint32_t loc[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = tid * PER + j;                     // rank order index
    const int d = descending ? kBins - 1 - r : r;
    loc[j] = hist[d];
    tot += loc[j];
  }
  const uint32_t incl = block_incl_scan<NT>(tot, sh);
  uint32_t before = incl - tot;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (before < need && need <= before + loc[j]) {
      const int r = tid * PER + j;
      res[0] = descending ? kBins - 1 - r : r;
      res[1] = before;
    }
    before += loc[j];
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) topk_clear(uint32_t* p, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0u;
}

__global__ void __launch_bounds__(256) topk_hist(TkArgs a) {
  __shared__ uint32_t h[kBins];
  const int t = blockIdx.y;
  const int p = a.q_pos[t];
  if (p + 1 <= a.k) return;
  const long s0 = (long)blockIdx.x * kTkChunk;
  if (s0 > p) return;
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0u;
  __syncthreads();
  const float4* row = reinterpret_cast<const float4*>(a.scores + (long)t * a.ld + s0);
  const int n = (int)min((long)kTkChunk, (long)p + 1 - s0);
  for (int i = threadIdx.x; i * 4 < n; i += 256) {
    const float4 v = row[i];
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i * 4 + j < n) atomicAdd(&h[order_key(e[j]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (long)t * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ void __launch_bounds__(256) topk_select(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[64];
  __shared__ uint32_t res[2];
  const int t = blockIdx.y;
  const int p = a.q_pos[t];
  if (p + 1 <= a.k) return;
  const long s0 = (long)blockIdx.x * kTkChunk;
  if (s0 > p) return;
  const uint32_t* gh = a.hist + (long)t * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = gh[i];
  __syncthreads();
  find_digit<256>(h, (uint32_t)a.k, true, sh, res);
  const uint32_t thr = res[0];
  const float4* row = reinterpret_cast<const float4*>(a.scores + (long)t * a.ld + s0);
  const int n = (int)min((long)kTkChunk, (long)p + 1 - s0);
  int32_t* out = a.idx + (long)t * a.k;
  uint64_t* cand = a.cand + (long)t * a.cap;
  uint32_t* cnt = a.cnt + (long)t * 4;
  for (int base = 0; base < n; base += 256 * 4) {      // uniform trip count per wave
    const int i = base / 4 + threadIdx.x;
    float e[4] = {0.f, 0.f, 0.f, 0.f};
    if (i * 4 < n) {
      const float4 v = row[i];
      e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = i * 4 + j < n;
      const uint32_t key = order_key(e[j]);
      const uint32_t dg = key >> 21;
      const int s = (int)(s0 + i * 4 + j);
      const bool above = valid && dg > thr;
      const bool at = valid && dg == thr;
      const uint32_t pa = wave_alloc(&cnt[0], above);
      if (above && pa < (uint32_t)a.k) out[pa] = s;
      const uint32_t pc = wave_alloc(&cnt[1], at);
      if (at && pc < (uint32_t)a.cap) cand[pc] = ((uint64_t)key << 32) | (uint32_t)s;
    }
  }
}

constexpr int kFinNT = 1024;

// One workgroup per row.
__global__ void __launch_bounds__(kFinNT) topk_finalize(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t nsel;
  __shared__ int32_t srt[2048];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = a.q_pos[t];
  const int k = a.k;
  int32_t* out = a.idx + (long)t * k;
  if (p + 1 <= k) {
    for (int j = tid; j < k; j += kFinNT) out[j] = j <= p ? j : -1;
    return;
  }
  const uint32_t* cnt = a.cnt + (long)t * 4;
  const uint32_t n_gt = cnt[0];
  const uint32_t nc = cnt[1];
  const uint64_t* cand = a.cand + (long)t * a.cap;
  uint32_t need = (uint32_t)k - n_gt;                     // 1 <= need <= nc
  // --- exact threshold key among the candidates: digits key[20:10] then key[9:0]
  uint32_t prefix = (uint32_t)(cand[0] >> 32) >> 21;     // all candidates share the top digit
  uint32_t above_cnt = 0;                                  // candidates with key > T*
  {
    // digit 2 (11 bits)
    for (int i = tid; i < kBins; i += kFinNT) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += kFinNT) atomicAdd(&h[((uint32_t)(cand[i] >> 32) >> 10) & 0x7FFu], 1u);
    __syncthreads();
    find_digit<kFinNT>(h, need, true, sh, res);
    prefix = (prefix << 11) | res[0];
    above_cnt = res[1];
    const uint32_t need2 = need - res[1];
    __syncthreads();
    // digit 3 (10 bits) among candidates matching the 22-bit prefix
    for (int i = tid; i < kBins; i += kFinNT) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += kFinNT) {
      const uint32_t key = (uint32_t)(cand[i] >> 32);
      if ((key >> 10) == prefix) atomicAdd(&h[key & 0x3FFu], 1u);
    }
    __syncthreads();
    find_digit<kFinNT>(h, need2, true, sh, res);
    prefix = (prefix << 10) | res[0];
    above_cnt += res[1];
    __syncthreads();
  }
  const uint32_t tkey = prefix;                           // exact k-th largest key
  const uint32_t take_eq = need - above_cnt;              // >= 1
  // count ties
  if (tid == 0) nsel = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < nc; i += kFinNT)
    if ((uint32_t)(cand[i] >> 32) == tkey) atomicAdd(&nsel, 1u);
  __syncthreads();
  const uint32_t n_eq = nsel;
  __syncthreads();
  // position threshold among ties (lowest positions win): radix select over 31-bit positions
  uint32_t pos_thr = 0x7FFFFFFFu;
  if (take_eq < n_eq) {
    uint32_t pfx = 0;
    uint32_t needp = take_eq;
    const int shifts[3] = {20, 9, 0};
    const int widths[3] = {11, 11, 9};
    for (int d = 0; d < 3; ++d) {
      for (int i = tid; i < kBins; i += kFinNT) h[i] = 0u;
      __syncthreads();
      const int sh_hi = shifts[d] + widths[d];
      for (uint32_t i = tid; i < nc; i += kFinNT) {
        const uint64_t c = cand[i];
        const uint32_t key = (uint32_t)(c >> 32), pos = (uint32_t)c;
        if (key == tkey && (sh_hi >= 31 || (pos >> sh_hi) == pfx))
          atomicAdd(&h[(pos >> shifts[d]) & ((1u << widths[d]) - 1u)], 1u);
      }
      __syncthreads();
      find_digit<kFinNT>(h, needp, false, sh, res);
      pfx = (pfx << widths[d]) | res[0];
      needp -= res[1];
      __syncthreads();
    }
    pos_thr = pfx;
  }
  // append the selected candidates after the n_gt positions written by topk_select
  if (tid == 0) nsel = n_gt;
  __syncthreads();
  for (uint32_t i = tid; i < nc; i += kFinNT) {
    const uint64_t c = cand[i];
    const uint32_t key = (uint32_t)(c >> 32), pos = (uint32_t)c;
    if (key > tkey || (key == tkey && pos <= pos_thr)) {
      const uint32_t slot = atomicAdd(&nsel, 1u);
      if (slot < (uint32_t)k) out[slot] = (int32_t)pos;
    }
  }
  __syncthreads();
  // ascending order: bitonic sort of the k positions in LDS
  int n2 = 1;
  while (n2 < k) n2 <<= 1;
  for (int j = tid; j < n2; j += kFinNT) srt[j] = j < k ? out[j] : 0x7FFFFFFF;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int j = tid; j < n2 / 2; j += kFinNT) {
        const int lo = 2 * j - (j & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const int x = srt[lo], y = srt[hi];
        if ((x > y) == up) { srt[lo] = y; srt[hi] = x; }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < k; j += kFinNT) out[j] = srt[j];
}

}  // namespace dsa

using dsa_host::fail;
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn);

static long tk_cap(int32_t max_kv_len) { return ((long)max_kv_len + 63) / 64 * 64; }
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

extern "C" size_t dsa_topk_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k) {
  (void)k;
  if (num_q <= 0 || max_kv_len <= 0) return 0;
  const size_t hist = align256((size_t)num_q * dsa::kBins * 4);
  const size_t cnt = align256((size_t)num_q * 4 * 4);
  const size_t cand = align256((size_t)num_q * tk_cap(max_kv_len) * 8);
  return hist + cnt + cand;
}

extern "C" dsa_status dsa_topk(const dsa_batch* bt, const float* scores, int64_t ld, int32_t k,
                               int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_topk";
  dsa_status st = dsa_check_batch(bt, fn);
  if (st != DSA_OK) return st;
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "%s: k must be in [1, 2048] (got %d)", fn, k);
  if (bt->num_q == 0) return DSA_OK;
  if (!scores || !idx) return fail(DSA_ERR_INVALID_ARG, "%s: scores/idx is NULL", fn);
  if (ld < bt->max_kv_len || ld % 4) return fail(DSA_ERR_INVALID_ARG, "%s: ld must be >= max_kv_len and a multiple of 4", fn);
  if ((uintptr_t)scores & 15) return fail(DSA_ERR_INVALID_ARG, "%s: scores must be 16-byte aligned", fn);
  const size_t need = dsa_topk_workspace_size(bt->num_q, bt->max_kv_len, k);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  const int T = bt->num_q;
  dsa::TkArgs a{};
  a.q_pos = bt->q_pos; a.scores = scores; a.ld = ld; a.k = k; a.T = T; a.idx = idx;
  char* w = (char*)ws;
  a.hist = (uint32_t*)w;
  const size_t hist_b = align256((size_t)T * dsa::kBins * 4);
  a.cnt = (uint32_t*)(w + hist_b);
  const size_t cnt_b = align256((size_t)T * 16);
  a.cand = (uint64_t*)(w + hist_b + cnt_b);
  a.cap = tk_cap(bt->max_kv_len);
  hipStream_t s = (hipStream_t)stream;
  const long nclear = (long)(hist_b + cnt_b) / 4;
  const unsigned cgrid = (unsigned)std::min<long>((nclear + 255) / 256, 1024);
  hipLaunchKernelGGL(dsa::topk_clear, dim3(cgrid), dim3(256), 0, s, a.hist, nclear);
  if (T > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: more than 65535 query tokens", fn);
  const dim3 g2((unsigned)((bt->max_kv_len + dsa::kTkChunk - 1) / dsa::kTkChunk), (unsigned)T);
  hipLaunchKernelGGL(dsa::topk_hist, g2, dim3(256), 0, s, a);
  hipLaunchKernelGGL(dsa::topk_select, g2, dim3(256), 0, s, a);
  hipLaunchKernelGGL(dsa::topk_finalize, dim3((unsigned)T), dim3(dsa::kFinNT), 0, s, a);
  return dsa_host::check_launch(fn);
}
