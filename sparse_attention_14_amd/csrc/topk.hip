// Top-k token selection on gfx950: exact radix select over order-preserving fp32 keys.
//
// [LI] "Lightning Indexer" (jsqmd.com/news/787325): the indexer ends in a TopK; the page
// points at its single-core sort-and-merge tail at batch 4 and proposes sorting inside the
// preceding vector stage and merging at the end.  Here a row is split across many
// workgroups instead, so a decode batch of 8 rows still spreads over the whole chip:
//
//   hist   : each workgroup histograms the top 11 bits of its 4096-score chunk in LDS and
//            adds the non-zero bins to the row's histogram
//   select : every workgroup re-derives the threshold digit b* (the digit holding the k-th
//            largest key) from the row histogram and writes its chunk's survivors (digit >=
//            b*) in position order to its own slot (block scans, no contended atomics)
//   finalize: one workgroup per row finds the exact k-th key T* with two more 11/10-bit
//            digits over the survivors (staged in LDS), then walks them in position order
//            keeping key > T* and the first (k - #above) keys equal to T*: the output is
//            ascending with no sort, and ties go to the lower position.  It then zeroes the
//            row's histogram for the next call.  (A last-workgroup-finalizes scheme inside
//            the select pass needs a device-scope release per workgroup, which writes back
//            the L2 and costs more than the extra launch.)
//
// [SFA] step 2: slots past the selection are -1.  Keys: fp32 bits, sign-flipped so that
// unsigned order equals numeric order; -0.0 is mapped to +0.0 first.
#include <algorithm>

#include "common.h"

namespace dsa {

constexpr int kBins = 2048;          // 11-bit digits
constexpr int kTkChunk = 4096;       // scores per workgroup
constexpr int kTkNT = 256;           // threads per workgroup
constexpr int kPerThr = kTkChunk / kTkNT;
constexpr int kSurvCap = 8192;      // survivors staged in LDS by the finalizing workgroup

// Workspace (zero-filled before the first call; every call leaves it zero-filled again):
//   hist [T][kBins] u32   row histogram of the top digit
//   cnt  [T][nch] u32     survivors per chunk
//   surv [T][nch][kTkChunk] u64  (key << 32 | position), in position order per chunk
struct TkArgs {
  const int32_t* q_pos; const float* scores; long ld; int k; int T; int nch;
  int32_t* idx; uint32_t* hist; uint32_t* cnt; uint64_t* surv;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                              // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive block scan of one value per thread (NT threads).
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

// LDS histogram over kBins digits: the digit holding the `need`-th largest element.
// res[0] = digit, res[1] = elements in larger digits.
template <int NT>
__device__ void find_digit_desc(const uint32_t* hist, uint32_t need, uint32_t* sh, uint32_t* res) {
  constexpr int PER = kBins / NT;
  const int tid = threadIdx.x;
  uint32_t loc[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { loc[j] = hist[kBins - 1 - (tid * PER + j)]; tot += loc[j]; }
  const uint32_t incl = block_incl_scan<NT>(tot, sh);
  uint32_t before = incl - tot;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (before < need && need <= before + loc[j]) { res[0] = kBins - 1 - (tid * PER + j); res[1] = before; }
    before += loc[j];
  }
  __syncthreads();
}

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
  uint32_t* gh = a.hist + (long)t * kBins;
  for (int i = threadIdx.x; i < kBins; i += kTkNT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Select pass: one workgroup per row chunk writes the chunk's survivors (digit >= the
// threshold digit b*) in position order to its own slot.
__global__ void __launch_bounds__(kTkNT) topk_select(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[64];
  __shared__ uint32_t res[4];
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int p = a.q_pos[t];
  const int k = a.k;
  if (p + 1 <= k) return;                                 // short rows: finalize writes them
  const int nch = (p + kTkChunk) / kTkChunk;              // chunks covering 0 .. p
  const int ch = blockIdx.x;
  if (ch >= nch) return;
  const uint32_t* gh = a.hist + (long)t * kBins;
  {
    uint32_t v[kBins / kTkNT];                             // batched loads, then LDS
#pragma unroll
    for (int j = 0; j < kBins / kTkNT; ++j) v[j] = gh[tid + j * kTkNT];
#pragma unroll
    for (int j = 0; j < kBins / kTkNT; ++j) h[tid + j * kTkNT] = v[j];
  }
  __syncthreads();
  find_digit_desc<kTkNT>(h, (uint32_t)k, sh, res);
  const uint32_t thr = res[0];

  const long s0 = (long)ch * kTkChunk;
  const int n = (int)min((long)kTkChunk, (long)p + 1 - s0);
  const float* row = a.scores + (long)t * a.ld + s0;
  uint32_t keys[kPerThr];
  uint32_t mine = 0;
  float4 vv[kPerThr / 4];
#pragma unroll
  for (int j = 0; j < kPerThr / 4; ++j) {                // thread owns 16 consecutive scores
    const int e0 = min(tid * kPerThr + 4 * j, (int)(((a.ld - s0) & ~3L) - 4));
    vv[j] = *reinterpret_cast<const float4*>(row + e0);   // in-bounds; masked below
  }
#pragma unroll
  for (int j = 0; j < kPerThr / 4; ++j) {
    const int e0 = tid * kPerThr + 4 * j;
    const float f[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t key = order_key(f[q]);
      const bool keep = e0 + q < n && (key >> 21) >= thr;
      keys[4 * j + q] = keep ? key : 0u;
      mine += keep;
    }
  }
  const uint32_t incl = block_incl_scan<kTkNT>(mine, sh);
  uint32_t pos = incl - mine;
  uint64_t* sv = a.surv + ((long)t * a.nch + ch) * kTkChunk;
#pragma unroll
  for (int e = 0; e < kPerThr; ++e)
    if (keys[e]) sv[pos++] = ((uint64_t)keys[e] << 32) | (uint32_t)(s0 + tid * kPerThr + e);
  if (tid == kTkNT - 1) a.cnt[(long)t * a.nch + ch] = incl;
}

// Finalize: one workgroup per row.  Finds the exact k-th key T* with two more 11/10-bit digits
// over the survivors, then walks them in position order keeping key > T* and the first
// (k - #above) keys equal to T* -- ascending output, ties to the lower position, no sort --
// and zeroes the row's histogram for the next call.
constexpr int kFinNT = 512;

__global__ void __launch_bounds__(kFinNT) topk_finalize(TkArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[64];
  __shared__ uint32_t res[4];
  __shared__ uint32_t chunk_off[65];
  __shared__ uint64_t sv_lds[kSurvCap];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = a.q_pos[t];
  const int k = a.k;
  int32_t* out = a.idx + (long)t * k;
  if (p + 1 <= k) {                                       // short row: everything, then -1
    for (int j = tid; j < k; j += kFinNT) out[j] = j <= p ? j : -1;
    return;
  }
  const int nch = (p + kTkChunk) / kTkChunk;
  uint32_t* gh = a.hist + (long)t * kBins;
  {
    uint32_t v[kBins / kFinNT];
#pragma unroll
    for (int j = 0; j < kBins / kFinNT; ++j) v[j] = gh[tid + j * kFinNT];
#pragma unroll
    for (int j = 0; j < kBins / kFinNT; ++j) h[tid + j * kFinNT] = v[j];
  }
  if (tid == 0) {
    uint32_t acc = 0;
    for (int c = 0; c < nch; ++c) { chunk_off[c] = acc; acc += a.cnt[(long)t * a.nch + c]; }
    chunk_off[nch] = acc;
  }
  __syncthreads();
  find_digit_desc<kFinNT>(h, (uint32_t)k, sh, res);
  const uint32_t thr = res[0];
  const uint32_t n_gt = res[1];
  const uint32_t nsurv = chunk_off[nch];
  const uint64_t* sall = a.surv + (long)t * a.nch * kTkChunk;
  // survivors in position order: staged in LDS when they fit (the usual case), else read from
  // the per-chunk slots (rows with massive ties)
  const bool in_lds = nsurv <= kSurvCap;
  if (in_lds) {
    for (int c = 0; c < nch; ++c) {
      const uint32_t n0 = chunk_off[c], nc = chunk_off[c + 1] - n0;
      const uint64_t* src = sall + (long)c * kTkChunk;
      for (uint32_t i = tid; i < nc; i += kFinNT) sv_lds[n0 + i] = src[i];
    }
  }
  __syncthreads();
  auto surv_at = [&](uint32_t i) -> uint64_t {
    if (in_lds) return sv_lds[i];
    int lo = 0, hi = nch - 1;
    while (lo < hi) { const int mid = (lo + hi + 1) >> 1; if (chunk_off[mid] <= i) lo = mid; else hi = mid - 1; }
    return sall[(long)lo * kTkChunk + (i - chunk_off[lo])];
  };
  const uint32_t need = (uint32_t)k - n_gt;
  uint32_t prefix = thr, above = 0, need2;
  for (int i = tid; i < kBins; i += kFinNT) h[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < nsurv; i += kFinNT) {
    const uint32_t key = (uint32_t)(surv_at(i) >> 32);
    if ((key >> 21) == thr) atomicAdd(&h[(key >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  find_digit_desc<kFinNT>(h, need, sh, res);
  prefix = (prefix << 11) | res[0];
  above = res[1];
  need2 = need - res[1];
  for (int i = tid; i < kBins; i += kFinNT) h[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < nsurv; i += kFinNT) {
    const uint32_t key = (uint32_t)(surv_at(i) >> 32);
    if ((key >> 10) == prefix) atomicAdd(&h[key & 0x3FFu], 1u);
  }
  __syncthreads();
  find_digit_desc<kFinNT>(h, need2, sh, res);
  const uint32_t tkey = (prefix << 10) | res[0];
  above += res[1];
  const uint32_t take_eq = need - above;                 // ties at tkey kept, lowest positions first
  // ordered pass over contiguous per-thread segments: keep key > tkey and the first take_eq
  // keys == tkey (two block scans: tie ranks, then output slots)
  const uint32_t seg = (nsurv + kFinNT - 1) / kFinNT;
  const uint32_t b0 = min(nsurv, tid * seg), b1 = min(nsurv, b0 + seg);
  uint32_t my_ties = 0;
  for (uint32_t i = b0; i < b1; ++i) my_ties += ((uint32_t)(surv_at(i) >> 32) == tkey);
  const uint32_t tie_base = block_incl_scan<kFinNT>(my_ties, sh) - my_ties;
  uint32_t my_keep = 0, rank = tie_base;
  for (uint32_t i = b0; i < b1; ++i) {
    const uint32_t key = (uint32_t)(surv_at(i) >> 32);
    if (key == tkey) my_keep += (++rank <= take_eq);
    else my_keep += (key > tkey);
  }
  uint32_t slot = block_incl_scan<kFinNT>(my_keep, sh) - my_keep;
  rank = tie_base;
  for (uint32_t i = b0; i < b1; ++i) {
    const uint64_t v = surv_at(i);
    const uint32_t key = (uint32_t)(v >> 32);
    const bool keep = key == tkey ? (++rank <= take_eq) : (key > tkey);
    if (keep) {
      if (slot < (uint32_t)k) out[slot] = (int32_t)(uint32_t)v;
      ++slot;
    }
  }
  // leave the row's histogram zeroed for the next call
  for (int i = tid; i < kBins; i += kFinNT) gh[i] = 0u;
}

}  // namespace dsa

using dsa_host::fail;
dsa_status dsa_check_batch(const dsa_batch* bt, const char* fn);

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static int tk_nch(int32_t max_kv_len) { return (max_kv_len + dsa::kTkChunk - 1) / dsa::kTkChunk; }

struct TkLayout { size_t hist, cnt, surv, total; };
static TkLayout tk_layout(int32_t T, int32_t max_kv_len) {
  TkLayout L{};
  const int nch = tk_nch(max_kv_len);
  L.hist = 0;
  L.cnt = align256((size_t)T * dsa::kBins * 4);
  L.surv = L.cnt + align256((size_t)T * nch * 4);
  L.total = L.surv + align256((size_t)T * nch * dsa::kTkChunk * 8);
  return L;
}

extern "C" size_t dsa_topk_workspace_size(int32_t num_q, int32_t max_kv_len, int32_t k) {
  (void)k;
  if (num_q <= 0 || max_kv_len <= 0) return 0;
  return tk_layout(num_q, max_kv_len).total;
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
  if (bt->max_kv_len > 64 * dsa::kTkChunk) return fail(DSA_ERR_UNSUPPORTED, "%s: max_kv_len above %d", fn, 64 * dsa::kTkChunk);
  const TkLayout L = tk_layout(bt->num_q, bt->max_kv_len);
  if (!ws || ws_bytes < L.total) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, L.total);
  if ((uintptr_t)ws & 255) return fail(DSA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (bt->num_q > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: more than 65535 query tokens", fn);
  const int T = bt->num_q;
  dsa::TkArgs a{};
  a.q_pos = bt->q_pos; a.scores = scores; a.ld = ld; a.k = k; a.T = T; a.idx = idx;
  a.nch = tk_nch(bt->max_kv_len);
  char* w = (char*)ws;
  a.hist = (uint32_t*)(w + L.hist);
  a.cnt = (uint32_t*)(w + L.cnt);
  a.surv = (uint64_t*)(w + L.surv);
  hipStream_t s = (hipStream_t)stream;
  const dim3 g2((unsigned)a.nch, (unsigned)T);
  hipLaunchKernelGGL(dsa::topk_hist, g2, dim3(dsa::kTkNT), 0, s, a);
  hipLaunchKernelGGL(dsa::topk_select, g2, dim3(dsa::kTkNT), 0, s, a);
  hipLaunchKernelGGL(dsa::topk_finalize, dim3((unsigned)T), dim3(dsa::kFinNT), 0, s, a);
  return dsa_host::check_launch(fn);
}
