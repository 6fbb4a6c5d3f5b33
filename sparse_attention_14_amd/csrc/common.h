// Shared device/host helpers of the gfx950 DSA kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 is the upper half of an fp32; widening is exact.
__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<u16>(u >> 16);
}
// Two fp32 -> packed bf16 (a in the low half), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// fp16 <-> fp32 (IEEE binary16; narrowing rounds to nearest even).
__device__ __forceinline__ float f16_bits_to_f32(u16 h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ u16 f32_to_f16_bits(float f) {
  return __builtin_bit_cast(u16, static_cast<_Float16>(f));
}

// Make the compiler retire the load that produced `v` here (an empty asm that reads the
// register): used before a stream of loads issued from inline asm, so that the compiler's own
// later waits for such a register cannot also drain the asm-issued loads it cannot count.
template <typename T>
__device__ __forceinline__ void retire(const T& v) { asm volatile("" :: "v"(v)); }

// A pointer that is the same in every lane, moved to scalar registers (the direct-to-LDS loads
// take their base address from SGPRs).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Order-preserving key of an fp32 score: unsigned comparison of keys equals numeric comparison
// of the scores (-0.0 is mapped to +0.0 first, so the two compare equal).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr int kHistBins = 2048;          // top-k radix histogram: the top 11 bits of the key
constexpr int kHistShards = 4;           // copies of each row histogram (spread atomic traffic)
// The top-k select pass's per-row state in its workspace, read by the finalize pass and by the
// attention kernel that resolves its own slice of the selection: per chunk of kTkChunk scores,
// the count above the threshold digit and of candidates, a position bitmap and kTkCap
// candidate slots (key << 32 | position).
constexpr int kTkChunk = 4096;           // scores per chunk
constexpr int kTkCW = kTkChunk / 32;     // bitmap words per chunk
constexpr int kTkCap = 512;              // candidate slots per chunk
constexpr int kTkLoad = 4096;            // candidate entries of a row read in the first trip

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

// A workgroup barrier: __syncthreads(), or with LDS_ONLY a barrier that orders LDS traffic only
// (it does not wait for global loads in flight, e.g. direct-to-LDS DMA issued earlier).
template <bool LDS_ONLY>
__device__ __forceinline__ void block_barrier() {
  if constexpr (LDS_ONLY) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else __syncthreads();
}

// Exclusive prefix sum over the NT threads of the block (one barrier); `total` gets the sum.
// sh holds NT/64 words; consecutive uses of one sh must be separated by a barrier.
template <int NT, bool LDS_ONLY = false>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[w] = inc;
  block_barrier<LDS_ONLY>();
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
template <int NT, bool LDS_ONLY = false>
__device__ void find_digit_desc(const uint32_t* hist, uint32_t need, uint32_t* sh, uint32_t* res) {
  constexpr int PER = kHistBins / NT;
  const int tid = threadIdx.x;
  uint32_t loc[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { loc[j] = hist[kHistBins - 1 - (tid * PER + j)]; tot += loc[j]; }
  uint32_t all;
  uint32_t before = block_excl_scan<NT, LDS_ONLY>(tot, sh, all);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (before < need && need <= before + loc[j]) { res[0] = kHistBins - 1 - (tid * PER + j); res[1] = before; }
    before += loc[j];
  }
  block_barrier<LDS_ONLY>();
}

// Debug poisoning (DSA_DEBUG_POISON=1, race detection): fill an LDS object with all-one bytes --
// NaN as fp32/bf16, -1 as int, every bit set in a bitmap -- so that a read before the kernel's
// own write changes the results.  Called by every thread before any other LDS access.
__device__ __forceinline__ void poison_lds(void* p, unsigned bytes) {
  uint32_t* w = static_cast<uint32_t*>(p);
  for (unsigned i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xFFFFFFFFu;
}

// Flat workgroup id remapped so that consecutive logical ids land on one XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8); logical id
// w = xcd * per_xcd + slot keeps neighbours (which share data) in one L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int per = (n + 7) / 8;
  const int xcd = id % 8, slot = id / 8;
  const int full = n % 8 == 0 ? 8 : n % 8;           // XCDs that hold `per` items
  int w = xcd < full ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
  return w;
}

}  // namespace dsa

// Host-side helpers (defined in api.hip).
namespace dsa_host {
dsa_status fail(dsa_status st, const char* fmt, ...);
dsa_status check_launch(const char* what);
// DSA_DEBUG_POISON=1 in the environment: kernels poison their LDS before use and the library's
// written-before-read workspace regions are filled with all-one bytes before each call (a debug
// mode for eager calls; its fill kernels are not meant for graph capture)
bool debug_poison();
void poison_fill(void* p, size_t bytes, hipStream_t s);
// A selection still pending in the top-k workspace after the select pass (per-row threshold
// digit, per-chunk counts, bitmaps and candidate slots, the digit histograms), resolved by the
// attention kernel itself; idx receives the selection.  See sfa.hip / topk.hip.
struct SfaSel {
  const float* scores; long ld;
  const uint32_t* bg; const uint32_t* cnt; const uint32_t* bits; const uint64_t* slots;
  uint32_t* hist; uint32_t* hist2; int nch; int32_t* idx;
};
}  // namespace dsa_host
