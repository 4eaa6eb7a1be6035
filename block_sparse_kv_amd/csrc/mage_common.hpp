// Shared device-side definitions for the gfx950 kernels of the MAGE hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mage {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;      // attention / score work-groups: 4 waves
constexpr int kTileKeys = 64;      // keys staged in LDS per iteration
constexpr int kMaxRows = 128;      // R = B * G rows per KV head, 4 row blocks of 32
constexpr int kMaxSeqs = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Query head of row (b, g) of KV head h: h * gs + g0 + g. A call whose head
// group holds more than kMaxRows rows (block * group) runs in sub-groups of
// G <= kMaxRows / block heads; gs is then the full group size and g0 the
// sub-group's first head (gs = 0: the group is not split).
__host__ __device__ __forceinline__ int q_head(int h, int g, int G, int gs, int g0) {
  return h * (gs ? gs : G) + g0 + g;
}

// Host-side sequence table carried in kernel arguments (ragged paged batches).
struct SeqLens {
  int32_t n[kMaxSeqs];
};

// Dense work-group numbering over (unit, chunk) pairs when the units' lengths
// differ (paged layout): the work-groups [first[s], first[s+1]) belong to
// sequence s, which has Hkv units of cdiv(n_s, chunk) chunks each (unit-major).
// A grid of first[S] work-groups then holds no empty (unit, chunk) slots,
// whose dispatch would delay the real ones.
struct ChunkMap {
  int32_t first[kMaxSeqs + 1];
  int32_t on;               // 0: uniform lengths, unit = wg / nchunk, chunk = wg % nchunk
};

__device__ __forceinline__ void map_chunk(const ChunkMap& m, const SeqLens& lens, int S, int Hkv, int chunk,
                                          int nchunk, int wg, int& u, int& c) {
  if (!m.on) {
    u = wg / nchunk;
    c = wg - u * nchunk;
    return;
  }
  int lo = 0, hi = S - 1;   // the last sequence whose first work-group is <= wg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m.first[mid] <= wg) lo = mid;
    else hi = mid - 1;
  }
  const int nch = (lens.n[lo] + chunk - 1) / chunk;
  const int local = wg - m.first[lo];
  const int h = local / nch;
  u = lo * Hkv + h;
  c = local - h * nch;
}

// KV row addressing shared by the exact pass, the score sweep and the sparse
// step. Contiguous: [S][Hkv][N][d]. Paged: pool [P][Hkv][page][d] with
// position p of sequence s in page table[s * max_pages + (p >> shift)].
struct KvSource {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;  // null for the contiguous layout
  int32_t max_pages;
  int32_t page_shift;
  int32_t n_uniform;          // contiguous prefix length (all sequences)
};

__device__ __forceinline__ int64_t kv_row(const KvSource& kv, int s, int h, int hkv, int p,
                                          int d) {
  if (kv.page_table == nullptr) {
    return ((static_cast<int64_t>(s) * hkv + h) * kv.n_uniform + p) * d;
  }
  const int64_t page = kv.page_table[static_cast<int64_t>(s) * kv.max_pages + (p >> kv.page_shift)];
  const int slot = p & ((1 << kv.page_shift) - 1);
  return (((page * hkv + h) << kv.page_shift) + slot) * d;
}

__device__ __forceinline__ int seq_len_of(const KvSource& kv, const SeqLens& lens, int s) {
  return kv.page_table ? lens.n[s] : kv.n_uniform;
}

// Lanes l and l ^ 32 hold the two halves of one row. v_permlane32_swap
// exchanges the upper half of one register with the lower half of another;
// with both operands = x, the two results hold x and x[l ^ 32] in every lane
// (in either order), so a symmetric combination of them is the pair result.
__device__ __forceinline__ float wave_max_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// bf16 pair (packed in one dword) -> two fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed fp16 pair, round to nearest even (one v_cvt_pk_f16_f32 on
// gfx950). Used for bf16 V values (exact in fp16 for |v| in [2^-14, 65504])
// and for probabilities in [0, 1].
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 r;
  r.x = static_cast<_Float16>(a);
  r.y = static_cast<_Float16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

#ifdef MAGE_TRACE
// Debug-only phase timestamps (100 MHz real-time counter) per work-group.
__device__ uint64_t g_trace[8192][8];
#define MAGE_TRACE_POINT(slot)                                              \
  do {                                                                      \
    if (threadIdx.x == 0 && blockIdx.x < 8192)                               \
      mage::g_trace[blockIdx.x][slot] = __builtin_amdgcn_s_memrealtime();  \
  } while (0)
#define MAGE_TRACE_NOW() __builtin_amdgcn_s_memrealtime()
// shader-clock counter beside the real-time one (row 4096 + work-group)
#define MAGE_TRACE_CLK(slot)                                                            \
  do {                                                                                  \
    if (threadIdx.x == 0 && blockIdx.x < 4096)                                          \
      mage::g_trace[4096 + blockIdx.x][slot] = __builtin_amdgcn_s_memtime();            \
  } while (0)
#define MAGE_TRACE_ADD(slot, v)                                             \
  do {                                                                      \
    if (threadIdx.x == 0 && blockIdx.x < 8192) mage::g_trace[blockIdx.x][slot] += (v); \
  } while (0)
#else
#define MAGE_TRACE_POINT(slot) \
  do {                         \
  } while (0)
#define MAGE_TRACE_NOW() 0ull
#define MAGE_TRACE_CLK(slot) \
  do {                       \
  } while (0)
#define MAGE_TRACE_ADD(slot, v) \
  do {                          \
  } while (0)
#endif

}  // namespace mage
