// Anchor re-selection diagnostics on gfx950: the block's mean query and the
// overlap of two top-k index sets.
//
// Step-dLLM page (abstract): a sparse mask chosen at an anchor step is reused
// until the next anchor step, where it is chosen again. How much of a step's
// own top-k set the set in use still covers (its recall) is what decides the
// anchor period; idx_overlap_kernel counts that overlap per (sequence, KV
// head). The mean query is the other block query that the MAGE page's
// "Approach" (block-average query) can be read as: selecting by the
// probability under it is the main selection run on a one-row block.
#pragma once

#include <cmath>

#include "mage_common.hpp"

namespace mage {

struct MeanQueryParams {
  const uint16_t* q;   // bf16 [S][B][Hq][d]
  uint16_t* qbar;      // bf16 [S][Hkv][d] (= [S][1][Hkv][d])
  int32_t S, B, Hq, Hkv, G, D;
};

// bf16 nearest to x, ties to even, for x = 0 or |x| in the normal range:
// x = m * 2^e with |m| in [0.5, 1); rint (ties to even) of m * 2^8 keeps 8
// significant bits, so the rounded value is exact in fp32 and its upper half
// is the bf16 pattern. Both zeros give +0.
__device__ __forceinline__ uint16_t bf16_nearest_even(double x) {
  if (x == 0.0) return 0;
  int e = 0;
  const double m = frexp(x, &e);
  const double r = rint(ldexp(m, 8));
  const float f = static_cast<float>(ldexp(r, e - 8));
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// One thread per (sequence, KV head, dimension). The sum of the B*G bf16
// values in fp64 is exact unless their magnitudes span more than about 2^38,
// and the division is correctly rounded, so the result is the exact mean
// rounded once (a rounded quotient with a non-power-of-two divisor cannot land
// on a bf16 tie).
__global__ __launch_bounds__(256) void mean_query_kernel(MeanQueryParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(p.S) * p.Hkv * p.D) return;
  const int e = static_cast<int>(i % p.D);
  const int64_t sh = i / p.D;
  const int h = static_cast<int>(sh % p.Hkv), s = static_cast<int>(sh / p.Hkv);
  double acc = 0.0;
  for (int b = 0; b < p.B; ++b) {
    const uint16_t* row = p.q + ((static_cast<int64_t>(s) * p.B + b) * p.Hq + h * p.G) * p.D + e;
    for (int g = 0; g < p.G; ++g)
      acc += static_cast<double>(__uint_as_float(static_cast<uint32_t>(row[g * p.D]) << 16));
  }
  p.qbar[i] = bf16_nearest_even(acc / (static_cast<double>(p.B) * p.G));
}

struct OverlapParams {
  const int32_t* a;    // int32 [rows][k]: ascending valid entries, then negative padding
  const int32_t* b;    // int32 [rows][k], the same form
  int32_t* common;     // int32 [rows]: |valid(a) ∩ valid(b)|
  int32_t* count_a;    // int32 [rows] or null: |valid(a)|
  int32_t* count_b;    // int32 [rows] or null: |valid(b)|
  int32_t rows, k;
};

// Length of the valid (non-negative) prefix of an index row.
__device__ __forceinline__ int valid_prefix(const int32_t* r, int k) {
  int lo = 0, hi = k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (r[mid] >= 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// One work-group per row: every valid entry of a is looked up in b's valid
// prefix by binary search. Rows that break the ascending form give a
// meaningless count but every read stays inside the row.
constexpr int kOverlapThreads = 256;
__global__ __launch_bounds__(kOverlapThreads) void idx_overlap_kernel(OverlapParams p) {
  __shared__ int s_sum[kOverlapThreads / kWave];
  const int row = blockIdx.x;
  const int32_t* a = p.a + static_cast<int64_t>(row) * p.k;
  const int32_t* b = p.b + static_cast<int64_t>(row) * p.k;
  const int na = valid_prefix(a, p.k), nb = valid_prefix(b, p.k);
  int c = 0;
  for (int i = threadIdx.x; i < na; i += kOverlapThreads) {
    const int v = a[i];
    int lo = 0, hi = nb;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (b[mid] < v)
        lo = mid + 1;
      else
        hi = mid;
    }
    c += (lo < nb && b[lo] == v) ? 1 : 0;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) s_sum[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kOverlapThreads / kWave; ++w) t += s_sum[w];
    p.common[row] = t;
    if (p.count_a) p.count_a[row] = na;
    if (p.count_b) p.count_b[row] = nb;
  }
}

}  // namespace mage
