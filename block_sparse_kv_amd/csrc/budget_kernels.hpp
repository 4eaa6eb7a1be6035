// Head-adaptive budgets on gfx950: one budget per sequence, shared by its KV
// heads (Step-dLLM page, abstract: a head-adaptive global budget that
// compresses heads with concentrated attention harder).
//
// The sequence keeps the K = k * Hkv largest block-averaged scores over all
// of its (KV head, position) pairs. The scores of one sequence are Hkv rows
// of one stride each, so they form one row of Hkv * stride entries in which
// entry h * stride + p is (head h, position p): the ordinary top-k of that
// row (ties to the lower entry, so to the lower head, then the lower
// position) is the global selection. Entries past a paged sequence's length
// are zeroed first; scores are positive wherever a position exists, so a
// zero is only ever taken when fewer than K positions exist, and the split
// drops it. budget_split_kernel then cuts the ascending global entries into
// per-head index rows and counts.
#pragma once

#include "mage_common.hpp"

namespace mage {

struct GapZeroParams {
  float* scores;            // row u at scores + u * stride
  int64_t stride;
  int32_t rows, rows_per_seq;
  SeqLens lens;             // n of sequence u / rows_per_seq
};

// One work-group per row: entries [n, stride) of the row become +0.
__global__ __launch_bounds__(256) void gap_zero_kernel(GapZeroParams p) {
  const int u = blockIdx.x;
  if (u >= p.rows) return;
  const int n = p.lens.n[u / p.rows_per_seq];
  float* row = p.scores + static_cast<int64_t>(u) * p.stride;
  for (int64_t i = n + threadIdx.x; i < p.stride; i += 256) row[i] = 0.f;
}

struct BudgetSplitParams {
  const int32_t* gidx;      // [S][K]: ascending entries h * stride + p, then -1
  int32_t* idx;             // [S][Hkv][K]: head h's positions ascending, then -1
  int32_t* counts;          // [S][Hkv]
  int64_t stride;
  int32_t S, Hkv, K;
  int32_t n_uniform;        // >= 0: every sequence's length; else lens
  SeqLens lens;
};

// One work-group per (sequence, KV head). The row is ascending, so the head's
// segment starts at the number of entries below h * stride and ends at the
// number below h * stride + n (positions past n, zeroed gaps, are dropped):
// both are counted by all threads at once (independent loads) rather than
// found by a chain of dependent binary-search loads.
__global__ __launch_bounds__(256) void budget_split_kernel(BudgetSplitParams p) {
  __shared__ int s_part[2][256 / kWave];
  const int u = blockIdx.x;
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  if (s >= p.S) return;
  const int n = p.n_uniform >= 0 ? p.n_uniform : p.lens.n[s];
  const int32_t* g = p.gidx + static_cast<int64_t>(s) * p.K;
  const int64_t base = static_cast<int64_t>(h) * p.stride;
  int below_lo = 0, below_hi = 0;
  for (int j0 = threadIdx.x; j0 < p.K; j0 += 16 * 256) {   // sixteen loads in flight per step
    int32_t x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = j0 + q * 256 < p.K ? g[j0 + q * 256] : -1;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t v = x[q];
      below_lo += (v >= 0 && v < base) ? 1 : 0;
      below_hi += (v >= 0 && v < base + n) ? 1 : 0;
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    below_lo += __shfl_xor(below_lo, off, kWave);
    below_hi += __shfl_xor(below_hi, off, kWave);
  }
  if ((threadIdx.x & (kWave - 1)) == 0) {
    s_part[0][threadIdx.x / kWave] = below_lo;
    s_part[1][threadIdx.x / kWave] = below_hi;
  }
  __syncthreads();
  int lo = 0, hi = 0;
#pragma unroll
  for (int w = 0; w < 256 / kWave; ++w) {
    lo += s_part[0][w];
    hi += s_part[1][w];
  }
  const int cnt = hi - lo;
  int32_t* out = p.idx + static_cast<int64_t>(u) * p.K;
  for (int j0 = threadIdx.x; j0 < p.K; j0 += 16 * 256) {   // all loads of a step before its stores
    int32_t x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int j = j0 + q * 256;
      x[q] = j < cnt ? static_cast<int32_t>(g[lo + j] - base) : -1;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (j0 + q * 256 < p.K) out[j0 + q * 256] = x[q];
  }
  if (threadIdx.x == 0) p.counts[u] = cnt;
}

}  // namespace mage
