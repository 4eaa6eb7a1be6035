// Page-granular selection on gfx950: page scores from the block-averaged
// position scores, and the expansion of the chosen pages into positions.
//
// The block-sparse view of the selection (Step-dLLM page, abstract: a
// block-sparse mask; KV pages as the unit a gather reads): P consecutive
// positions form a page, a page's score is the sum of its positions' scores,
// the top pages per (sequence, KV head) come from the same top-k kernels as
// the position selection, and every chosen page is kept whole, so the later
// steps read P consecutive rows (4 KiB of K per page at P = 16, d = 128).
#pragma once

#include "mage_common.hpp"

namespace mage {

struct PageSumParams {
  const float* scores;      // row u at scores + u * stride, n_u valid entries
  int64_t stride;
  float* page_scores;       // row u at page_scores + u * pstride, cdiv(n_u, P) entries
  int64_t pstride;
  int32_t rows, rows_per_seq;
  int32_t n_uniform;        // >= 0: every row has this many positions; else lens
  int32_t page_tokens;      // P
  int32_t pages_max;        // cdiv(max n_u, P)
  int32_t vec4;             // every page starts 16-byte aligned (P and stride multiples of 4)
  SeqLens lens;
};

// One thread per (row, page); the page's positions are summed in position
// order in fp32 (a page score is at most 1, its relative rounding error about
// P * 2^-24).
__global__ __launch_bounds__(256) void page_sum_kernel(PageSumParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int row = static_cast<int>(i / p.pages_max);
  const int pg = static_cast<int>(i - static_cast<int64_t>(row) * p.pages_max);
  if (row >= p.rows) return;
  const int n = p.n_uniform >= 0 ? p.n_uniform : p.lens.n[row / p.rows_per_seq];
  const int64_t p0 = static_cast<int64_t>(pg) * p.page_tokens;
  if (p0 >= n) return;
  const int cnt = static_cast<int>(min(static_cast<int64_t>(p.page_tokens), n - p0));
  const float* src = p.scores + static_cast<int64_t>(row) * p.stride + p0;
  float s = 0.f;
  int t = 0;
  if (p.vec4) {   // four positions per load, added in the same order
    for (; t + 4 <= cnt; t += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + t);
      s += v[0];
      s += v[1];
      s += v[2];
      s += v[3];
    }
  }
  for (; t < cnt; ++t) s += src[t];
  p.page_scores[static_cast<int64_t>(row) * p.pstride + pg] = s;
}

struct PageExpandParams {
  const int32_t* page_idx;  // [rows][k_pages]: ascending page ids, then -1
  int32_t* idx;             // [rows][k_pages * P]: positions, -1 past n_u or for missing pages
  int32_t rows, rows_per_seq, n_uniform, k_pages, page_tokens;
  SeqLens lens;
};

// One thread per output slot (row, page slot j, offset t).
__global__ __launch_bounds__(256) void page_expand_kernel(PageExpandParams p) {
  const int64_t per_row = static_cast<int64_t>(p.k_pages) * p.page_tokens;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= per_row * p.rows) return;
  const int row = static_cast<int>(i / per_row);
  const int64_t rem = i - row * per_row;
  const int j = static_cast<int>(rem / p.page_tokens), t = static_cast<int>(rem % p.page_tokens);
  const int n = p.n_uniform >= 0 ? p.n_uniform : p.lens.n[row / p.rows_per_seq];
  const int pg = p.page_idx[static_cast<int64_t>(row) * p.k_pages + j];
  const int64_t pos = static_cast<int64_t>(pg) * p.page_tokens + t;
  p.idx[i] = (pg >= 0 && pos < n) ? static_cast<int32_t>(pos) : -1;
}

}  // namespace mage
