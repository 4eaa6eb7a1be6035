// Selection kernels of the MAGE hot path on gfx950: the block-averaged score
// sweep and the per-(sequence, KV head) top-k.
//
// Score (MAGE page, atlas.scime.ai summary, "Problem" and "Approach": the
// step-1 exact pass reveals one top-k subset for the whole block): for prefix
// position p of KV head h,
//     score[p] = (1/R) sum_r exp(scale q_r.k_p - M_r) / L_r
// over the R = B*G rows sharing the head, with (M_r, L_r) the row's final
// softmax max and sum from the exact pass. In log2 units the kernel computes
// exp2(x_r[p] - c_r) with c_r = M_r + log2 L_r.
//
// Top-k: the k_eff largest scores, ties to the lower position, ascending
// output. Scores are >= +0, so their fp32 bit patterns order like the values
// and the selection is integer work on those bits. The score sweep adds every
// score to a 1024-bin histogram of its row (top bits of the pattern); the
// top-k launch then finds the bin holding the row's k-th largest score, has
// each work-group compact its chunk's scores in that bin and above (in
// position order) to a candidate slice, and the row's last work-group runs an
// MSB-first radix select (8-bit digits, LDS histograms) over the candidates
// for the k-th largest pattern T and how many entries equal to T to keep; an
// index-ordered compaction (each thread owns a contiguous run, block prefix
// sums give the output offsets) keeps every entry > T and the
// lowest-positioned entries == T, so the output is already ascending.
#pragma once

#include "attn_kernels.hpp"
#include "mage_common.hpp"
#include "tile_io.hpp"

namespace mage {

// Cross-lane steps through DPP (data-parallel primitives: a VALU operand
// read from another lane of the same row of 16, or a row broadcast), which
// cost one dependent VALU operation each instead of an LDS permute round trip.
// dpp_ctrl codes: row_shr:n = 0x110 + n; row_bcast:15 = 0x142; row_bcast:31 = 0x143.
// Lanes whose source is outside the row, or whose row is masked off, read 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_read(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, kRowMask, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps
// 1, 2, 4, 8 inside each row of 16, then row 0's total is added to row 1 and
// row 2's to row 3 (row_bcast:15), then lane 31's sum to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += static_cast<int>(dpp_read<0x111, 0xf>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_read<0x112, 0xf>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_read<0x114, 0xf>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_read<0x118, 0xf>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_read<0x142, 0xa>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_read<0x143, 0xc>(static_cast<uint32_t>(v)));
  return v;
}

// Bitwise OR over the 64 lanes of a wave (the same steps as the scan; lane 63
// ends with the OR of every lane), returned uniform.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp_read<0x111, 0xf>(v);
  v |= dpp_read<0x112, 0xf>(v);
  v |= dpp_read<0x114, 0xf>(v);
  v |= dpp_read<0x118, 0xf>(v);
  v |= dpp_read<0x142, 0xa>(v);
  v |= dpp_read<0x143, 0xc>(v);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// x + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] in every lane: v_permlane16_swap and
// v_permlane32_swap with both operands = x give x and its partner lane's value
// (in either order), and the sum is symmetric.
__device__ __forceinline__ uint32_t sum_over_rows(uint32_t x) {
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] + a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] + b[1];
}


// Score histogram: bin of a non-negative fp32 score = its bit pattern >> 20
// (exponent and three mantissa bits: eighth-octave bins over [0, 2); every
// score >= 2 shares the top bin). Bit patterns order like the values, so the
// bin of the k-th largest score, read off a row's histogram, bounds the
// top-k: every score in a higher bin is in it, every score in a lower bin is
// not.
constexpr int kHistBins = 1024;
constexpr int kHistShift = 20;

__device__ __forceinline__ uint32_t hist_bin(uint32_t bits) {
  return min(bits >> kHistShift, static_cast<uint32_t>(kHistBins - 1));
}

// hist[bin] += 1 for every lane with `active` (one LDS atomic per lane: the
// LDS serializes same-bin lanes in hardware, which costs less than peeling
// off the wave's distinct bins in a loop).
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, uint32_t bin, bool active) {
  if (active) atomicAdd(&hist[bin], 1u);
}

// Adds a work-group's LDS histogram into the row's histogram in global memory
// (zero before the first work-group of the row adds to it): one device-scope
// atomic add per non-zero bin. A chunk's scores occupy a few dozen of the
// 1024 bins, so the adds of all the row's work-groups meet on few addresses
// and little at a time; adding every bin instead serializes 1024 adds per
// work-group at the memory side.
template <int kNT>
__device__ __forceinline__ void publish_hist(const uint32_t* s_hist, uint32_t* row_hist) {
  for (int b = threadIdx.x; b < kHistBins; b += kNT) {
    const uint32_t v = s_hist[b];
    if (v != 0u) __hip_atomic_fetch_add(row_hist + b, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct ScoreParams {
  const uint16_t* q;
  KvSource kv;
  const float* part_ml;     // the exact pass's split (max, sum) per (unit, chunk, row), log2 units
  int32_t exact_chunk;      // its keys per chunk and chunks per unit (slot = unit * exact_nchunk + chunk)
  int32_t exact_nchunk;
  float* scores;            // [S][Hkv][stride]
  int64_t stride;
  uint32_t* hist;           // [S * Hkv][kHistBins], zero on entry: each row's score histogram (or null)
  int32_t k;                // rows with min(k, N_s) == N_s take no histogram
  int32_t S, B, Hq, Hkv, G, R;
  int32_t gs, g0;           // query-head stride and sub-group offset (q_head)
  int32_t r_total;          // rows the score averages over (R, or the whole group's when split)
  int32_t accumulate;       // add to the scores already stored (later sub-groups of a split group)
  int32_t chunk, nchunk;
  int32_t reverse;          // sweep tiles last-to-first
  float scale_log2;
  SeqLens lens;
  ChunkMap map;             // work-group -> (unit, chunk)
};

// Positions per score work-group; sized so that two work-groups fit in one
// CU's LDS. Each work-group adds its chunk's histogram into the row's.
constexpr int kScoreChunk = 2048;      // positions per work-group (largest)
constexpr int kScoreChunkMin = 512;    // smallest, for short prefixes
constexpr int kStatBatch = 16;         // chunk statistics merged per batch (as the step-1 merge)

// The K tiles are loaded non-temporally (this sweep is their last use in the
// step). kPaged: the chunk's page ids are staged in LDS; the contiguous form
// leaves that table out, which lets four work-groups share a CU.
template <int D, int kStages, bool kPaged>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreParams p) {
  using G = TileGeom<D>;
  constexpr int kNks = D / 16;
  constexpr bool kNt = true;
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kStages * G::kBytes];
  __shared__ int32_t s_pages[kPaged ? kScoreChunk + 1 : 1];
  __shared__ float s_col[2][4][kTileKeys];
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ float s_crow[kMaxRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, n = lane & 31;
  int u, c;
  map_chunk(p.map, p.lens, p.S, p.Hkv, p.chunk, p.nchunk, blockIdx.x, u, c);
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  const int ns = seq_len_of(p.kv, p.lens, s);
  const int e0 = c * p.chunk, e1 = min(e0 + p.chunk, ns);
  if (e0 >= e1) return;
  const int nrb = (p.R + 31) >> 5;
  const bool computes = w < nrb;
  constexpr bool paged = kPaged;   // the host picks the form by the cache's layout
  const int pshift = p.kv.page_shift, pmask = (1 << p.kv.page_shift) - 1;
  const int64_t seq_base = paged ? 0 : (static_cast<int64_t>(s) * p.Hkv + h) * p.kv.n_uniform;
  const int page0 = e0 >> pshift;
  if (paged) {
    const int32_t* ptab = p.kv.page_table + static_cast<int64_t>(s) * p.kv.max_pages;
    const int np = ((e1 - 1) >> pshift) - page0 + 1;
    for (int i = tid; i < np; i += kThreads) s_pages[i] = ptab[page0 + i];
  }

  // A operand: Q row 32w + n, d slice 16ks + 8hh
  bf16x8 qf[kNks];
  {
    const int r = 32 * w + n;
    if (computes && r < p.R) {
      const int b = r / p.G, g = r - b * p.G;
      const uint16_t* qrow = p.q + ((static_cast<int64_t>(s) * p.B + b) * p.Hq + q_head(h, g, p.G, p.gs, p.g0)) * D;
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, load16(qrow + 16 * ks + 8 * hh));
    } else {
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  uint32_t kofs[kNks];
  k_frag_offsets<D>(n, hh, kofs);
  const uint32_t ring_base = lds_addr(s_ring);
  const float inv_r = 1.f / static_cast<float>(p.r_total);
  for (int b = tid; b < kHistBins; b += kThreads) s_hist[b] = 0u;
  __syncthreads();

  auto row_off = [&](int e) -> int64_t {
    const int pos = min(e, e1 - 1);
    if (paged) {
      const int64_t page = s_pages[(pos >> pshift) - page0];
      return (((page * p.Hkv + h) << pshift) + (pos & pmask)) * D;
    }
    return (seq_base + pos) * D;
  };
  const int ntiles = (e1 - e0 + kTileKeys - 1) / kTileKeys;
  // sweep order: last tile first when p.reverse (re-reads what the exact pass read last)
  auto tile_of = [&](int t) { return p.reverse ? ntiles - 1 - t : t; };
  // Tile loads are asm DMA (so the fragment reads below can be ordinary LDS
  // loads the compiler schedules): a full tile of contiguous rows (contiguous
  // layout, or 16-row-aligned in pages of >= 16 rows) takes the wave-uniform
  // base + fixed per-lane offset form; other tiles load row by row.
  constexpr int kKRowsPerInstr = kWave / G::kUnits;
  uint32_t koff[G::kInstr];
#pragma unroll
  for (int j = 0; j < G::kInstr; ++j) {
    const int slot = w * G::kInstr + j;
    const int unit = slot * kWave + lane;
    const int r = unit / G::kUnits, uk = (unit % G::kUnits) ^ (r & (G::kUnits - 1));
    koff[j] = static_cast<uint32_t>(((r - slot * kKRowsPerInstr) * D + uk * 8) * 2);
  }
  const bool fast_rows = !paged || pshift >= 4;
  const char* kbytes = reinterpret_cast<const char*>(p.kv.k);
  auto row_bytes = [&](int pos) -> int64_t {
    if (paged) {
      const int64_t page = __builtin_amdgcn_readfirstlane(s_pages[(pos >> pshift) - page0]);
      return ((((page * p.Hkv + h) << pshift) + (pos & pmask)) * D) * 2;
    }
    return ((seq_base + pos) * D) * 2;
  };
  // A wave's slices cover tile rows wrow .. wrow + 15, contiguous in memory
  // (one page of >= 16 rows when paged), so a full tile takes one row address
  // per wave (one page-list read) plus per-lane offsets fixed for the loop.
  constexpr int kWaveRows = G::kInstr * kKRowsPerInstr;
  static_assert(kWaveRows == 16, "a wave's slices span 16 tile rows");
  const int wrow = w * kWaveRows;
  uint32_t k_lane[G::kInstr];
#pragma unroll
  for (int j = 0; j < G::kInstr; ++j) k_lane[j] = koff[j] + static_cast<uint32_t>(j * kKRowsPerInstr * G::kRowBytes);
  auto issue = [&](int t) {
    const int base = e0 + tile_of(t) * kTileKeys;
    const uint32_t st = ring_base + (t % kStages) * G::kBytes + static_cast<uint32_t>(w * G::kInstr * 1024);
    if (fast_rows && base + kTileKeys <= e1 && (!paged || (base & 15) == 0)) {
      const char* rows = kbytes + row_bytes(base + wrow);
#pragma unroll
      for (int j = 0; j < G::kInstr; ++j) dma16<kNt>(rows, k_lane[j], st + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < G::kInstr; ++j) {
        const int slot = w * G::kInstr + j;
        const int unit = slot * kWave + lane;
        const int r = unit / G::kUnits, uk = (unit % G::kUnits) ^ (r & (G::kUnits - 1));
        dma16_sync<kNt>(p.kv.k + row_off(base + r) + uk * 8, st + j * 1024);
      }
    }
  };
  // column sums of tile t live in s_col[t & 1]; one iteration later (one
  // barrier per tile) each wave reduces 16 of the columns over the row blocks
  // column col of tile t: the sum over the row blocks, scaled, stored and
  // counted in the histogram
  auto reduce_store = [&](int t, int col) {
    const int e = e0 + tile_of(t) * kTileKeys + col;
    float sc = 0.f;
    if (e < e1) {
      float sum = 0.f;
      for (int ww = 0; ww < nrb; ++ww) sum += s_col[t & 1][ww][col];
      float* dst = p.scores + static_cast<int64_t>(u) * p.stride + e;
      sc = sum * inv_r;
      if (p.accumulate) sc = *dst + sc;
      *dst = sc;
    }
    wave_hist_add(s_hist, hist_bin(__float_as_uint(sc)), e < e1);
  };
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < ntiles) issue(t);
  // while the first tiles load: each row's final max + log2(sum) over the
  // whole prefix, the merge of the exact pass's chunk statistics (the same
  // arithmetic as the step-1 merge), one row per thread. (The wait for these
  // loads also covers the tile loads issued before them.)
  if (tid < kMaxRows) {
    float M, L;
    const int nchx = (ns + p.exact_chunk - 1) / p.exact_chunk;
    merge_row_stats<kStatBatch>(p.part_ml, static_cast<int64_t>(u) * p.exact_nchunk, nchx, tid, M, L);
    s_crow[tid] = M + __log2f(L);
  }
  __syncthreads();
  // accumulator register i of this lane is row 32w + 8(i/4) + 4hh + (i%4);
  // crow = -(max + log2 sum) of that row (rows past R: -inf, probability 0)
  float crow[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
    crow[i] = (computes && r < p.R) ? -s_crow[r] : -__builtin_inff();
  }
  for (int t = 0; t < ntiles; ++t) {
    wait_tiles<G::kInstr, kStages - 1>(min(kStages - 2, ntiles - 1 - t));
    wg_barrier();
    if (t + kStages - 1 < ntiles) issue(t + kStages - 1);
    // each wave reduces 16 of the previous tile's columns (lanes 0-15)
    if (t > 0 && lane < kTileKeys / 4) reduce_store(t - 1, 16 * w + lane);
    const uint32_t k_base = ring_base + (t % kStages) * G::kBytes;
    if (computes) {
      f32x16 acc[2];
      bf16x8 kf[2][kNks];
      // both halves' fragment reads go out together; each product starts
      // when its own fragments have landed
      k_frags_lds<D>(k_base, kofs, kf[0]);
      k_frags_lds<D>(k_base + 32 * G::kRowBytes, kofs, kf[1]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[kb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < kNks; ++ks)
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf[kb][ks], acc[kb], 0, 0, 0);
      }
      // S[row][key 32kb + n]; sum the probabilities of this wave's 32 rows
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float col = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) col += fast_exp2(__builtin_fmaf(acc[kb][i], p.scale_log2, crow[i]));
        col = wave_sum_pair(col);
        if (hh == 0) s_col[t & 1][w][32 * kb + n] = col;
      }
    }
    wait_lgkmcnt0();
  }
  __syncthreads();
  if (lane < kTileKeys / 4) reduce_store(ntiles - 1, 16 * w + lane);
  if (p.hist == nullptr || min(p.k, ns) == ns) return;   // every position is selected: no histogram
  __syncthreads();
  publish_hist<kThreads>(s_hist, p.hist + static_cast<int64_t>(u) * kHistBins);
}

// ---------------------------------------------------------------------------
// top-k

// Top-k work-group: 1024 threads. In its candidate phase it takes
// a chunk of one row (kLocalChunk or kWideChunk positions); the last of a
// row's work-groups then selects among the row's candidates on its register
// path, which holds up to kFinalMax entries (8 per thread), or kFinalMaxWide
// (12 per thread, for large k) in the wide variant.
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kFinalMax = 8192;
constexpr int kFinalMaxWide = 12288;
// candidates per thread that the final pass holds in registers when more
// than the LDS takes (rows with many scores in the k-th score's bin)
constexpr int kOverflowPer = 24;
constexpr int kLocalChunk = 4096;
// candidate chunk of rows whose 4096-position chunks would take more than one
// round of the CUs (many or long rows): half the work-groups, each with twice
// the positions
constexpr int kWideChunk = 8192;
// histogram pass of the standalone top-k: one 256-thread work-group per chunk
constexpr int kHistThreads = 256;
// chunks per row the final pass can index (rows up to 2^25 positions)
constexpr int kMaxLocalChunks = 8192;

struct TopkParams {
  const float* scores;      // row u at scores + u * stride
  int64_t stride;
  int32_t* idx;             // [rows][k]
  int32_t k;
  uint32_t* hist;           // [rows][kHistBins]: the row's score histogram (complete before the
                            //   top-k launch: built by the score sweep or topk_hist_kernel)
  uint32_t* cand_bits;      // per row: chunk c's candidates at c * chunk
  int32_t* cand_pos;
  int64_t cand_stride;      // nchunk * chunk
  int32_t* cand_count;      // [rows][nchunk]
  uint32_t* arrivals;       // [rows]: work-groups of the row done with their candidates; zero on entry
  int32_t rows;
  int32_t rows_per_seq;     // row u belongs to sequence u / rows_per_seq
  int32_t n_uniform;        // >= 0: every row has this many entries; else lens
  int32_t nchunk;
  SeqLens lens;
  ChunkMap map;             // work-group -> (row, chunk of `chunk` positions)
  int32_t chunk;            // positions per candidate chunk: kLocalChunk or kWideChunk
};

struct TopkShared {
  uint32_t hist[4096 + 256];
  __attribute__((aligned(16))) int32_t wsum[kTopkWaves];
  __attribute__((aligned(16))) int32_t wsum2[kTopkWaves];
  int32_t res[3];
};

// Sum of the kW per-wave values in w[] (vector LDS reads, broadcast to all
// lanes) and the part of it contributed by waves below `wv`.
template <int kW>
__device__ __forceinline__ void wave_totals(const int32_t* w, int wv, int& below, int& total) {
  static_assert(kW % 4 == 0, "whole 16-byte reads");
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4* v = reinterpret_cast<const i4*>(w);
  below = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < kW / 4; ++q) {
    const i4 x = v[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      total += x[e];
      below += (4 * q + e < wv) ? x[e] : 0;
    }
  }
}

// Block-wide inclusive prefix sum of one int per thread (kW waves); also
// returns the total. wsum: kW ints of LDS, 16-byte aligned.
template <int kW = kTopkWaves>
__device__ __forceinline__ int block_inclusive_scan(int v, int32_t* wsum, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  int before;
  wave_totals<kW>(wsum, wv, before, total);
  __syncthreads();
  return v + before;
}

// Bitwise OR over the work-group (one value per thread); result valid after return.
__device__ __forceinline__ uint32_t block_or(uint32_t v, int32_t* wsum) {
  v = wave_or(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) wsum[wv] = static_cast<int32_t>(v);
  __syncthreads();
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4* w = reinterpret_cast<const i4*>(wsum);
  uint32_t all = 0;
#pragma unroll
  for (int q = 0; q < kTopkWaves / 4; ++q) {
    const i4 x = w[q];
    all |= static_cast<uint32_t>(x[0] | x[1] | x[2] | x[3]);
  }
  __syncthreads();
  return all;
}

// MSB-first radix select over n bit patterns: the kk-th largest value T, and
// how many entries equal to T belong to the top kk (need >= 1). The bits
// above the highest bit in which the entries differ are common to all of them
// and are skipped, so the first 12-bit digit already separates the values
// (a digit taken from the sign and exponent alone would send most scores to a
// few histogram bins and serialize the LDS atomics).
template <class Get>
__device__ void radix_select(Get data, int n, int kk, TopkShared& sh, uint32_t& T, int& need) {
  const int tid = threadIdx.x;
  const uint32_t first = data(0);
  uint32_t diff = 0;
  for (int i = tid; i < n; i += kTopkThreads) diff |= data(i) ^ first;
  diff = block_or(diff, sh.wsum);
  if (diff == 0) {  // all entries equal
    T = first;
    need = kk;
    return;
  }
  int hi = 31 - __clz(diff);  // highest differing bit
  uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
  uint32_t prefix = first & pmask;
  int rem = kk;
  while (hi >= 0) {
    const int width = min(12, hi + 1), lo = hi - width + 1, nb = 1 << width;
    for (int i = tid; i < nb; i += kTopkThreads) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t x = data(i);
      if ((x & pmask) == prefix) atomicAdd(&sh.hist[(x >> lo) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins [t*per, t*per + per); count above = entries with larger digits
    const int per = (nb + kTopkThreads - 1) / kTopkThreads;
    const int b0 = tid * per;
    int mine = 0;
    for (int b = 0; b < per; ++b)
      if (b0 + b < nb) mine += static_cast<int>(sh.hist[b0 + b]);
    int total;
    const int incl = block_inclusive_scan(mine, sh.wsum, total);
    int above = total - incl;  // entries in bins above this thread's range
    for (int b = per - 1; b >= 0; --b) {
      const int bin = b0 + b;
      if (bin >= nb) continue;
      const int cnt = static_cast<int>(sh.hist[bin]);
      if (above < rem && rem <= above + cnt) {
        sh.res[0] = bin;
        sh.res[1] = rem - above;
      }
      above += cnt;
    }
    __syncthreads();
    const int digit = sh.res[0];
    rem = sh.res[1];
    prefix |= static_cast<uint32_t>(digit) << lo;
    pmask |= static_cast<uint32_t>(nb - 1) << lo;
    __syncthreads();
    hi = lo - 1;
  }
  T = prefix;
  need = rem;
}

// Keep entries > T and the first `need` entries == T, in index order.
// Writes out_pos[j] = pos_of(i) (and out_bits[j] = data(i) if out_bits).
// Thread t owns the contiguous run [t*per, t*per + per); two block-wide scans
// (of the runs' equal-to-T counts, then of their selected counts) give every
// thread its output offset, so the loop over the data has no barriers.
template <class Get, class PosOf>
__device__ void ordered_compact(Get data, int n, uint32_t T, int need, PosOf pos_of,
                                uint32_t* out_bits, int32_t* out_pos, TopkShared& sh, int cap) {
  const int tid = threadIdx.x;
  const int per = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  int n_eq = 0;
  for (int i = i0; i < i1; ++i) n_eq += data(i) == T;
  int eq_total;
  const int eq_before = block_inclusive_scan(n_eq, sh.wsum, eq_total) - n_eq;
  // equal-to-T entries this run keeps: ranks eq_before .. eq_before + n_eq - 1, those below need
  const int keep_eq = max(0, min(n_eq, need - eq_before));
  int n_sel = keep_eq;
  for (int i = i0; i < i1; ++i) n_sel += data(i) > T;
  int sel_total;
  int o = block_inclusive_scan(n_sel, sh.wsum2, sel_total) - n_sel;
  int eq_seen = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = data(i);
    bool sel = x > T;
    if (x == T) sel = eq_seen++ < keep_eq;
    if (sel) {
      if (o < cap) {
        out_pos[o] = pos_of(i);
        if (out_bits) out_bits[o] = x;
      }
      ++o;
    }
  }
}

// ---- register-resident variants -------------------------------------------
// Thread t holds the contiguous run of elements [t*kPer, t*kPer + kPer) in
// registers (entries at or past n are invalid). Histograms are per wave
// (16 waves x 256 bins of 8-bit digits): atomics only meet inside a wave, where
// scores sharing their top bits would otherwise queue on a few LDS words.
template <int kPer>
__device__ __forceinline__ int run_valid(int n) {
  return max(0, min(kPer, n - static_cast<int>(threadIdx.x) * kPer));
}

// eq_total (optional) receives the number of entries equal to T: the count of
// the bin chosen in the last pass, which holds exactly the entries equal to T.
template <int kPer>
__device__ void radix_select_regs(const uint32_t (&v)[kPer], int n, int kk, TopkShared& sh, uint32_t& T,
                                  int& need, int* eq_total = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nv = run_valid<kPer>(n);
  if (tid == 0) sh.res[0] = static_cast<int32_t>(v[0]);
  __syncthreads();
  const uint32_t first = static_cast<uint32_t>(sh.res[0]);
  uint32_t diff = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j < nv) diff |= v[j] ^ first;
  diff = block_or(diff, sh.wsum);
  if (diff == 0) {  // all entries equal
    T = first;
    need = kk;
    if (eq_total) *eq_total = n;
    return;
  }
  int hi = 31 - __clz(diff);
  uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
  uint32_t prefix = first & pmask;
  int rem = kk, bin_count = 0;
  uint32_t* hist = sh.hist + wv * 256;          // this wave's histogram
  uint32_t* total = sh.hist + kTopkWaves * 256;  // bin totals over the waves
  while (hi >= 0) {
    const int width = min(8, hi + 1), lo = hi - width + 1, nb = 1 << width;
#pragma unroll
    for (int b = lane; b < 256; b += kWave) hist[b] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j < nv && (v[j] & pmask) == prefix) atomicAdd(&hist[(v[j] >> lo) & (nb - 1)], 1u);
    __syncthreads();
    // wave w totals bins 16w .. 16w+15 over the 16 wave histograms
    {
      const int bin = wv * 16 + (lane & 15), part = lane >> 4;   // 4 lanes per bin, 4 histograms each
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < kTopkWaves / 4; ++q) c += sh.hist[(part * (kTopkWaves / 4) + q) * 256 + bin];
      c = sum_over_rows(c);
      if (lane < 16) total[bin] = c;
    }
    __syncthreads();
    if (wv == 0) {
      // lane l holds the 4 bins of digits 4(63-l) .. 4(63-l)+3 (largest digits in lane 0)
      typedef uint32_t u4 __attribute__((ext_vector_type(4)));
      const u4 c4 = reinterpret_cast<const u4*>(total)[63 - lane];
      const int s = static_cast<int>(c4[0] + c4[1] + c4[2] + c4[3]);
      const int incl = wave_inclusive_scan(s);
      int above = incl - s;
      if (above < rem && rem <= incl) {
        for (int e = 3; e >= 0; --e) {
          const int c = static_cast<int>(c4[e]);
          if (above < rem && rem <= above + c) {
            sh.res[0] = 4 * (63 - lane) + e;
            sh.res[1] = rem - above;
            sh.res[2] = c;
          }
          above += c;
        }
      }
    }
    __syncthreads();
    const int digit = sh.res[0];
    rem = sh.res[1];
    bin_count = sh.res[2];
    prefix |= static_cast<uint32_t>(digit) << lo;
    pmask |= static_cast<uint32_t>(nb - 1) << lo;
    hi = lo - 1;
  }
  T = prefix;
  need = rem;
  if (eq_total) *eq_total = bin_count;
  __syncthreads();   // res is rewritten by the next select
}

// The same (T, need) as radix_select_regs, with less work when the k-th value
// sits in a sparse part of the distribution (the usual case for top-k of a
// softmax average): the first 8-bit digit is histogrammed over a sample (each
// thread's first element), a window of digits around the sample's k-th value
// is chosen with a margin, one packed block scan gives the exact numbers of
// entries above (A) and inside (M) the window, the window's entries are
// compacted to `cand` (LDS, kCand entries), and the remaining digits are
// selected among them (the kk-th largest overall is the (kk - A)-th largest
// candidate, and every entry equal to it is a candidate). When the window
// misses the k-th value or holds more than kCand entries, the full select runs.
constexpr int kCand = 2 * kTopkThreads;

template <int kPer>
__device__ void radix_select_sampled(const uint32_t (&v)[kPer], int n, int kk, TopkShared& sh, uint32_t* cand,
                                     uint32_t& T, int& need, int& eq_total) {
  eq_total = -1;   // unknown unless the candidate path computes it
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nv = run_valid<kPer>(n);
  if (tid == 0) sh.res[0] = static_cast<int32_t>(v[0]);
  __syncthreads();
  const uint32_t first = static_cast<uint32_t>(sh.res[0]);
  uint32_t diff = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j < nv) diff |= v[j] ^ first;
  diff = block_or(diff, sh.wsum);
  MAGE_TRACE_POINT(4);
  if (diff == 0) {  // all entries equal
    T = first;
    need = kk;
    return;
  }
  const int hi = 31 - __clz(diff);
  const int width = min(8, hi + 1), lo = hi - width + 1, nb = 1 << width;
  uint32_t* total = sh.hist + kTopkWaves * 256;
  if (tid < 256) total[tid] = 0u;
  if (tid == 0) {
    sh.res[0] = nb - 1;  // defaults: window from the top digit ...
    sh.res[1] = 0;       // ... down to the bottom one
  }
  __syncthreads();
  const int m = min(kTopkThreads, (n + kPer - 1) / kPer);  // threads holding data = sample size
  if (nv > 0) atomicAdd(&total[(v[0] >> lo) & (nb - 1)], 1u);
  __syncthreads();
  if (wv == 0) {
    // lane l holds digits 4(63-l)+3 .. 4(63-l) (largest digits in lane 0)
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 c4 = reinterpret_cast<const u4*>(total)[63 - lane];
    const int s4 = static_cast<int>(c4[0] + c4[1] + c4[2] + c4[3]);
    const int incl = wave_inclusive_scan(s4);
    // sample counts at the k-th value: kk * m / n; window edges a quarter + 4 away
    const float tk = static_cast<float>(kk) * static_cast<float>(m) / static_cast<float>(n);
    const float t_hi = 0.75f * tk - 4.f, t_lo = 1.25f * tk + 4.f;
    int above = incl - s4;
    for (int e = 3; e >= 0; --e) {
      const int c = static_cast<int>(c4[e]);
      const int d = 4 * (63 - lane) + e;
      // the digit at which the count of samples >= digit first exceeds the edge
      if (static_cast<float>(above) <= t_hi && static_cast<float>(above + c) > t_hi) sh.res[0] = d;
      if (static_cast<float>(above) <= t_lo && static_cast<float>(above + c) > t_lo) sh.res[1] = d;
      above += c;
    }
  }
  __syncthreads();
  const int d_hi = sh.res[0], d_lo = sh.res[1];
  MAGE_TRACE_POINT(5);
  // exact counts above and inside the window, packed (both totals < 2^16)
  int a_loc = 0, m_loc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j < nv) {
      const int d = static_cast<int>((v[j] >> lo) & (nb - 1));
      a_loc += d > d_hi;
      m_loc += (d >= d_lo && d <= d_hi);
    }
  const int packed = (a_loc << 16) | m_loc;
  int tot;
  const int incl = block_inclusive_scan(packed, sh.wsum, tot);
  const int A = tot >> 16, M = tot & 0xffff;
  MAGE_TRACE_POINT(6);
  if (!(A < kk && kk <= A + M) || M > kCand) {
    radix_select_regs<kPer>(v, n, kk, sh, T, need, &eq_total);
    return;
  }
  int o = (incl - packed) & 0xffff;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j < nv) {
      const int d = static_cast<int>((v[j] >> lo) & (nb - 1));
      if (d >= d_lo && d <= d_hi) cand[o++] = v[j];
    }
  __syncthreads();
  MAGE_TRACE_POINT(7);
  uint32_t c2[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) c2[q] = cand[min(2 * tid + q, M - 1)];
  radix_select_regs<2>(c2, M, kk - A, sh, T, need, &eq_total);
}

// Keep entries > T and the first `need` entries == T, in index order:
// out_pos[o] = pos_of(j) (and out_bits[o] = value if out_bits).
// eq_total: the number of entries equal to T if known (>= 0); when it equals
// need, every such entry is kept and the scan of tie ranks is skipped.
template <int kPer, class PosOf>
__device__ void ordered_compact_regs(const uint32_t (&v)[kPer], int n, uint32_t T, int need, PosOf pos_of,
                                     uint32_t* out_bits, int32_t* out_pos, TopkShared& sh, int eq_total,
                                     int cap) {
  const int nv = run_valid<kPer>(n);
  int n_eq = 0, n_gt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j < nv) {
      n_eq += v[j] == T;
      n_gt += v[j] > T;
    }
  int keep_eq = n_eq;
  if (eq_total != need) {
    int eq_all;
    const int eq_before = block_inclusive_scan(n_eq, sh.wsum, eq_all) - n_eq;
    keep_eq = max(0, min(n_eq, need - eq_before));
  }
  const int n_sel = keep_eq + n_gt;
  int sel_total;
  int o = block_inclusive_scan(n_sel, sh.wsum2, sel_total) - n_sel;
  int eq_seen = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j >= nv) break;
    bool sel = v[j] > T;
    if (v[j] == T) sel = eq_seen++ < keep_eq;
    if (sel) {
      if (o < cap) {   // (a consistent T and need select exactly cap entries)
        out_pos[o] = pos_of(j);
        if (out_bits) out_bits[o] = v[j];
      }
      ++o;
    }
  }
}

// Read thread t's run [t*kPer, t*kPer + kPer) of an LDS array (16-byte reads).
template <int kPer>
__device__ __forceinline__ void load_run(const uint32_t* lds, uint32_t (&v)[kPer]) {
  static_assert(kPer % 4 == 0, "runs of whole 16-byte words");
  const u32x4* src = reinterpret_cast<const u32x4*>(lds + threadIdx.x * kPer);
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const u32x4 x = src[q];
    v[4 * q] = x[0];
    v[4 * q + 1] = x[1];
    v[4 * q + 2] = x[2];
    v[4 * q + 3] = x[3];
  }
}

__device__ __forceinline__ int topk_row_len(const TopkParams& p, int u) {
  return p.n_uniform >= 0 ? p.n_uniform : p.lens.n[u / p.rows_per_seq];
}

// Zeroes the histograms and arrival counters of the standalone top-k's rows
// (the step-1 path has the exact pass do this). One work-group per row.
__global__ __launch_bounds__(kHistThreads) void topk_prep_kernel(TopkParams p) {
  const int u = blockIdx.x;
  if (u >= p.rows) return;
  for (int b = threadIdx.x; b < kHistBins; b += kHistThreads) p.hist[static_cast<int64_t>(u) * kHistBins + b] = 0u;
  if (threadIdx.x == 0) p.arrivals[u] = 0u;
}

// Histograms of user-supplied rows (the standalone top-k entry point; the
// selection path builds them in the score sweep). One work-group per (row,
// chunk) adds its chunk's histogram into the row's.
template <int kChunk>
__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(TopkParams p) {
  constexpr int kPer = kChunk / kHistThreads;
  __shared__ uint32_t s_hist[kHistBins];
  const int tid = threadIdx.x;
  int u, c;
  map_chunk(p.map, p.lens, p.rows / p.rows_per_seq, p.rows_per_seq, kChunk, p.nchunk, blockIdx.x, u, c);
  if (u >= p.rows) return;
  const int n = topk_row_len(p, u);
  const int start = c * kChunk;
  if (min(p.k, n) == n || start >= n) return;   // such rows need no histogram
  const int len = min(kChunk, n - start);
  for (int b = tid; b < kHistBins; b += kHistThreads) s_hist[b] = 0u;
  __syncthreads();
  const float* src = p.scores + static_cast<int64_t>(u) * p.stride + start;
  uint32_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = __float_as_uint(src[min(tid + j * kHistThreads, len - 1)]);
#pragma unroll
  for (int j = 0; j < kPer; ++j) wave_hist_add(s_hist, hist_bin(v[j]), tid + j * kHistThreads < len);
  __syncthreads();
  publish_hist<kHistThreads>(s_hist, p.hist + static_cast<int64_t>(u) * kHistBins);
}

// Agent-scope (cache bit sc1) accesses for what one work-group of a launch
// hands to another (relaxed agent-scope atomics); count_in orders them.
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Selection inside bin b* (< kHistBins - 1) by one wave: the rem-th largest
// (rem >= 1) of the m <= kWaveSelMax values in cand[] (all of them in bin b*,
// so only their low kHistShift = 20 bits differ), in MSB-first radix passes of
// 7, 7 and 6 bits over a wave-private LDS histogram (no work-group barriers).
// Returns the value T, how many values equal to T are among the rem largest
// (need), and how many values equal T (eq).
constexpr int kWaveSelMax = 512;

__device__ void wave_select_in_bin(const uint32_t* cand, int m, int rem, uint32_t bin_lo, uint32_t* whist,
                                   uint32_t& T, int& need, int& eq) {
  constexpr int kPer = kWaveSelMax / kWave;
  const int lane = threadIdx.x & 63;
  uint32_t c[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) c[j] = cand[min(lane + j * kWave, max(m - 1, 0))];
  uint32_t prefix = 0, pmask = 0;
  int cnt = 0;
  static_assert(kHistShift == 20, "passes cover bits 19..0");
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int width = pass < 2 ? 7 : 6, shift = pass == 0 ? 13 : (pass == 1 ? 6 : 0);
    const uint32_t dmask = (1u << width) - 1u;
    whist[2 * lane] = 0u;
    whist[2 * lane + 1] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (lane + j * kWave < m && (c[j] & pmask) == prefix) atomicAdd(&whist[(c[j] >> shift) & dmask], 1u);
    __builtin_amdgcn_wave_barrier();
    // lane l holds digits 127-2l and 126-2l (largest digits in lane 0)
    const int h0 = static_cast<int>(whist[127 - 2 * lane]), h1 = static_cast<int>(whist[126 - 2 * lane]);
    const int incl = wave_inclusive_scan(h0 + h1), above = incl - h0 - h1;
    const bool mine = above < rem && rem <= incl;
    const int src = __builtin_ctzll(__ballot(mine));
    int digit = 0, r2 = 0, c2 = 0;
    if (mine) {
      const bool first = rem <= above + h0;
      digit = first ? 127 - 2 * lane : 126 - 2 * lane;
      r2 = first ? rem - above : rem - above - h0;
      c2 = first ? h0 : h1;
    }
    digit = __builtin_amdgcn_readlane(digit, src);
    rem = __builtin_amdgcn_readlane(r2, src);
    cnt = __builtin_amdgcn_readlane(c2, src);
    prefix |= static_cast<uint32_t>(digit) << shift;
    pmask |= dmask << shift;
    __builtin_amdgcn_wave_barrier();
  }
  T = bin_lo | prefix;
  need = rem;
  eq = cnt;
}

// Top-k of every row, one launch. Work-group (row u, chunk c of kChunk
// positions):
//   1. From the row's histogram, the bin b* that holds the row's k-th largest
//      score: every score in a higher bin is in the top k, none in a lower one.
//   2. The chunk's scores in bins >= b*, in position order, go to the chunk's
//      candidate slice (device-scope stores), and their number to cand_count.
//   3. The work-group counts itself in on the row's arrival counter (count_in:
//      after its stores have drained); the last of the row's work-groups selects among
//      the row's candidates: the chunks' slices taken in chunk order are in
//      position order, the kk-th largest among them is the row's kk-th largest
//      (every larger score is a candidate), and the ordered compaction keeps
//      ties at the lowest positions, so the output is ascending.
// Rows whose every position is selected are written in step 1's place.
template <int kMax, int kChunk>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(TopkParams p) {
  constexpr int kLocalPer = kChunk / kTopkThreads;   // positions per thread in the candidate phase
  __shared__ uint32_t s_data[2 * kMax];   // bits, then positions (final pass)
  __shared__ int32_t s_off[kMaxLocalChunks + 1];
  __shared__ TopkShared sh;
  __shared__ int32_t s_sel[3];           // b*, scores in bins above b*, last arriver
  const int tid = threadIdx.x;
  int u, c;
  map_chunk(p.map, p.lens, p.rows / p.rows_per_seq, p.rows_per_seq, kChunk, p.nchunk, blockIdx.x, u, c);
  if (u >= p.rows) return;
  const int n = topk_row_len(p, u);
  const int kk = min(p.k, n);
  const int start = c * kChunk;
  if (start >= n) return;
  const int len = min(kChunk, n - start);
  int32_t* out = p.idx + static_cast<int64_t>(u) * p.k;
  MAGE_TRACE_POINT(0);
  if (kk == n) {  // every position is selected
    for (int i = tid; i < len; i += kTopkThreads) out[start + i] = start + i;
    if (c == 0)
      for (int i = n + tid; i < p.k; i += kTopkThreads) out[i] = -1;
    return;
  }
  // ---- 1. b* from the row histogram: thread t holds bin kHistBins-1-t (the largest in thread 0)
  uint32_t v[kLocalPer];
  {
    // this thread's run [start + t*kLocalPer, +kLocalPer) of the chunk, loads issued first
    const float* src = p.scores + static_cast<int64_t>(u) * p.stride + start;
#pragma unroll
    for (int j = 0; j < kLocalPer; ++j) v[j] = __float_as_uint(src[min(tid * kLocalPer + j, len - 1)]);
  }
  if (tid == 0) {
    s_sel[0] = 0;   // (a histogram that misses kk scores keeps everything)
    s_sel[1] = 0;
  }
  {
    const int h = static_cast<int>(p.hist[static_cast<int64_t>(u) * kHistBins + (kHistBins - 1 - tid)]);
    int total;
    const int incl = block_inclusive_scan(h, sh.wsum, total);
    const int above = incl - h;
    if (above < kk && kk <= incl) {
      s_sel[0] = kHistBins - 1 - tid;
      s_sel[1] = above;
    }
  }
  __syncthreads();
  MAGE_TRACE_POINT(1);
  const int b_star = s_sel[0], above = s_sel[1];
  // ---- 2. candidates: the chunk's scores in bins >= b*, in position order
  const uint32_t lo = static_cast<uint32_t>(b_star) << kHistShift;   // smallest pattern of bin b*
  const int nv = run_valid<kLocalPer>(len);
  int nkeep = 0;
#pragma unroll
  for (int j = 0; j < kLocalPer; ++j) nkeep += (j < nv && v[j] >= lo);
  int kept;
  int o = block_inclusive_scan(nkeep, sh.wsum2, kept) - nkeep;
  {
    uint32_t* cb = p.cand_bits + static_cast<int64_t>(u) * p.cand_stride + start;
    int32_t* cp = p.cand_pos + static_cast<int64_t>(u) * p.cand_stride + start;
    const int run0 = start + tid * kLocalPer;
#pragma unroll
    for (int j = 0; j < kLocalPer; ++j)
      if (j < nv && v[j] >= lo) {
        st_dev(cb + o, v[j]);
        st_dev(cp + o, run0 + j);
        ++o;
      }
    if (tid == 0) st_dev(p.cand_count + static_cast<int64_t>(u) * p.nchunk + c, kept);
  }
  // ---- 3. count in; the row's last work-group selects (the counter is zeroed
  // by the next exact pass)
  const int nch = (n + kChunk - 1) / kChunk;
  if (!count_in(p.arrivals + u, static_cast<uint32_t>(nch), false, &s_sel[2])) return;
  MAGE_TRACE_POINT(2);
  const int32_t* cnt = p.cand_count + static_cast<int64_t>(u) * p.nchunk;
  const uint32_t* bits = p.cand_bits + static_cast<int64_t>(u) * p.cand_stride;
  const int32_t* pos = p.cand_pos + static_cast<int64_t>(u) * p.cand_stride;
  // The first spec_per slots of every chunk's slice, loaded in the same round
  // trip as the counts: when no chunk kept more, they hold every candidate
  // and the second round trip of loads through the offsets is skipped. A
  // chunk keeps about 1.1-1.2 kk / nch candidates, so the window is twice
  // that (at least 64 slots, at most 4096 slots in all: four per thread).
  // Slots past a chunk's count hold stale values and are dropped once the
  // counts are known.
  constexpr int kSpecLoads = 4, kSpecMinShift = 6;
  const bool spec = (nch << kSpecMinShift) <= kSpecLoads * kTopkThreads;
  int spec_shift = kSpecMinShift;   // window 2^spec_shift slots per chunk
  while ((nch << spec_shift) < 2 * kk && (nch << (spec_shift + 1)) <= kSpecLoads * kTopkThreads) ++spec_shift;
  const int spec_per = 1 << spec_shift;
  uint32_t sb[kSpecLoads];
  int32_t sp[kSpecLoads];
  if (spec) {
#pragma unroll
    for (int j = 0; j < kSpecLoads; ++j) {
      // clamped: the slots past the window repeat its last one
      const int i = min(tid + j * kTopkThreads, (nch << spec_shift) - 1);
      const int64_t sl = static_cast<int64_t>(i >> spec_shift) * kChunk + (i & (spec_per - 1));
      sb[j] = ld_dev(bits + sl);
      sp[j] = ld_dev(pos + sl);
    }
  }
  // s_off[c] = candidates before chunk c (thread t sums a contiguous run of chunks)
  bool over = false;
  {
    const int per = (nch + kTopkThreads - 1) / kTopkThreads;
    const int c0 = min(tid * per, nch), c1 = min(c0 + per, nch);
    int mine = 0;
    for (int cc = c0; cc < c1; ++cc) {
      const int k1 = ld_dev(cnt + cc);
      mine += k1;
      over |= k1 > spec_per;
    }
    int total;
    int oo = block_inclusive_scan(mine, sh.wsum, total) - mine;
    for (int cc = c0; cc < c1; ++cc) {
      s_off[cc] = oo;
      oo += ld_dev(cnt + cc);
    }
    if (tid == 0) s_off[nch] = total;
  }
  // (the barrier runs in every case: it also orders the s_off writes above
  // before the reads below)
  const bool any_over = __syncthreads_or(over) != 0;
  const bool spec_all = spec && !any_over;
  const int total = s_off[nch];
  // candidate i -> its index in the chunk slices (binary search over s_off)
  auto slot_of = [&](int i) -> int64_t {
    int a = 0, b = nch - 1;
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (s_off[mid] <= i) a = mid; else b = mid - 1;
    }
    return static_cast<int64_t>(a) * kChunk + (i - s_off[a]);
  };
  uint32_t T;
  int need;
  if (total <= kMax) {
    constexpr int kPer = kMax / kTopkThreads;
    if (spec_all) {
      // every candidate is among the speculative loads: place them in order
      // (entries past total are never read)
#pragma unroll
      for (int j = 0; j < kSpecLoads; ++j) {
        const int i = tid + j * kTopkThreads;
        const int cc = i >> spec_shift, o = i & (spec_per - 1);
        if (i < (nch << spec_shift) && o < s_off[cc + 1] - s_off[cc]) {
          s_data[s_off[cc] + o] = sb[j];
          s_data[kMax + s_off[cc] + o] = static_cast<uint32_t>(sp[j]);
        }
      }
    } else {
      uint32_t vb[kPer];
      int32_t vp[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = min(tid + j * kTopkThreads, total - 1);   // clamped; entries past total are never used
        const int64_t sl = slot_of(i);
        vb[j] = ld_dev(bits + sl);
        vp[j] = ld_dev(pos + sl);
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        s_data[tid + j * kTopkThreads] = vb[j];
        s_data[kMax + tid + j * kTopkThreads] = static_cast<uint32_t>(vp[j]);
      }
    }
    __syncthreads();
    uint32_t w[kPer], wpos[kPer];
    load_run<kPer>(s_data, w);
    load_run<kPer>(s_data + kMax, wpos);
    MAGE_TRACE_POINT(3);
    int eq_total;
    // the bin-b* candidates to LDS (s_data's first half is free again: every
    // thread holds its entries in registers); when they are as many as the
    // histogram says and few enough, one wave selects among them
    const int nw = run_valid<kPer>(total);
    int nb = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) nb += (j < nw && static_cast<int>(hist_bin(w[j])) == b_star);
    int mt;
    int ob = block_inclusive_scan(nb, sh.wsum, mt) - nb;
    if (b_star < kHistBins - 1 && mt == total - above && mt <= kWaveSelMax && above < kk && kk <= total) {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (j < nw && static_cast<int>(hist_bin(w[j])) == b_star) s_data[ob++] = w[j];
      __syncthreads();
      if (tid < kWave) {
        uint32_t t;
        int nd, eq;
        wave_select_in_bin(s_data, mt, kk - above, static_cast<uint32_t>(b_star) << kHistShift, sh.hist, t, nd, eq);
        if (tid == 0) {
          sh.res[0] = static_cast<int32_t>(t);
          sh.res[1] = nd;
          sh.res[2] = eq;
        }
      }
      __syncthreads();
      T = static_cast<uint32_t>(sh.res[0]);
      need = sh.res[1];
      eq_total = sh.res[2];
      __syncthreads();   // sh is reused by the compaction
    } else {
      radix_select_sampled<kPer>(w, total, kk, sh, s_data, T, need, eq_total);
    }
    MAGE_TRACE_POINT(4);
    ordered_compact_regs<kPer>(w, total, T, need, [&](int j) { return static_cast<int32_t>(wpos[j]); }, nullptr,
                               out, sh, eq_total, kk);
  } else if (total <= kOverflowPer * kTopkThreads) {
    // more candidates than the LDS holds: each thread's contiguous run of their
    // scores in registers, its loads all in flight at once; positions are
    // loaded for the kept entries only
    uint32_t w[kOverflowPer];
#pragma unroll
    for (int j = 0; j < kOverflowPer; ++j) w[j] = ld_dev(bits + slot_of(min(tid * kOverflowPer + j, total - 1)));
    int eq_total;
    radix_select_regs<kOverflowPer>(w, total, kk, sh, T, need, &eq_total);
    ordered_compact_regs<kOverflowPer>(
        w, total, T, need, [&](int j) { return ld_dev(pos + slot_of(tid * kOverflowPer + j)); }, nullptr, out, sh,
        eq_total, kk);
  } else {
    auto get = [&](int i) { return ld_dev(bits + slot_of(i)); };
    radix_select(get, total, kk, sh, T, need);
    ordered_compact(get, total, T, need, [&](int i) { return ld_dev(pos + slot_of(i)); }, nullptr, out, sh, kk);
  }
  for (int i = kk + tid; i < p.k; i += kTopkThreads) out[i] = -1;
  MAGE_TRACE_POINT(5);
}

}  // namespace mage
