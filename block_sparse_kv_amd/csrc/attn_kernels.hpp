// Attention kernels of the MAGE hot path on gfx950.
//
// One kernel template serves the step-1 exact pass (split over the prefix)
// and the later-step sparse pass (split over the gathered index list). Both
// follow the MAGE page ("MAGE: All-[MASK] Block Already Knows Where to Look
// in Block Diffusion LLM", atlas.scime.ai summary, "Approach"): exact
// attention at step 1, attention over the reused top-k rows afterwards.
//
// Work-group = 4 waves. Wave w owns query rows 32w..32w+31 of one KV head
// (row r = b * G + g), so the block's B tokens and the G query heads that
// share the KV head form one MFMA tile and every K/V row staged in LDS is used
// by all of them. K/V tiles of 64 rows stream global->LDS through a ring of
// kStages buffers (direct LDS loads). Per tile and wave:
//   S^T[key][row] = K Q^T       v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//                               B = Q held in registers)
//   online softmax on the rows  (exp2, scale * log2(e) folded in)
//   O^T[d][row] += V^T P^T      v_mfma_f32_32x32x16_bf16, twice: P is split
//                               into bf16 hi + lo (P - hi), so the product keeps
//                               ~16 mantissa bits of P; V^T comes straight from
//                               the row-major bf16 tile via transpose reads.
// K rows enter the A operand in the order pi(m) (bits 2 and 3 of m swapped):
// then accumulator registers 8s..8s+7 of a lane hold 8 consecutive keys, which
// is the B operand layout of the PV product, so P never leaves registers.
#pragma once

#include <type_traits>

#include "mage_common.hpp"
#include "tile_io.hpp"

namespace mage {

struct AttnParams {
  const uint16_t* q;        // bf16 [S][B][Hq][d]
  KvSource kv;
  const int32_t* idx;       // sparse pass: int32 [S][Hkv][idx_k]; null for the exact pass
  int32_t idx_k;
  float* o;                 // fp32 [S][B][Hq][d]
  float* lse;               // fp32 [S][B][Hq] or null
  float* part_o;            // partial O, MFMA accumulator order, per (unit, chunk)
  float* part_ml;           // partial (max, sum) per (unit, chunk, row)
  int32_t S, B, Hq, Hkv, G, R;
  int32_t chunk;            // keys (exact) or idx entries (sparse) per work-group
  int32_t nchunk;           // chunks per unit in the grid
  int32_t xcd_group;        // 1: keep the chunks of a unit on one XCD (grid padded to 8 units)
  float scale_log2;         // scale * log2(e)
  SeqLens lens;             // paged layout: N_s per sequence
};

struct MergeParams {
  const float* part_o;
  const float* part_ml;
  float* o;
  float* lse;               // nullable
  float* rowstat;           // per (unit, row): max + log2(sum), log2 units
  int32_t S, B, Hq, Hkv, G, R, nrb;
  int32_t chunk, nchunk;
  int32_t n_uniform;        // >= 0: entries per unit (prefix length or idx count); < 0: lens
  SeqLens lens;
};

constexpr int kMaxSparseChunk = 4096;   // idx entries per sparse work-group (LDS row table)
constexpr int kMaxChunkPages = 4096;    // page ids per exact-pass work-group (paged layout)

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// float4 offset of (slot, wave, d-block, register group, lane) in part_o
template <int D>
__device__ __forceinline__ int64_t part_o_index(int64_t slot, int w, int db, int i4, int lane) {
  return ((((slot * 4 + w) * (D / 32) + db) * 4 + i4) * kWave + lane);
}

// Write final O (and lse) of row 32w + (lane & 31) from an O^T accumulator.
template <int D>
__device__ __forceinline__ void store_rows(const AttnParams& p, int s, int h, int w, int lane,
                                           float m, float l, const f32x16 (&acc)[D / 32]) {
  const int n = lane & 31, hh = lane >> 5;
  const int r = 32 * w + n;
  if (r >= p.R) return;
  const int b = r / p.G, g = r - b * p.G, j = h * p.G + g;
  const int64_t row = (static_cast<int64_t>(s) * p.B + b) * p.Hq + j;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* orow = p.o + row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 v;
      v[0] = acc[db][4 * i4 + 0] * inv;
      v[1] = acc[db][4 * i4 + 1] * inv;
      v[2] = acc[db][4 * i4 + 2] * inv;
      v[3] = acc[db][4 * i4 + 3] * inv;
      *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i4 + 4 * hh) = v;
    }
  if (hh == 0 && p.lse != nullptr)
    p.lse[row] = l > 0.f ? (m + __log2f(l)) * kLn2 : -__builtin_inff();
}

// A row's softmax reference max is raised only when a tile's max exceeds it by
// more than 2^kLazyLog2 (log2 units): the running O and sum are then rescaled,
// otherwise probabilities up to 2^kLazyLog2 are accumulated as they are. The
// result is the same softmax; the rescale (64 multiplies per lane) becomes rare.
constexpr float kLazyLog2 = 8.f;

// 8 waves: wave w handles row block w % 4 and key half w / 4 (keys 32h..32h+31
// of every 64-key tile); the two waves of a row block merge at the end. Two
// waves per SIMD lets one wave's softmax run under the other's MFMAs.
constexpr int kAttnThreads = 512;

// Online-softmax update of one 32-key half tile for one wave, then PV.
//   k_base: LDS address of the half's first K row; kofs: this lane's K
//   fragment offsets; v_addr: LDS address of the V tile + half offset + this
//   lane's transpose-read offset; okm: validity bits of the half's 32 keys.
template <int D>
__device__ __forceinline__ void attend_half(uint32_t k_base, uint32_t v_addr,
                                            const uint32_t (&kofs)[D / 16],
                                            const bf16x8 (&qf)[D / 16], uint32_t okm,
                                            float scale_log2, float& m_run, float& l_run,
                                            f32x16 (&oacc)[D / 32], int lane) {
  constexpr int kNdb = D / 32, kNks = D / 16;
  const int hh = lane >> 5;
  f32x16 sacc;
  {
    bf16x8 kf[kNks];
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    k_frags<D, 0>(k_base, kofs, kf);
#pragma unroll
    for (int ks = 0; ks < kNks; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], sacc, 0, 0, 0);
  }
  // register i holds key 16(i/8) + 8hh + (i%8) of the half; raw q.k here
  float mt = -__builtin_inff();
  if (okm == ~0u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 16 * (i >> 3) + 8 * hh + (i & 7);
      const float x = ((okm >> key) & 1) ? sacc[i] : -__builtin_inff();
      sacc[i] = x;
      mt = fmaxf(mt, x);
    }
  }
  mt = wave_max_pair(mt) * scale_log2;  // scale > 0
  const bool grow = mt > m_run + kLazyLog2;
  if (__ballot(grow)) {
    const float m_new = grow ? mt : m_run;
    const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < kNdb; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    m_run = m_new;
  }
  const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pv = fast_exp2(__builtin_fmaf(sacc[i], scale_log2, neg_m));
    sacc[i] = pv;
    rs += pv;
  }
  l_run += wave_sum_pair(rs);
  // P = hi + lo, both bf16 (hi rounded to nearest, lo = P - hi rounded again)
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf16x8 phi[2], plo[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    u32x4 hw, lw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = sacc[8 * s2 + 2 * j], x1 = sacc[8 * s2 + 2 * j + 1];
      bf2 h;
      h.x = static_cast<__bf16>(x0);
      h.y = static_cast<__bf16>(x1);
      const uint32_t hb = __builtin_bit_cast(uint32_t, h);
      bf2 l;
      l.x = static_cast<__bf16>(x0 - __uint_as_float(hb << 16));
      l.y = static_cast<__bf16>(x1 - __uint_as_float(hb & 0xffff0000u));
      hw[j] = hb;
      lw[j] = __builtin_bit_cast(uint32_t, l);
    }
    phi[s2] = __builtin_bit_cast(bf16x8, hw);
    plo[s2] = __builtin_bit_cast(bf16x8, lw);
  }
  bf16x8 vf[kNdb][2];
  vt_frags_half<D>(v_addr, vf);
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], phi[s2], oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], plo[s2], oacc[db], 0, 0, 0);
    }
}

template <int D, bool kSparse, int kStages>
__global__ __launch_bounds__(kAttnThreads) void attn_chunk_kernel(AttnParams p) {
  using G = TileGeom<D, kAttnThreads>;
  constexpr int kNdb = D / 32, kNks = D / 16;
  constexpr int kStageBytes = 2 * G::kBytes;
  static_assert(kStages * kStageBytes >= 4 * kWave * (2 + 16 * kNdb) * 4, "pair-merge area");
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kStages * kStageBytes];
  // sparse: K/V row index of every entry of the chunk (-1 = skipped)
  // exact, paged: page ids of the chunk
  __shared__ int32_t s_tab[kSparse ? kMaxSparseChunk : kMaxChunkPages];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = w & 3, kh = w >> 2;
  const int hh = lane >> 5, n = lane & 31;
  const int units = p.S * p.Hkv;
  int u, c;
  if (p.xcd_group) {
    const int x = blockIdx.x & 7, jj = blockIdx.x >> 3;
    u = (jj / p.nchunk) * 8 + x;
    c = jj % p.nchunk;
  } else {
    u = blockIdx.x / p.nchunk;
    c = blockIdx.x % p.nchunk;
  }
  if (u >= units) return;
  MAGE_TRACE_POINT(0);
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  const int ns = seq_len_of(p.kv, p.lens, s);
  const int e0 = c * p.chunk;
  const int e1 = kSparse ? min(e0 + p.chunk, p.idx_k) : min(e0 + p.chunk, ns);
  if (e0 >= e1) return;  // exact pass: chunk past this sequence's end
  const int nrb = (p.R + 31) >> 5;
  const bool computes = rb < nrb;
  const bool paged = p.kv.page_table != nullptr;
  const int pshift = p.kv.page_shift, pmask = (1 << p.kv.page_shift) - 1;
  const int64_t seq_base = paged ? 0 : (static_cast<int64_t>(s) * p.Hkv + h) * p.kv.n_uniform;
  const int32_t* ptab = paged ? p.kv.page_table + static_cast<int64_t>(s) * p.kv.max_pages : nullptr;

  // ---- prologue: row tables in LDS -----------------------------------------
  const int cnt = e1 - e0;
  const int page0 = e0 >> pshift;
  if constexpr (kSparse) {
    for (int i = tid; i < cnt; i += kAttnThreads) {
      const int pos = p.idx[static_cast<int64_t>(u) * p.idx_k + e0 + i];
      int row = -1;
      if (pos >= 0 && pos < ns) {
        if (paged)
          row = ((ptab[pos >> pshift] * p.Hkv + h) << pshift) + (pos & pmask);
        else
          row = static_cast<int>(seq_base + pos);
      }
      s_tab[i] = row;
    }
  } else {
    if (paged) {
      const int np = ((e1 - 1) >> pshift) - page0 + 1;
      for (int i = tid; i < np; i += kAttnThreads) s_tab[i] = ptab[page0 + i];
    }
  }

  // Q rows of this row block as MFMA B operand fragments (d slice 16ks + 8hh .. +7)
  bf16x8 qf[kNks];
  {
    const int r = 32 * rb + n;
    if (computes && r < p.R) {
      const int b = r / p.G, g = r - b * p.G;
      const uint16_t* qrow = p.q + ((static_cast<int64_t>(s) * p.B + b) * p.Hq + h * p.G + g) * D;
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, load16(qrow + 16 * ks + 8 * hh));
    } else {
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  __syncthreads();  // row tables visible, Q loads complete (vmcnt drained)
  MAGE_TRACE_POINT(1);

  // element offset of the K/V row holding chunk entry e (always a readable row)
  auto row_of_entry = [&](int e) -> int64_t {
    if constexpr (kSparse) {
      const int row = s_tab[min(e, e1 - 1) - e0];
      return static_cast<int64_t>(row < 0 ? 0 : row) * D;
    } else {
      const int pos = min(e, e1 - 1);
      if (paged) {
        const int64_t page = s_tab[(pos >> pshift) - page0];
        return (((page * p.Hkv + h) << pshift) + (pos & pmask)) * D;
      }
      return (seq_base + pos) * D;
    }
  };
  auto valid_entry = [&](int e) -> bool {
    if constexpr (kSparse) return e < e1 && s_tab[e - e0] >= 0;
    else return e < e1;
  };

  f32x16 oacc[kNdb];
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;
  uint32_t kofs[kNks];
  k_frag_offsets<D>(swap_bits23(n), hh, kofs);
  const uint32_t ring_base = lds_addr(s_ring);
  const uint32_t k_half = kh * 32 * G::kRowBytes;
  const uint32_t v_half = G::kBytes + kh * 2048 + vt_lane_offset(lane);

  const int ntiles = (cnt + kTileKeys - 1) / kTileKeys;
  auto issue = [&](int tile) {
    uint8_t* st = s_ring + (tile % kStages) * kStageBytes;
    const int base = e0 + tile * kTileKeys;
    issue_tile<D, true, kAttnThreads>(st, st + G::kBytes, p.kv.k, p.kv.v,
                                      [&](int r) { return row_of_entry(base + r); }, w, lane);
  };
  // One barrier per tile: after it, every wave's loads of tile t have landed
  // and every wave has finished tile t-1, whose stage is refilled right away.
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < ntiles) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    wait_tiles<2 * G::kInstr, kStages - 1>(min(kStages - 2, ntiles - 1 - t));
    wg_barrier();
    if (t + kStages - 1 < ntiles) issue(t + kStages - 1);
    if (computes) {
      const uint32_t st = ring_base + (t % kStages) * kStageBytes;
      const uint64_t okm = __ballot(valid_entry(e0 + t * kTileKeys + lane));
      attend_half<D>(st + k_half, st + v_half, kofs, qf, static_cast<uint32_t>(okm >> (32 * kh)),
                     p.scale_log2, m_run, l_run, oacc, lane);
    }
    wait_lgkmcnt0();
  }
  __syncthreads();  // the ring is reused below
  MAGE_TRACE_POINT(2);

  // ---- merge the two key halves of each row block through LDS ---------------
  {
    float* xch = reinterpret_cast<float*>(s_ring) + rb * kWave * (2 + 16 * kNdb);
    if (computes && kh == 1) {
      xch[lane] = m_run;
      xch[kWave + lane] = l_run;
#pragma unroll
      for (int db = 0; db < kNdb; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(2 + 16 * db + i) * kWave + lane] = oacc[db][i];
    }
    __syncthreads();
    if (computes && kh == 0) {
      const float m1 = xch[lane], l1 = xch[kWave + lane];
      const float M = fmaxf(m_run, m1);
      const float Mu = M == -__builtin_inff() ? 0.f : M;
      const float a0 = fast_exp2(m_run - Mu), a1 = fast_exp2(m1 - Mu);
      l_run = l_run * a0 + l1 * a1;
      m_run = M;
#pragma unroll
      for (int db = 0; db < kNdb; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          oacc[db][i] = oacc[db][i] * a0 + xch[(2 + 16 * db + i) * kWave + lane] * a1;
    }
  }

  if (kSparse && p.nchunk == 1) {
    if (computes && kh == 0) store_rows<D>(p, s, h, rb, lane, m_run, l_run, oacc);
    return;
  }

  // partial result of this chunk
  const int64_t slot = static_cast<int64_t>(u) * p.nchunk + c;
  if (computes && kh == 0) {
#pragma unroll
    for (int db = 0; db < kNdb; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v{oacc[db][4 * i4], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]};
        *reinterpret_cast<f32x4*>(p.part_o + 4 * part_o_index<D>(slot, rb, db, i4, lane)) = v;
      }
    if (hh == 0) {
      p.part_ml[(slot * kMaxRows + 32 * rb + n) * 2 + 0] = m_run;
      p.part_ml[(slot * kMaxRows + 32 * rb + n) * 2 + 1] = l_run;
    }
  }
  MAGE_TRACE_POINT(3);
}

// Merge of split partials (exact pass: chunks of the prefix; sparse pass:
// chunks of the index list). One work-group per (unit, row block, d block);
// wave i4 handles accumulator registers 4*i4..4*i4+3. Also writes lse and, if
// rowstat is non-null, the per-row max + log2(sum) that the score sweep needs.
// A separate launch rather than an in-kernel last-arriver merge: on gfx950 the
// device-scope fence such a handoff needs writes back the XCD's whole L2.
template <int D>
__global__ __launch_bounds__(kThreads) void exact_merge_kernel(MergeParams p) {
  constexpr int kNdb = D / 32;
  constexpr int kBatch = 16;
  const int tid = threadIdx.x, lane = tid & 63, i4 = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  int bid = blockIdx.x;
  const int db = bid % kNdb;
  bid /= kNdb;
  const int w = bid % p.nrb;
  const int u = bid / p.nrb;
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  const int ns = p.n_uniform >= 0 ? p.n_uniform : p.lens.n[s];
  const int nch = (ns + p.chunk - 1) / p.chunk;
  const int r = 32 * w + n;
  const int64_t slot0 = static_cast<int64_t>(u) * p.nchunk;
  // one pass: a running max; each batch's loads are all in flight together
  float M = -__builtin_inff(), L = 0.f;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nch; c0 += kBatch) {
    float mb[kBatch], lb[kBatch];
    f32x4 vb[kBatch];
    // loads from clamped (always valid) slots, all issued before any use;
    // slots past the end get weight 0 afterwards
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t slot = slot0 + min(c0 + j, nch - 1);
      mb[j] = p.part_ml[(slot * kMaxRows + r) * 2];
      lb[j] = p.part_ml[(slot * kMaxRows + r) * 2 + 1];
      vb[j] = *reinterpret_cast<const f32x4*>(p.part_o + 4 * part_o_index<D>(slot, w, db, i4, lane));
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (c0 + j >= nch) mb[j] = -__builtin_inff();
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mb = fmaxf(Mb, mb[j]);
    if (Mb == -__builtin_inff()) continue;
    const float f = fast_exp2(M - Mb);  // M = -inf gives 0
    L *= f;
    acc[0] *= f;
    acc[1] *= f;
    acc[2] *= f;
    acc[3] *= f;
    M = Mb;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wc = fast_exp2(mb[j] - M);
      L += lb[j] * wc;
      acc[0] += wc * vb[j][0];
      acc[1] += wc * vb[j][1];
      acc[2] += wc * vb[j][2];
      acc[3] += wc * vb[j][3];
    }
  }
  if (r >= p.R) return;
  const int b = r / p.G, g = r - b * p.G, j = h * p.G + g;
  const int64_t row = (static_cast<int64_t>(s) * p.B + b) * p.Hq + j;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  f32x4 v{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  *reinterpret_cast<f32x4*>(p.o + row * D + 32 * db + 8 * i4 + 4 * hh) = v;
  if (db == 0 && i4 == 0 && hh == 0) {
    const float c2 = M + __log2f(L);
    if (p.lse != nullptr) p.lse[row] = c2 * kLn2;
    if (p.rowstat != nullptr) p.rowstat[static_cast<int64_t>(u) * kMaxRows + r] = c2;
  }
}

}  // namespace mage
