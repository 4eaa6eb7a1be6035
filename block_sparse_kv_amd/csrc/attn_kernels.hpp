// Attention kernels of the MAGE hot path on gfx950: the step-1 exact pass
// (split over the prefix), the later-step sparse pass (split over the reused
// index list) and the merge of split partials. Method: "MAGE: All-[MASK]
// Block Already Knows Where to Look in Block Diffusion LLM" (atlas.scime.ai
// summary, "Approach"): exact attention at step 1, attention over the reused
// top-k rows at every later step of the block.
//
// A wave owns 32 query rows of one KV head (row r = b * G + g), so the block's
// B tokens and the G query heads that share the KV head form one MFMA tile and
// every K/V row staged in LDS serves all of them. Per 32-key half tile:
//   S^T[key][row] = K Q^T       v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//                               B = Q held in registers)
//   online softmax on the rows  (exp2, scale * log2(e) folded in)
//   O^T[d][row] += V^T P^T      v_mfma_f32_32x32x16_bf16, twice: P is split
//                               into bf16 hi + lo (P - hi), so the product keeps
//                               ~16 mantissa bits of P; V^T comes straight from
//                               the row-major bf16 tile via transpose reads.
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
  int32_t gs, g0;           // query-head stride and sub-group offset (q_head); 0, 0 when unsplit
  int32_t chunk;            // keys (exact) or idx entries (sparse) per work-group
  int32_t nchunk;           // chunks per unit in the grid
  float scale_log2;         // scale * log2(e)
  SeqLens lens;             // paged layout: N_s per sequence
  ChunkMap map;             // exact pass: work-group -> (unit, chunk)
  const uint16_t* k_blk;    // sparse pass: bf16 [S][Hkv][B][d], the block's own rows, taken by
  const uint16_t* v_blk;    //   the last chunk of every unit; null = prefix rows only
  const int32_t* counts;    // sparse pass: per-unit entry counts (head-adaptive budgets); null =
                            //   idx_k entries each. Work-groups are then numbered densely per
  int32_t seq_slots;        //   sequence: seq_slots (unit, chunk) slots, units in head order
  uint32_t* arrivals;       // sparse pass, uniform chunks: one counter per (unit, row block), zero
                            //   between launches; non-null = the last work-group of a (unit, row
                            //   block) to finish merges its chunks (no merge launch)
  uint32_t* zero_hist;      // exact pass before a selection: the unit's score histogram [U][1024]
  uint32_t* zero_count;     //   and its top-k arrival counter [U] are zeroed by chunk 0 (or null)
};

struct MergeParams {
  const float* part_o;
  const float* part_ml;
  float* o;
  float* lse;               // nullable
  int32_t S, B, Hq, Hkv, G, R, nrb;
  int32_t gs, g0;           // query-head stride and sub-group offset (q_head)
  int32_t chunk, nchunk;
  int32_t n_uniform;        // >= 0: entries per unit (prefix length or idx count); < 0: lens
  SeqLens lens;
  const int32_t* counts;    // sparse pass with per-unit counts (capped at n_uniform): the chunks
  int32_t seq_slots;        //   of sequence s are slots s * seq_slots + (chunks of lower heads) + c
};

constexpr int kMaxChunkPages = 4096;    // page ids per exact-pass work-group (paged layout)

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// float4 offset of (slot, wave, d-block, register group, lane) in part_o
template <int D>
__device__ __forceinline__ int64_t part_o_index(int64_t slot, int w, int db, int i4, int lane) {
  return ((((slot * 4 + w) * (D / 32) + db) * 4 + i4) * kWave + lane);
}

// Partials handed from work-group to work-group inside one launch are stored
// and read with the agent-scope cache bit (sc1) and ordered by count_in.
constexpr int kScopeDevice = 16;   // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// One lane's share of the merge of a (unit, row block)'s split partials:
// accumulator registers 4*i4..4*i4+3 of d block db, for kTasks consecutive
// register groups i4 = i40 .. i40 + kTasks - 1, of row r, over chunks slot0 ..
// slot0 + nch - 1. Returns the max M (log2 units), the sum L and the
// unnormalised O (kTasks float4). Batches of kBatch chunks keep all their
// loads in flight together (loads from clamped, always valid slots; slots past
// the end get weight 0). kHandoff: the partials were stored in this launch by
// other work-groups and are read with device-scope loads.
template <int D, int kBatch, int kTasks, bool kHandoff>
__device__ __forceinline__ void merge_chunks(const float* part_o, const float* part_ml, int64_t slot0, int nch,
                                             int rb, int db, int i40, int lane, int r, float& M, float& L,
                                             f32x4 (&acc)[kTasks]) {
  constexpr int64_t kSlotF4 = 4 * (D / 32) * 4 * kWave;   // float4 per slot
  const float* o0 = part_o + 4 * part_o_index<D>(slot0, 0, 0, 0, 0);
  const float* ml0 = part_ml + slot0 * kMaxRows * 2;
  const __amdgpu_buffer_rsrc_t ro = raw_rsrc(o0, static_cast<uint32_t>(nch * kSlotF4 * 16));
  M = -__builtin_inff();
  L = 0.f;
#pragma unroll
  for (int q = 0; q < kTasks; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nch; c0 += kBatch) {
    float mb[kBatch], lb[kBatch];
    f32x4 vb[kBatch][kTasks];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = min(c0 + j, nch - 1);
      const int mf = (c * kMaxRows + r) * 2;
      if constexpr (kHandoff) {
        // (M, L) as two device-scope atomic loads: this compiler narrows a
        // buffer load whose result is only partly read (a b64 load split into
        // two floats comes out as one dword); each float4 of O is read whole
        mb[j] = __hip_atomic_load(ml0 + mf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lb[j] = __hip_atomic_load(ml0 + mf + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        mb[j] = ml0[mf];
        lb[j] = ml0[mf + 1];
      }
#pragma unroll
      for (int q = 0; q < kTasks; ++q) {
        const int of = static_cast<int>(part_o_index<D>(c, rb, db, i40 + q, lane));
        if constexpr (kHandoff)
          vb[j][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, of * 16, 0, kScopeDevice));
        else
          vb[j][q] = *reinterpret_cast<const f32x4*>(o0 + 4 * static_cast<int64_t>(of));
      }
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
#pragma unroll
    for (int q = 0; q < kTasks; ++q) {
      acc[q][0] *= f;
      acc[q][1] *= f;
      acc[q][2] *= f;
      acc[q][3] *= f;
    }
    M = Mb;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wc = fast_exp2(mb[j] - M);
      L += lb[j] * wc;
#pragma unroll
      for (int q = 0; q < kTasks; ++q) {
        acc[q][0] += wc * vb[j][q][0];
        acc[q][1] += wc * vb[j][q][1];
        acc[q][2] += wc * vb[j][q][2];
        acc[q][3] += wc * vb[j][q][3];
      }
    }
  }
}

// The merged (max, sum) of row r over the split chunks slot0 .. slot0 + nch - 1
// (log2 units): the (M, L) half of merge_chunks, same batches and order, so
// both give the same bits for the same kBatch.
template <int kBatch>
__device__ __forceinline__ void merge_row_stats(const float* part_ml, int64_t slot0, int nch, int r, float& M,
                                                float& L) {
  const float* ml0 = part_ml + slot0 * kMaxRows * 2;
  M = -__builtin_inff();
  L = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kBatch) {
    float mb[kBatch], lb[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int mf = (min(c0 + j, nch - 1) * kMaxRows + r) * 2;
      mb[j] = ml0[mf];
      lb[j] = ml0[mf + 1];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (c0 + j >= nch) mb[j] = -__builtin_inff();
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mb = fmaxf(Mb, mb[j]);
    if (Mb == -__builtin_inff()) continue;
    const float f = fast_exp2(M - Mb);
    L *= f;
    M = Mb;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wc = fast_exp2(mb[j] - M);
      L += lb[j] * wc;
    }
  }
}

// A row's softmax reference max is raised only when a tile's max exceeds it by
// more than 2^kLazyLog2 (log2 units): the running O and sum are then rescaled,
// otherwise probabilities up to 2^kLazyLog2 are accumulated as they are. The
// result is the same softmax; the rescale (64 multiplies per lane) becomes rare.
constexpr float kLazyLog2 = 8.f;

// Exact-pass work-group: 8 waves, two per SIMD.
constexpr int kAttnThreads = 512;

// One 32-key half tile of one wave, in three phases so that a loop can issue
// the QK product of the next tile before the softmax of the current one:
//   qk_half      S^T[key][row] = K Q^T (8 MFMAs at d = 128)
//   softmax_half online-softmax update, P = exp2(scale * S - m) split into
//                bf16 hi + lo (P - hi), both rounded to nearest
//   pv_half      O^T[d][row] += V^T hi^T + V^T lo^T
// Register i of the S accumulator holds key 16(i/8) + 8hh + (i%8) of the half
// (K rows enter in the order pi(m), bits 2 and 3 of m swapped), which is the B
// operand layout of the PV product, so P never leaves registers.
// l_part is the lane's share of its row's sum (the keys of its half); the two
// shares of a row are added once, after the last tile (rescales apply to both).
template <int D>
__device__ __forceinline__ f32x16 qk_half(uint32_t k_base, const uint32_t (&kofs)[D / 16],
                                          const bf16x8 (&qf)[D / 16]) {
  constexpr int kNks = D / 16;
  bf16x8 kf[kNks];
  f32x16 sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
  k_frags<D, 0>(k_base, kofs, kf);
#pragma unroll
  for (int ks = 0; ks < kNks; ++ks)
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], sacc, 0, 0, 0);
  return sacc;
}

// okm: validity bits of the half's 32 keys (only read when kMasked). No
// branch: the rescale of the running O by `alpha` is left to the caller
// (needed when __ballot(grow) is set), so the whole softmax is one scheduling
// region that the MFMAs of another tile can interleave with.
template <bool kMasked>
__device__ __forceinline__ void softmax_half(f32x16 sacc, uint32_t okm, float scale_log2, float& m_run,
                                             float& l_part, float& alpha, bool& grow, bf16x8 (&phi)[2],
                                             bf16x8 (&plo)[2], int lane) {
  const int hh = lane >> 5;
  float mt = -__builtin_inff();
  if constexpr (kMasked) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 16 * (i >> 3) + 8 * hh + (i & 7);
      sacc[i] = ((okm >> key) & 1) ? sacc[i] : -__builtin_inff();
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[i]);
  mt = wave_max_pair(mt) * scale_log2;  // scale > 0
  grow = mt > m_run + kLazyLog2;
  const float m_new = grow ? mt : m_run;
  alpha = grow ? fast_exp2(m_run - m_new) : 1.f;   // m_run = -inf gives 0
  l_part *= alpha;
  m_run = m_new;
  const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pv = fast_exp2(__builtin_fmaf(sacc[i], scale_log2, neg_m));
    sacc[i] = pv;
    rs += pv;
  }
  l_part += rs;
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    u32x4 hw, lw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = sacc[8 * s2 + 2 * j], x1 = sacc[8 * s2 + 2 * j + 1];
      bf2 h;
      h.x = static_cast<__bf16>(x0);
      h.y = static_cast<__bf16>(x1);
      uint32_t hb = __builtin_bit_cast(uint32_t, h);
      // hidden from the compiler, which otherwise converts x0 a second time to
      // form the first term's fp32 value instead of shifting the packed word
      asm volatile("" : "+v"(hb));
      bf2 l;
      l.x = static_cast<__bf16>(x0 - __uint_as_float(hb << 16));
      l.y = static_cast<__bf16>(x1 - __uint_as_float(hb & 0xffff0000u));
      hw[j] = hb;
      lw[j] = __builtin_bit_cast(uint32_t, l);
    }
    phi[s2] = __builtin_bit_cast(bf16x8, hw);
    plo[s2] = __builtin_bit_cast(bf16x8, lw);
  }
}

template <int D>
__device__ __forceinline__ void rescale_o(bool grow, float alpha, f32x16 (&oacc)[D / 32]) {
  if (__ballot(grow)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
  }
}

template <int D, int kVB = kTileKeys * 64>
__device__ __forceinline__ void pv_half(uint32_t v_addr, const bf16x8 (&phi)[2], const bf16x8 (&plo)[2],
                                        f32x16 (&oacc)[D / 32]) {
  constexpr int kNdb = D / 32;
  bf16x8 vf[kNdb][2];
  vt_frags_half<D, kVB>(v_addr, vf);
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], phi[s2], oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], plo[s2], oacc[db], 0, 0, 0);
    }
}

// The three phases back to back (loops that do not pipeline).
template <int D, int kVB = kTileKeys * 64>
__device__ __forceinline__ void attend_half(uint32_t k_base, uint32_t v_addr,
                                            const uint32_t (&kofs)[D / 16],
                                            const bf16x8 (&qf)[D / 16], uint32_t okm,
                                            float scale_log2, float& m_run, float& l_part,
                                            f32x16 (&oacc)[D / 32], int lane) {
  bf16x8 phi[2], plo[2];
  float alpha;
  bool grow;
  const f32x16 sacc = qk_half<D>(k_base, kofs, qf);
  if (okm == ~0u)
    softmax_half<false>(sacc, okm, scale_log2, m_run, l_part, alpha, grow, phi, plo, lane);
  else
    softmax_half<true>(sacc, okm, scale_log2, m_run, l_part, alpha, grow, phi, plo, lane);
  rescale_o<D>(grow, alpha, oacc);
  pv_half<D, kVB>(v_addr, phi, plo, oacc);
}

// Exact pass (step 1): one work-group per (unit, chunk of the prefix).
// 8 waves: wave w takes row block w % 4 and key half w / 4 (keys 32h..32h+31
// of every 64-key tile); the two waves of a row block merge at the end.
// K/V tiles stream global -> LDS through a ring of kStages stages with one
// barrier per tile. The loop is software-pipelined: in iteration t a wave
// issues the QK product of tile t+1 and then runs the softmax and PV of tile
// t, so the MFMAs of one tile run under the vector work of the other.
// kSplitIssue: the tile loads are issued by the four key-half-1 waves; else
// every wave issues its own slices (kept for measurements). kPagedForm: the
// kernel reads paged caches (the chunk's page list is staged in LDS).
template <int D, int kStages, bool kSplitIssue, bool kPagedForm>
__global__ __launch_bounds__(kAttnThreads) void exact_chunk_kernel(AttnParams p) {
  using G = TileGeom<D, kAttnThreads>;
  constexpr int kNdb = D / 32, kNks = D / 16;
  static_assert(kStages == 3 || kStages == 4, "K(t+1)..K(t+kStages) and V(t-1)..V(t+kStages-2) are resident or in flight");
  static_assert(2 * kStages * G::kBytes >= 4 * kWave * (2 + 16 * kNdb) * 4, "pair-merge area");
  // K ring (kStages tiles) followed by the V ring (kStages tiles)
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[2 * kStages * G::kBytes];
  __shared__ int32_t s_pages[kPagedForm ? kMaxChunkPages : 1];   // paged layout: page ids of the chunk

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = w & 3, kh = w >> 2;
  const int hh = lane >> 5, n = lane & 31;
  const int units = p.S * p.Hkv;
  int u, c;
  map_chunk(p.map, p.lens, p.S, p.Hkv, p.chunk, p.nchunk, blockIdx.x, u, c);
  if (u >= units) return;
  MAGE_TRACE_POINT(0);
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  const int ns = seq_len_of(p.kv, p.lens, s);
  const int e0 = c * p.chunk;
  const int e1 = min(e0 + p.chunk, ns);
  if (e0 >= e1) return;  // chunk past this sequence's end
  const int nrb = (p.R + 31) >> 5;
  const bool computes = rb < nrb;
  const bool paged = kPagedForm && p.kv.page_table != nullptr;
  const int pshift = p.kv.page_shift, pmask = (1 << p.kv.page_shift) - 1;
  const int64_t seq_base = paged ? 0 : (static_cast<int64_t>(s) * p.Hkv + h) * p.kv.n_uniform;
  const int32_t* ptab = paged ? p.kv.page_table + static_cast<int64_t>(s) * p.kv.max_pages : nullptr;
  const int cnt = e1 - e0;
  // the last tile of the chunk is read as the 64 rows ending at e1 when it is
  // partial (shifted back into the prefix), so the page list starts 64 rows
  // before the chunk
  const int page0 = max(e0 - kTileKeys, 0) >> pshift;
  if (paged) {
    const int np = ((e1 - 1) >> pshift) - page0 + 1;
    for (int i = tid; i < np; i += kAttnThreads) s_pages[i] = ptab[page0 + i];
  }
  if (c == 0 && p.zero_hist != nullptr) {
    // the selection that follows adds its score histogram into this row and
    // counts its top-k work-groups here
    for (int b = tid; b < 1024; b += kAttnThreads) p.zero_hist[static_cast<int64_t>(u) * 1024 + b] = 0u;
    if (tid == 0) p.zero_count[u] = 0u;
  }

  // Q rows of this row block as MFMA B operand fragments (d slice 16ks + 8hh .. +7)
  bf16x8 qf[kNks];
  {
    const int r = 32 * rb + n;
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
  __syncthreads();   // page table visible
  // Q fragments in registers before any tile load: the tile loads are asm the
  // compiler does not count, so it must see its own loads complete here
  wait_vmcnt<0>();
  MAGE_TRACE_POINT(1);
  MAGE_TRACE_CLK(1);

  // element offset of the K/V row of prefix position e (clamped into the chunk)
  auto row_of = [&](int e) __attribute__((always_inline)) -> int64_t {
    const int pos = min(e, e1 - 1);
    if (paged) {
      const int64_t page = s_pages[(pos >> pshift) - page0];
      return (((page * p.Hkv + h) << pshift) + (pos & pmask)) * D;
    }
    return (seq_base + pos) * D;
  };
  // A partial last tile is loaded as the 64 rows ending at e1 when e1 >= 64
  // (all of them rows of this sequence); its first 64 - (cnt mod 64) keys
  // belong to the previous tile and are masked. The same keys form the same
  // tiles in both layouts, so paged and contiguous results are bit-identical.
  // Prefixes shorter than 64 clamp the rows past e1 and mask them.
  const int last_t = (cnt - 1) / kTileKeys;
  const int tail = cnt - last_t * kTileKeys;            // keys in the last tile, 1..64
  const bool shift_last = tail < kTileKeys && e1 >= kTileKeys;
  auto tile_base = [&](int t) __attribute__((always_inline)) -> int {
    return (t == last_t && shift_last) ? e1 - kTileKeys : e0 + t * kTileKeys;
  };
  // validity bits of this wave's key half of tile t
  auto half_mask = [&](int t) __attribute__((always_inline)) -> uint32_t {
    if (t == last_t && tail < kTileKeys) {
      if (shift_last) {
        const int lo = kTileKeys - tail - 32 * kh;     // first valid key of the half
        return lo <= 0 ? ~0u : (lo >= 32 ? 0u : ~((1u << lo) - 1u));
      }
      const int nv = tail - 32 * kh;
      return nv >= 32 ? ~0u : (nv <= 0 ? 0u : ((1u << nv) - 1u));
    }
    return ~0u;
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
  const uint32_t v_lane = kh * 2048 + vt_lane_offset(lane);
  auto k_slot_m = [&](int m) __attribute__((always_inline)) -> uint32_t { return ring_base + m * G::kBytes; };   // m = tile mod kStages
  auto v_slot_m = [&](int m) __attribute__((always_inline)) -> uint32_t { return ring_base + (kStages + m) * G::kBytes; };
  auto k_slot = [&](int tile) __attribute__((always_inline)) -> uint32_t { return k_slot_m(tile % kStages); };
  auto v_slot = [&](int tile) __attribute__((always_inline)) -> uint32_t { return v_slot_m(tile % kStages); };

  const int ntiles = (cnt + kTileKeys - 1) / kTileKeys;
  // Full tiles: each DMA instruction covers 4 (K) or 16 (V) consecutive rows,
  // which are contiguous in memory (contiguous layout, or one page when pages
  // hold >= 16 rows). Its address is then a wave-uniform base (the slice's first
  // row) plus a per-lane byte offset fixed for the whole loop, so the loop
  // writes no VGPR that an in-flight load still reads. Other tiles take the
  // clamped per-lane path.
  constexpr int kKRowsPerInstr = kWave / G::kUnits;        // 4 at d = 128
  // Tile loads are issued by the four key-half-1 waves only: wave w (w >= 4)
  // issues the slices of waves w - 4 and w in two passes. Each SIMD holds one
  // wave of each key half, so while one issues the next tiles the other is
  // already in its MFMA region. The per-lane offsets of the slices of waves
  // w - 4 and w are equal for K and kInstr d blocks apart for V.
  // (kSplitIssue false: every wave issues its own slices)
  constexpr bool split_issue = kSplitIssue;
  const bool issuer = !split_issue || w >= 4;
  uint32_t koff[G::kInstr], voff[G::kInstr];
#pragma unroll
  for (int j = 0; j < G::kInstr; ++j) {
    const int slot = (w & 3) * G::kInstr + j;
    const int unit = slot * kWave + lane;
    const int r = unit / G::kUnits, uk = (unit % G::kUnits) ^ (r & (G::kUnits - 1));
    koff[j] = static_cast<uint32_t>(((r - slot * kKRowsPerInstr) * D + uk * 8) * 2);
    const int db = slot >> 2, rv = (lane >> 2);
    voff[j] = static_cast<uint32_t>((rv * D + 32 * db + 8 * (lane & 3)) * 2);
  }
  const bool fast_rows = !paged || pshift >= 4;
  // byte address of the K row of prefix position pos (wave-uniform pos)
  auto row_bytes = [&](int pos) __attribute__((always_inline)) -> int64_t {
    if (paged) {
      const int64_t page = __builtin_amdgcn_readfirstlane(s_pages[(pos >> pshift) - page0]);
      return ((((page * p.Hkv + h) << pshift) + (pos & pmask)) * D) * 2;
    }
    return ((seq_base + pos) * D) * 2;
  };
  // a shifted tile of a paged cache need not start on a 16-row page boundary
  auto fast_tile = [&](int tile) __attribute__((always_inline)) -> bool {
    const int base = tile_base(tile);
    return fast_rows && base + kTileKeys <= e1 && (!paged || (base & 15) == 0);
  };
  // All tile loads are asm DMA that the compiler does not track; completion is
  // accounted for with wait_tiles. K rows of tile tk and V rows of tile tv
  // (either may be -1: none) go to their ring slots.
  const char* kbytes = reinterpret_cast<const char*>(p.kv.k);
  const char* vbytes = reinterpret_cast<const char*>(p.kv.v);
  auto issue_slices = [&](int tk, int tv, int ws) __attribute__((always_inline)) {   // the slices of wave ws of the 8-wave layout
    const bool fk = tk >= 0 && fast_tile(tk), fv = tv >= 0 && fast_tile(tv);
    const int bk = tk >= 0 ? tile_base(tk) : 0, bv = tv >= 0 ? tile_base(tv) : 0;
    const uint32_t lk = tk >= 0 ? k_slot(tk) : 0u, lv = tv >= 0 ? v_slot(tv) : 0u;
    // slices ws and ws - 4 are 4 * kInstr slices apart: kInstr V d blocks of 32 values
    const uint32_t vadd = ws >= 4 ? static_cast<uint32_t>(G::kInstr * 32 * 2) : 0u;
    if (fk && fv) {
#pragma unroll
      for (int j = 0; j < G::kInstr; ++j) {
        const int slot = ws * G::kInstr + j;
        dma16x2<true>(kbytes + row_bytes(bk + slot * kKRowsPerInstr), koff[j], lk + slot * 1024,
                      vbytes + row_bytes(bv + ((slot & 3) << 4)), voff[j] + vadd, lv + slot * 1024);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < G::kInstr; ++j) {
      const int slot = ws * G::kInstr + j;
      if (fk) {
        dma16(kbytes + row_bytes(bk + slot * kKRowsPerInstr), koff[j], lk + slot * 1024);
      } else if (tk >= 0) {
        const int unit = slot * kWave + lane;
        const int r = unit / G::kUnits, uk = (unit % G::kUnits) ^ (r & (G::kUnits - 1));
        dma16_sync(p.kv.k + row_of(bk + r) + uk * 8, lk + slot * 1024);
      }
      if (fv) {
        dma16<true>(vbytes + row_bytes(bv + ((slot & 3) << 4)), voff[j] + vadd, lv + slot * 1024);
      } else if (tv >= 0) {
        const int db = slot >> 2, rv = ((slot & 3) << 4) + (lane >> 2);
        dma16_sync<true>(p.kv.v + row_of(bv + rv) + 32 * db + 8 * (lane & 3), lv + slot * 1024);
      }
    }
  };
  auto issue = [&](int tk, int tv) __attribute__((always_inline)) {
    if constexpr (split_issue) {
      if (!issuer) return;
#pragma unroll 1
      for (int pass = 0; pass < 2; ++pass) issue_slices(tk, tv, __builtin_amdgcn_readfirstlane((w & 3) + 4 * pass));
    } else {
      issue_slices(tk, tv, w);
    }
  };
  // Steady state (contiguous rows, full tiles before the last): a tile's K
  // (V) rows are one 16 KiB run at k_run (v_run) + tile * kBytes, so each of
  // an issuing wave's slices is that base plus a per-lane offset and an LDS
  // offset fixed for the whole loop. A wave issues about one instruction
  // every four cycles, and the general path's per-slice address and branch
  // work (about 150 instructions a tile) kept the issuing waves out of their
  // MFMA region for most of a tile.
  constexpr int kSlices = (split_issue ? 2 : 1) * G::kInstr;   // slices per issuing wave and tile
  uint32_t k_lane[kSlices], v_lane_dma[kSlices], lds_slice[kSlices];
#pragma unroll
  for (int i = 0; i < kSlices; ++i) {
    const int pass = i / G::kInstr, j = i % G::kInstr;
    const int ws = split_issue ? (w & 3) + 4 * pass : w;
    const int slot = ws * G::kInstr + j;
    k_lane[i] = koff[j] + static_cast<uint32_t>(slot * kKRowsPerInstr * G::kRowBytes);
    v_lane_dma[i] = voff[j] + (ws >= 4 ? static_cast<uint32_t>(G::kInstr * 32 * 2) : 0u) +
                    static_cast<uint32_t>(((slot & 3) << 4) * G::kRowBytes);
    lds_slice[i] = static_cast<uint32_t>(slot * 1024);
  }
  const char* k_run = kbytes + (seq_base + e0) * G::kRowBytes;
  const char* v_run = vbytes + (seq_base + e0) * G::kRowBytes;
  // K rows of tile tk into LDS lk, V rows of tile tk - 2 into lv; tk < last_t
  auto issue_steady = [&](int tk, uint32_t lk, uint32_t lv) __attribute__((always_inline)) {
    if (!issuer) return;
    const char* kt = k_run + static_cast<int64_t>(tk) * G::kBytes;
    const char* vt = v_run + static_cast<int64_t>(tk - 2) * G::kBytes;
#pragma unroll
    for (int i = 0; i < kSlices; ++i)
      dma16x2<true>(kt, k_lane[i], lk + lds_slice[i], vt, v_lane_dma[i], lv + lds_slice[i]);
  };
  // Steady state of the paged form (pages of >= 16 rows and a chunk that
  // starts on a 64-row boundary, so each slice's rows lie in one page): the
  // page ids of an issuing wave's slices are read from the chunk's page list
  // in one batch, behind one wait, and each slice's address is then scalar
  // arithmetic. The general path waits for one page-list read per slice, each
  // queued behind the other waves' fragment reads.
  auto issue_steady_paged = [&](int tk, uint32_t lk, uint32_t lv) __attribute__((always_inline)) {
    if (!issuer) return;
    const int bk = e0 + tk * kTileKeys, bv = bk - 2 * kTileKeys;   // rows of tiles tk and tk - 2
    int pk[kSlices], pv[kSlices];
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
      const int ws = split_issue ? (w & 3) + 4 * (i / G::kInstr) : w;
      const int slot = ws * G::kInstr + i % G::kInstr;
      pk[i] = s_pages[((bk + slot * kKRowsPerInstr) >> pshift) - page0];
      pv[i] = s_pages[((bv + ((slot & 3) << 4)) >> pshift) - page0];
    }
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
      const int ws = split_issue ? (w & 3) + 4 * (i / G::kInstr) : w;
      const int j = i % G::kInstr, slot = ws * G::kInstr + j;
      const uint32_t vadd = ws >= 4 ? static_cast<uint32_t>(G::kInstr * 32 * 2) : 0u;
      const int rk = bk + slot * kKRowsPerInstr, rv = bv + ((slot & 3) << 4);
      const int64_t pgk = __builtin_amdgcn_readfirstlane(pk[i]), pgv = __builtin_amdgcn_readfirstlane(pv[i]);
      const int64_t ka = (((pgk * p.Hkv + h) << pshift) + (rk & pmask)) * G::kRowBytes;
      const int64_t va = (((pgv * p.Hkv + h) << pshift) + (rv & pmask)) * G::kRowBytes;
      dma16x2<true>(kbytes + ka, koff[j], lk + slot * 1024, vbytes + va, voff[j] + vadd, lv + slot * 1024);
    }
  };
  // Load group g = what iteration g reads: K rows of tile g+1 and V rows of
  // tile g-1. Iteration t waits for group t, with the kStages - 2 groups after
  // it still allowed in flight, and issues group t + kStages - 1 into the
  // slots of K(t) and V(t-2), which no wave reads any more once every wave
  // has passed the barrier of iteration t (K(t) was read by the QK product and
  // V(t-2) by the PV product of iteration t-1).
  constexpr int kPerTile = (split_issue ? 2 : 1) * G::kInstr;   // issuers: two slices per tile
  auto group_k = [&](int g) __attribute__((always_inline)) { return g + 1 < ntiles ? g + 1 : -1; };
  auto group_v = [&](int g) __attribute__((always_inline)) { return g >= 1 && g - 1 < ntiles ? g - 1 : -1; };
  auto group_tiles = [&](int g) __attribute__((always_inline)) { return (group_k(g) >= 0) + (group_v(g) >= 0); };
  auto wait_group = [&](int g) __attribute__((always_inline)) {
    // the others have none in flight
    int pending = 0;
#pragma unroll
    for (int j = 1; j <= kStages - 2; ++j) pending += group_tiles(g + j);
    wait_tiles<kPerTile, 2 * (kStages - 2) + 1>(pending);
    wg_barrier();
  };

  issue(0, -1);
#pragma unroll
  for (int g = 0; g < kStages - 1; ++g) issue(group_k(g), group_v(g));
  {
    int pending = 0;   // everything but K(0)
#pragma unroll
    for (int g = 0; g < kStages - 1; ++g) pending += group_tiles(g);
    wait_tiles<kPerTile, 2 * (kStages - 1) + 1>(pending);
  }
  wg_barrier();
  f32x16 s_cur;
  if (computes) s_cur = qk_half<D>(k_slot(0) + k_half, kofs, qf);

  // Iteration t: the PV product of tile t-1 (probabilities from iteration
  // t-1), the QK product of tile t+1 and the softmax of tile t are
  // independent, so the fragment reads are issued first and the MFMAs of
  // both products are interleaved with the softmax's vector instructions.
  // The running O takes the rescale of tile t's softmax after PV of tile t-1,
  // whose probabilities were taken against the previous max. The last
  // iteration's QK product re-reads tile t (result unused), which keeps the
  // region free of branches.
  bf16x8 ph[2], pl[2];
  const bool partial = cnt % kTileKeys != 0;
  [[maybe_unused]] uint64_t trace_acc[4] = {0, 0, 0, 0};
  // t = 0: softmax of tile 0 and QK of tile 1
  auto first = [&](auto masked) __attribute__((always_inline)) {
    wait_group(0);
    issue(group_k(kStages - 1), group_v(kStages - 1));
    if (computes) {
      float alpha;
      bool grow;
      softmax_half<decltype(masked)::value>(s_cur, half_mask(0), p.scale_log2, m_run, l_run, alpha, grow,
                                            ph, pl, lane);
      if (ntiles > 1) s_cur = qk_half<D>(k_slot(1) + k_half, kofs, qf);
    }
  };
  // phase: t mod kStages as a compile-time constant (then every ring slot of
  // the iteration is a constant and the LDS addresses are loop-invariant
  // bases plus immediate offsets), or -1
  auto middle = [&](int t, auto masked, auto steady, auto phase) __attribute__((always_inline)) {
    constexpr int kPh = decltype(phase)::value;
    [[maybe_unused]] const uint64_t tr0 = MAGE_TRACE_NOW();
    wait_group(t);
    [[maybe_unused]] const uint64_t tr1 = MAGE_TRACE_NOW();
    if constexpr (decltype(steady)::value) {
      const int m0 = kPh >= 0 ? kPh : t % kStages;   // K tile t + kStages; V tile t + kStages - 2
      const uint32_t lk = k_slot_m(m0), lv = v_slot_m((m0 + kStages - 2) % kStages);
      if (paged)
        issue_steady_paged(t + kStages, lk, lv);
      else
        issue_steady(t + kStages, lk, lv);
    } else {
      issue(group_k(t + kStages - 1), group_v(t + kStages - 1));
    }
    if (computes) {
      const uint32_t okm = half_mask(t);
      const int mk = kPh >= 0 ? (kPh + 1) % kStages : (t + 1 < ntiles ? t + 1 : t) % kStages;
      const int mv = kPh >= 0 ? (kPh + kStages - 1) % kStages : (t - 1) % kStages;
      const uint32_t kb = k_slot_m(mk) + k_half;
      [[maybe_unused]] const uint64_t tr2 = MAGE_TRACE_NOW();
      bf16x8 vf[kNdb][2], kf[kNks];
      // the V fragments are read at this base plus immediate offsets; with a
      // run-time slot the base is hidden from loop strength reduction, which
      // would otherwise keep one address register per fragment and update all
      // of them every iteration
      uint32_t va = v_slot_m(mv) + v_lane;
      if constexpr (kPh < 0) asm volatile("" : "+v"(va));
      vt_frags_half_lds<D>(va, vf);
      k_frags_lds<D>(kb, kofs, kf);
#pragma unroll
      for (int db = 0; db < kNdb; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], ph[s2], oacc[db], 0, 0, 0);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], pl[s2], oacc[db], 0, 0, 0);
        }
      f32x16 s_nxt;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_nxt[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks)
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s_nxt, 0, 0, 0);
      bf16x8 phn[2], pln[2];
      float alpha;
      bool grow;
      softmax_half<decltype(masked)::value>(s_cur, okm, p.scale_log2, m_run, l_run, alpha, grow, phn, pln,
                                            lane);
      // order: half the V reads, the start of the softmax, the other V reads,
      // PV MFMAs of the first d blocks, the K reads, the remaining MFMAs, each
      // MFMA followed by five vector instructions (at most 16 LDS reads are
      // ever outstanding, so every wait can name the read it needs)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kNdb, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kNdb, 0);
#pragma unroll
      for (int i = 0; i < 2 * kNdb; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kNks, 0);
#pragma unroll
      for (int i = 0; i < 2 * kNdb + kNks; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      // the softmax results are complete here, ahead of the rescale branch
      // (otherwise the compiler sinks their computation past it, out of the
      // region shared with the MFMAs)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) asm volatile("" : "+v"(phn[s2]), "+v"(pln[s2]));
      asm volatile("" : "+v"(l_run));
      [[maybe_unused]] const uint64_t tr3 = MAGE_TRACE_NOW();
      rescale_o<D>(grow, alpha, oacc);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        ph[s2] = phn[s2];
        pl[s2] = pln[s2];
      }
      s_cur = s_nxt;
      [[maybe_unused]] const uint64_t tr4 = MAGE_TRACE_NOW();
      trace_acc[0] += tr1 - tr0;
      trace_acc[1] += tr2 - tr1;
      trace_acc[2] += tr3 - tr2;
      trace_acc[3] += tr4 - tr3;
    }
  };
  if (ntiles == 1 && partial)
    first(std::true_type{});
  else
    first(std::false_type{});
  using dyn = std::integral_constant<int, -1>;
  int t = 1;
  // iterations whose load group (K rows of tile t + kStages, V rows of tile
  // t + kStages - 2) holds full tiles before the last take the steady issue,
  // unrolled by kStages from t = 1 so that each copy knows t mod kStages
  // (split issue: contiguous rows; every wave issuing: the paged form)
  const bool steady_ok = paged ? pshift >= 4 && (e0 & (kTileKeys - 1)) == 0 : split_issue;
  if (steady_ok) {
    for (; t + 2 * kStages - 1 < last_t; t += kStages) {
      middle(t, std::false_type{}, std::true_type{}, std::integral_constant<int, 1 % kStages>{});
      middle(t + 1, std::false_type{}, std::true_type{}, std::integral_constant<int, 2 % kStages>{});
      middle(t + 2, std::false_type{}, std::true_type{}, std::integral_constant<int, 3 % kStages>{});
      if constexpr (kStages == 4) middle(t + 3, std::false_type{}, std::true_type{}, std::integral_constant<int, 0>{});
    }
    for (; t + kStages < last_t; ++t) middle(t, std::false_type{}, std::true_type{}, dyn{});
  }
  for (; t + 1 < ntiles; ++t) middle(t, std::false_type{}, std::false_type{}, dyn{});
  if (ntiles > 1) {
    if (partial)
      middle(ntiles - 1, std::true_type{}, std::false_type{}, dyn{});
    else
      middle(ntiles - 1, std::false_type{}, std::false_type{}, dyn{});
  }
  // t = ntiles: PV of the last tile
  wait_group(ntiles);
  if (computes) {
    bf16x8 vf[kNdb][2];
    vt_frags_half_lds<D>(v_slot(ntiles - 1) + v_lane, vf);
#pragma unroll
    for (int db = 0; db < kNdb; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], ph[s2], oacc[db], 0, 0, 0);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][s2], pl[s2], oacc[db], 0, 0, 0);
      }
  }
  l_run = wave_sum_pair(l_run);
  MAGE_TRACE_ADD(4, trace_acc[0]);
  MAGE_TRACE_ADD(5, trace_acc[1]);
  MAGE_TRACE_ADD(6, trace_acc[2]);
  MAGE_TRACE_ADD(7, trace_acc[3]);
  __syncthreads();  // the ring is reused below
  MAGE_TRACE_POINT(2);
  MAGE_TRACE_CLK(2);

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

// ---------------------------------------------------------------------------
// Sparse step (later denoising steps over the reused index set).
//
// Work-group = 4 waves = one (unit, 32-row block, chunk of the index list).
// Wave w takes the contiguous quarter [w*kpw, (w+1)*kpw) of the chunk and
// streams it in 32-key tiles through its own LDS ring: the wave issues its
// own direct LDS loads and waits on its own vmcnt, so the key loop has no
// barrier. The four waves' (max, sum, O) are merged through LDS at the end;
// with one chunk per unit the result is final, else it is a partial in the
// layout exact_merge_kernel reads. Work-groups of the same (unit, chunk) are
// numbered 8 apart so that, with the round-robin placement of work-groups
// on the 8 XCDs, they share one L2 for the rows they all gather.
constexpr int kSparseWaves = 4;
constexpr int kHandoffBatch = 8;   // chunks whose partials the last arriver loads at once
constexpr int kSparseThreads = kSparseWaves * kWave;
constexpr int kSparseTileKeys = 32;
constexpr int kSparseMaxKpw = 1024;     // index entries per wave (LDS row table)

template <int D>
struct SparseTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kUnits = D / 8;                              // 16-byte units per row
  static constexpr int kKBytes = kSparseTileKeys * kRowBytes;      // K part of a stage
  static constexpr int kStageBytes = 2 * kKBytes;                  // K + V
  static constexpr int kInstr = kKBytes / (kWave * 16);            // DMA instructions per part
  static constexpr int kVBlock = kSparseTileKeys * 64;             // one 32-value d block of V
};

// DMA of one 32-key tile by one wave. K: row-major, unit u of row r at unit
// u ^ (r mod kUnits). V: [d/32][32 rows][32 values]. row(r) = element offset
// of tile row r (always a readable row).
template <int D, class RowOff>
__device__ __forceinline__ void issue_sparse_tile(uint8_t* k_lds, uint8_t* v_lds, const uint16_t* kbase,
                                                  const uint16_t* vbase, RowOff row, int lane) {
  using T = SparseTile<D>;
#pragma unroll
  for (int j = 0; j < T::kInstr; ++j) {
    const int unit = j * kWave + lane;
    const int r = unit / T::kUnits, phys = unit % T::kUnits;
    const int uk = phys ^ (r & (T::kUnits - 1));
    __builtin_amdgcn_global_load_lds(kbase + row(r) + uk * 8, k_lds + j * 1024, 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < T::kInstr; ++j) {
    const int db = j >> 1, r = ((j & 1) << 4) + (lane >> 2);
    __builtin_amdgcn_global_load_lds(vbase + row(r) + 32 * db + 8 * (lane & 3), v_lds + j * 1024, 16, 0, 0);
  }
}

template <int D, int kStages>
__global__ __launch_bounds__(kSparseThreads) void sparse_attn_kernel(AttnParams p) {
  using T = SparseTile<D>;
  constexpr int kNdb = D / 32, kNks = D / 16;
  constexpr int kWaveRing = kStages * T::kStageBytes;
  constexpr int kXchFloats = kWave * (2 + 16 * kNdb);
  static_assert(kWaveRing >= kXchFloats * 4, "merge area fits in a wave's ring");
  static_assert(2 * T::kInstr * (kStages - 1) < 64, "vmcnt is 6 bits");
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kSparseWaves * kWaveRing];
  __shared__ int32_t s_tab[kSparseWaves][kSparseMaxKpw];

  MAGE_TRACE_POINT(6);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, n = lane & 31;
  const int units = p.S * p.Hkv;
  const int nrb = (p.R + 31) >> 5;
  // blockIdx -> (g = unit * nchunk + chunk, row block): same g, ids 8 apart
  const int x = blockIdx.x & 7, jj = blockIdx.x >> 3;
  const int rb = jj % nrb;
  const int g = (jj / nrb) * 8 + x;
  int u, c, n_idx = p.idx_k;   // (unit, chunk) and the unit's index entries
  int64_t slot;                // partial slot
  bool direct = p.nchunk == 1; // the unit's only chunk: O and lse written here, no merge
  if (p.counts == nullptr) {
    if (g >= units * p.nchunk) return;
    u = g / p.nchunk;
    c = g - u * p.nchunk;
    slot = static_cast<int64_t>(u) * p.nchunk + c;
  } else {
    // per-unit counts: g = sequence * seq_slots + the chunk's place among the
    // sequence's chunks, heads in order
    const int sq = g / p.seq_slots;
    if (sq >= p.S) return;
    int lc = g - sq * p.seq_slots, head = 0;
    for (; head < p.Hkv; ++head) {
      const int nc = (max(0, min(p.counts[sq * p.Hkv + head], p.idx_k)) + p.chunk - 1) / p.chunk;
      if (lc < nc) {
        direct = nc == 1;
        break;
      }
      lc -= nc;
    }
    if (head == p.Hkv) return;   // past the sequence's last chunk
    u = sq * p.Hkv + head;
    c = lc;
    slot = g;
    n_idx = max(0, min(p.counts[u], p.idx_k));
  }
  MAGE_TRACE_POINT(0);
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  const int ns = seq_len_of(p.kv, p.lens, s);
  const int kpw = p.chunk / kSparseWaves;
  const int e0 = c * p.chunk + w * kpw;                 // this wave's entries [e0, e1)
  const int e1 = min(e0 + kpw, n_idx);
  const int cnt = max(0, e1 - e0);
  // the last chunk of a unit also takes the block's own rows: at most one more
  // 32-row tile per wave, rows [b0, b0 + nb) of this unit's B
  int b0 = 0, nb = 0;
  if (p.k_blk != nullptr && c == p.nchunk - 1) {
    const int bpw = (p.B + kSparseWaves - 1) / kSparseWaves;   // <= kSparseTileKeys (B <= 128)
    b0 = w * bpw;
    nb = max(0, min(b0 + bpw, p.B) - b0);
  }
  const bool paged = p.kv.page_table != nullptr;
  const int pshift = p.kv.page_shift, pmask = (1 << p.kv.page_shift) - 1;
  const int64_t seq_base = paged ? 0 : (static_cast<int64_t>(s) * p.Hkv + h) * p.kv.n_uniform;
  const int32_t* ptab = paged ? p.kv.page_table + static_cast<int64_t>(s) * p.kv.max_pages : nullptr;

  // Q fragments of this row block (MFMA B operand; d slice 16ks + 8hh .. +7)
  bf16x8 qf[kNks];
  {
    const int r = 32 * rb + n;
    if (r < p.R) {
      const int b = r / p.G, gg = r - b * p.G;
      const uint16_t* qrow = p.q + ((static_cast<int64_t>(s) * p.B + b) * p.Hq + q_head(h, gg, p.G, p.gs, p.g0)) * D;
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, load16(qrow + 16 * ks + 8 * hh));
    } else {
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  // row read for a skipped entry: position 0 of this (sequence, KV head), which
  // always holds finite data (a pool row outside every sequence may not)
  const int fallback_row = paged ? ((ptab[0] * p.Hkv + h) << pshift) : static_cast<int>(seq_base);
  // this wave's row table (wave-private LDS; -1 = entry skipped). Four entries
  // per lane and round: all index loads, then all page-table loads, are in
  // flight together (loads from clamped, always valid addresses).
  int32_t* tab = s_tab[w];
  const int32_t* idx_w = p.idx + static_cast<int64_t>(u) * p.idx_k + e0;
  for (int i0 = 0; i0 < cnt; i0 += 4 * kWave) {
    int pos[4], page[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pos[j] = idx_w[min(i0 + j * kWave + lane, cnt - 1)];
    if (paged) {
#pragma unroll
      for (int j = 0; j < 4; ++j) page[j] = ptab[min(max(pos[j], 0), ns - 1) >> pshift];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kWave + lane;
      const int ps = pos[j];
      int row = -1;
      if (ps >= 0 && ps < ns)
        row = paged ? ((page[j] * p.Hkv + h) << pshift) + (ps & pmask) : static_cast<int>(seq_base + ps);
      if (i < cnt) tab[i] = row;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // row table written and Q fragments in registers
  __builtin_amdgcn_wave_barrier();
  MAGE_TRACE_POINT(1);

  uint8_t* ring = s_ring + w * kWaveRing;
  const uint32_t ring_base = lds_addr(ring);
  const int ntp = (cnt + kSparseTileKeys - 1) / kSparseTileKeys;   // index-entry tiles
  const int ntiles = ntp + (nb > 0 ? 1 : 0);
  auto issue = [&](int t) {
    uint8_t* st = ring + (t % kStages) * T::kStageBytes;
    if (t < ntp) {
      const int base = t * kSparseTileKeys;
      issue_sparse_tile<D>(st, st + T::kKBytes, p.kv.k, p.kv.v,
                           [&](int r) {
                             const int row = tab[min(base + r, cnt - 1)];
                             return static_cast<int64_t>(row < 0 ? fallback_row : row) * D;
                           },
                           lane);
    } else {
      const int64_t row0 = static_cast<int64_t>(u) * p.B + b0;
      issue_sparse_tile<D>(st, st + T::kKBytes, p.k_blk, p.v_blk,
                           [&](int r) { return (row0 + min(r, nb - 1)) * D; }, lane);
    }
  };
  f32x16 oacc[kNdb];
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;
  uint32_t kofs[kNks];
  k_frag_offsets<D>(swap_bits23(n), hh, kofs);
  const uint32_t v_lane = T::kKBytes + vt_lane_offset(lane);
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < ntiles) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    if (t + kStages - 1 < ntiles) {
      issue(t + kStages - 1);   // refills the stage of tile t-1, whose reads are complete
      wait_tiles<2 * T::kInstr, kStages>(kStages - 1);
    } else {
      wait_tiles<2 * T::kInstr, kStages>(min(kStages - 1, ntiles - 1 - t));
    }
    if (t == 0) MAGE_TRACE_POINT(2);
    const int e = t * kSparseTileKeys + n;
    const bool ok = t < ntp ? e < cnt && tab[min(e, cnt - 1)] >= 0 : n < nb;
    const uint32_t okm = static_cast<uint32_t>(__ballot(ok));
    const uint32_t st = ring_base + (t % kStages) * T::kStageBytes;
    attend_half<D, T::kVBlock>(st, st + v_lane, kofs, qf, okm, p.scale_log2, m_run, l_run, oacc, lane);
  }

  l_run = wave_sum_pair(l_run);
  MAGE_TRACE_POINT(3);
  // ---- merge the four waves through LDS ---------------------------------------
  float* xch = reinterpret_cast<float*>(ring);   // this wave's ring is free now
  xch[lane] = m_run;
  xch[kWave + lane] = l_run;
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) xch[(2 + 16 * db + i) * kWave + lane] = oacc[db][i];
  __syncthreads();
  MAGE_TRACE_POINT(4);
  // split chunks with arrival counters: this work-group stores its partial at
  // device scope and counts itself in; the last of the (unit, row block) merges
  const bool handoff = p.arrivals != nullptr && !direct;
  if (w >= kNdb && !handoff) return;
  const int r = 32 * rb + n;
  if (w < kNdb) {
    const int db = w;   // this wave merges d block db of all four waves
    float mj[kSparseWaves], M = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kSparseWaves; ++j) {
      mj[j] = reinterpret_cast<const float*>(s_ring + j * kWaveRing)[lane];
      M = fmaxf(M, mj[j]);
    }
    const float Mu = M == -__builtin_inff() ? 0.f : M;
    float L = 0.f;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < kSparseWaves; ++j) {
      const float* xj = reinterpret_cast<const float*>(s_ring + j * kWaveRing);
      const float a = fast_exp2(mj[j] - Mu);
      L += xj[kWave + lane] * a;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += xj[(2 + 16 * db + i) * kWave + lane] * a;
    }
    if (direct) {
      if (r >= p.R) return;
      const int b = r / p.G, gg = r - b * p.G, j = q_head(h, gg, p.G, p.gs, p.g0);
      const int64_t row = (static_cast<int64_t>(s) * p.B + b) * p.Hq + j;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* orow = p.o + row * D + 32 * db + 4 * hh;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(orow + 8 * i4) =
            f32x4{acc[4 * i4] * inv, acc[4 * i4 + 1] * inv, acc[4 * i4 + 2] * inv, acc[4 * i4 + 3] * inv};
      if (db == 0 && hh == 0 && p.lse != nullptr)
        p.lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
      return;
    }
    if (handoff) {
      const __amdgpu_buffer_rsrc_t ro = raw_rsrc(p.part_o + 4 * part_o_index<D>(slot, 0, 0, 0, 0),
                                                 4 * (D / 32) * 4 * kWave * 16);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]}), ro,
            static_cast<int>(part_o_index<D>(0, rb, db, i4, lane)) * 16, 0, kScopeDevice);
      if (db == 0 && hh == 0) {
        const __amdgpu_buffer_rsrc_t rm = raw_rsrc(p.part_ml + slot * kMaxRows * 2, kMaxRows * 8);
        using u32x2 = __attribute__((ext_vector_type(2))) unsigned;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(M), __float_as_uint(L)}, rm, r * 8, 0,
                                              kScopeDevice);
      }
    } else {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(p.part_o + 4 * part_o_index<D>(slot, rb, db, i4, lane)) =
            f32x4{acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]};
      if (db == 0 && hh == 0) {
        p.part_ml[(slot * kMaxRows + r) * 2 + 0] = M;
        p.part_ml[(slot * kMaxRows + r) * 2 + 1] = L;
      }
    }
  }
  MAGE_TRACE_POINT(5);
  if (!handoff) return;
  // the row tables are free once every wave has left its tiles; the counter is
  // left at zero for the next launch
  if (!count_in(p.arrivals + static_cast<int64_t>(u) * (kMaxRows / 32) + rb, static_cast<uint32_t>(p.nchunk),
                true, &s_tab[0][0]))
    return;
  MAGE_TRACE_POINT(7);
  // the last arriver: wave w merges kTasks consecutive (d block, register
  // group) pairs of the 4 * kNdb, all chunks' loads of a batch in flight at once
  constexpr int kTasks = kNdb;
  const int t0 = w * kTasks, db = t0 >> 2, i40 = t0 & 3;
  float M, L;
  f32x4 acc[kTasks];
  merge_chunks<D, kHandoffBatch, kTasks, true>(p.part_o, p.part_ml, static_cast<int64_t>(u) * p.nchunk, p.nchunk,
                                               rb, db, i40, lane, r, M, L, acc);
  if (r < p.R) {
    const int b = r / p.G, gg = r - b * p.G;
    const int64_t row = (static_cast<int64_t>(s) * p.B + b) * p.Hq + q_head(h, gg, p.G, p.gs, p.g0);
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int q = 0; q < kTasks; ++q)
      *reinterpret_cast<f32x4*>(p.o + row * D + 32 * db + 8 * (i40 + q) + 4 * hh) =
          f32x4{acc[q][0] * inv, acc[q][1] * inv, acc[q][2] * inv, acc[q][3] * inv};
    if (t0 == 0 && hh == 0 && p.lse != nullptr) p.lse[row] = (M + __log2f(L)) * kLn2;
  }
}

// Merge of split partials (exact pass: chunks of the prefix; sparse pass:
// chunks of the index list). One work-group per (unit, row block, d block);
// wave i4 handles accumulator registers 4*i4..4*i4+3. Also writes lse. Used
// by the exact pass (its O and lse; the score sweep on the select stream
// merges the row statistics it needs itself, so this launch runs beside it)
// and by the sparse pass with per-unit counts; the sparse pass with uniform
// chunks merges inside its own launch (arrival counters).
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
  int nch = (ns + p.chunk - 1) / p.chunk;
  const int r = 32 * w + n;
  int64_t slot0 = static_cast<int64_t>(u) * p.nchunk;
  if (p.counts != nullptr) {
    // this unit's chunks follow those of the sequence's lower heads; never
    // past the sequence's slots (counts above the plan's bound lose chunks)
    int before = 0;
    for (int h2 = 0; h2 < h; ++h2) before += (max(0, min(p.counts[s * p.Hkv + h2], ns)) + p.chunk - 1) / p.chunk;
    nch = (max(0, min(p.counts[u], ns)) + p.chunk - 1) / p.chunk;
    if (nch == 1 && before < p.seq_slots) return;   // its one chunk wrote O and lse
    nch = max(0, min(nch, p.seq_slots - before));
    slot0 = static_cast<int64_t>(s) * p.seq_slots + before;
  }
  float M, L;
  f32x4 accs[1];
  merge_chunks<D, kBatch, 1, false>(p.part_o, p.part_ml, slot0, nch, w, db, i4, lane, r, M, L, accs);
  const f32x4 acc = accs[0];
  if (r >= p.R) return;
  const int b = r / p.G, g = r - b * p.G, j = q_head(h, g, p.G, p.gs, p.g0);
  const int64_t row = (static_cast<int64_t>(s) * p.B + b) * p.Hq + j;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  f32x4 v{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  *reinterpret_cast<f32x4*>(p.o + row * D + 32 * db + 8 * i4 + 4 * hh) = v;
  if (db == 0 && i4 == 0 && hh == 0 && p.lse != nullptr) p.lse[row] = (M + __log2f(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// Block attention: a block-diffusion layer's attention for the B tokens of the
// current block is the softmax over the selected prefix rows together with
// the block's own B rows, which every token of the block sees (the block is
// denoised jointly; MAGE page, "Problem" and "Approach" select only the
// prefix rows). The prefix part comes from the exact or sparse pass as a
// normalised O and its log-sum-exp; this kernel attends the block's queries
// to the block's keys and merges the two parts through their log-sum-exps:
//   O = (e^{lse_p} O_p + e^{lse_b} O_b) / (e^{lse_p} + e^{lse_b}),
//   lse = log(e^{lse_p} + e^{lse_b}).
// One wave per (unit, 32-row block); the B <= 128 block keys stream through a
// two-stage LDS ring of 32-key tiles.
struct BlockParams {
  const uint16_t* q;        // bf16 [S][B][Hq][d]
  const uint16_t* k_blk;    // bf16 [S][Hkv][B][d]: the block's own keys
  const uint16_t* v_blk;    // bf16 [S][Hkv][B][d]
  const float* o_pre;       // fp32 [S][B][Hq][d]: normalised attention over the prefix rows
  const float* lse_pre;     // fp32 [S][B][Hq]: its natural log-sum-exp (-inf: no prefix row)
  float* o;                 // fp32 [S][B][Hq][d]; may be o_pre
  float* lse;               // fp32 [S][B][Hq] or null; may be lse_pre
  int32_t S, B, Hq, Hkv, G, R;
  int32_t gs, g0;           // a sub-group of query heads: head stride, first head (0, 0: the whole group)
  float scale_log2;         // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(kWave) void block_attn_kernel(BlockParams p) {
  using T = SparseTile<D>;
  constexpr int kNdb = D / 32, kNks = D / 16;
  static_assert(2 * T::kInstr < 64, "vmcnt is 6 bits");
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[2 * T::kStageBytes];
  const int lane = threadIdx.x, hh = lane >> 5, n = lane & 31;
  const int nrb = (p.R + 31) >> 5;
  const int u = blockIdx.x / nrb, rb = blockIdx.x - (blockIdx.x / nrb) * nrb;
  if (u >= p.S * p.Hkv) return;
  const int s = u / p.Hkv, h = u - s * p.Hkv;

  bf16x8 qf[kNks];
  const int r = 32 * rb + n;
  {
    if (r < p.R) {
      const int b = r / p.G, gg = r - b * p.G;
      const uint16_t* qrow = p.q + ((static_cast<int64_t>(s) * p.B + b) * p.Hq + q_head(h, gg, p.G, p.gs, p.g0)) * D;
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, load16(qrow + 16 * ks + 8 * hh));
    } else {
#pragma unroll
      for (int ks = 0; ks < kNks; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  wait_vmcnt<0>();   // Q in registers before the untracked tile loads start

  const int64_t row0 = (static_cast<int64_t>(s) * p.Hkv + h) * p.B;   // first block row of this unit
  const int ntiles = (p.B + kSparseTileKeys - 1) / kSparseTileKeys;
  auto issue = [&](int t) {
    uint8_t* st = s_ring + (t & 1) * T::kStageBytes;
    issue_sparse_tile<D>(st, st + T::kKBytes, p.k_blk, p.v_blk,
                         [&](int rr) { return (row0 + min(t * kSparseTileKeys + rr, p.B - 1)) * D; }, lane);
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
  const uint32_t v_lane = T::kKBytes + vt_lane_offset(lane);
  issue(0);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      issue(t + 1);
      wait_vmcnt<2 * T::kInstr>();
    } else {
      wait_vmcnt<0>();
    }
    const uint32_t okm = static_cast<uint32_t>(__ballot(t * kSparseTileKeys + n < p.B));
    const uint32_t st = ring_base + (t & 1) * T::kStageBytes;
    attend_half<D, T::kVBlock>(st, st + v_lane, kofs, qf, okm, p.scale_log2, m_run, l_run, oacc, lane);
    // the stage of tile t is refilled by the issue of tile t+2, after the
    // next iteration's wait: its reads above have completed by then
  }
  l_run = wave_sum_pair(l_run);
  if (r >= p.R) return;
  const int b = r / p.G, gg = r - b * p.G;
  const int64_t row = (static_cast<int64_t>(s) * p.B + b) * p.Hq + q_head(h, gg, p.G, p.gs, p.g0);
  // log2 units: the block part's log-sum-exp is m + log2(l) (l >= 1)
  const float lb = m_run + __log2f(l_run);
  const float lp = p.lse_pre[row] * kLog2e;
  const float M = fmaxf(lb, lp);
  const float wp = fast_exp2(lp - M), wb = fast_exp2(lb - M);   // lp = -inf gives 0
  const float inv = 1.f / (wp + wb);
  const float cp = wp * inv, cb = wb * inv / l_run;
  const float* opre = p.o_pre + row * D + 4 * hh;
  float* orow = p.o + row * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(opre + 32 * db + 8 * i4);
      *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i4) =
          f32x4{cp * x[0] + cb * oacc[db][4 * i4], cp * x[1] + cb * oacc[db][4 * i4 + 1],
                cp * x[2] + cb * oacc[db][4 * i4 + 2], cp * x[3] + cb * oacc[db][4 * i4 + 3]};
    }
  if (hh == 0 && p.lse != nullptr) p.lse[row] = (M + __log2f(wp + wb)) * kLn2;
}

}  // namespace mage
