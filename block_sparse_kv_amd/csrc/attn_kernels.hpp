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
// share the KV head are one MFMA tile and every K/V row staged in LDS is used
// by all of them. Per 64-key tile:
//   S^T[key][row] = K Q^T        v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//                                B = Q held in registers)
//   online softmax on the rows   (exp2 with scale * log2(e) folded in)
//   O^T[d][row] += V^T P^T       v_mfma_f32_32x32x16_f16 (A = V^T from LDS,
//                                stored transposed as fp16, B = P as fp16)
// K is loaded into its MFMA A operand with the row order pi(m) (bits 2 and 3
// of m swapped); with that order the S^T accumulator registers 8s..8s+7 of a
// lane hold 8 consecutive keys, which is exactly the B operand layout of the
// PV product, so P never leaves registers.
#pragma once

#include "mage_common.hpp"

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
  uint32_t* counters;       // word 2u per unit, sparse pass only (self-resetting)
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
  int32_t n_uniform;        // >= 0: contiguous prefix length; < 0: use lens
  SeqLens lens;
};

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

template <int D, bool kSparse>
__global__ __launch_bounds__(kThreads) void attn_chunk_kernel(AttnParams p) {
  constexpr int kCpr = D / 8;                          // 16-byte pieces per K/V row
  constexpr int kKpt = kTileKeys * kCpr / kThreads;    // keys per thread per tile (4 or 2)
  constexpr int kNdb = D / 32;
  constexpr int kNks = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kTileKeys * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[D * kTileKeys];
  __shared__ int s_ok[kTileKeys];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int s = u / p.Hkv, h = u - s * p.Hkv;
  const int ns = seq_len_of(p.kv, p.lens, s);
  const int e0 = c * p.chunk;
  const int e1 = kSparse ? min(e0 + p.chunk, p.idx_k) : min(e0 + p.chunk, ns);
  if (e0 >= e1) return;  // exact pass: chunk past this sequence's end (never in the sparse grid)
  const int nrb = (p.R + 31) >> 5;
  const bool computes = w < nrb;

  // Q rows of this wave as MFMA B operand fragments (d slice 16ks + 8hh .. +7)
  bf16x8 qf[kNks];
  {
    const int r = 32 * w + n;
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

  f32x16 oacc[kNdb];
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;

  // loader mapping: piece lc of keys kg*kKpt .. kg*kKpt + kKpt-1
  const int lc = tid % kCpr, kg = tid / kCpr;
  u32x4 kreg[kKpt], vreg[kKpt];
  int okreg[kKpt];
  const int ntiles = (e1 - e0 + kTileKeys - 1) / kTileKeys;

  auto issue = [&](int tile) {
#pragma unroll
    for (int j = 0; j < kKpt; ++j) {
      const int e = e0 + tile * kTileKeys + kg * kKpt + j;
      bool ok = e < e1;
      int pos = e;
      if (kSparse) {
        pos = ok ? p.idx[static_cast<int64_t>(u) * p.idx_k + e] : -1;
        ok = ok && pos >= 0 && pos < ns;
      }
      okreg[j] = ok;
      if (ok) {
        const int64_t off = kv_row(p.kv, s, h, p.Hkv, pos, D) + lc * 8;
        kreg[j] = load16(p.kv.k + off);
        vreg[j] = load16(p.kv.v + off);
      } else {
        kreg[j] = u32x4{0, 0, 0, 0};
        vreg[j] = u32x4{0, 0, 0, 0};
      }
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < kKpt; ++j) {
      const int key = kg * kKpt + j;
      const int phys = lc ^ (key % kCpr);
      *reinterpret_cast<u32x4*>(&s_k[key * D + phys * 8]) = kreg[j];
      if (lc == 0) s_ok[key] = okreg[j];
    }
    // V^T in fp16: row d holds the tile's 64 keys; 16-byte key groups are
    // XOR-swizzled by (d & 7)
    const int key0 = kg * kKpt;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = lc * 8 + i;
      float vals[kKpt];
#pragma unroll
      for (int j = 0; j < kKpt; ++j)
        vals[j] = (i & 1) ? bf16_hi(vreg[j][i >> 1]) : bf16_lo(vreg[j][i >> 1]);
      const int kc = key0 >> 3, within = key0 & 7;
      uint16_t* dst = &s_vt[d * kTileKeys + ((kc ^ (d & 7)) << 3) + within];
      if constexpr (kKpt == 4) {
        u32x2 pk{pack_f16(vals[0], vals[1]), pack_f16(vals[2], vals[3])};
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = pack_f16(vals[0], vals[1]);
      }
    }
  };

  issue(0);
  const int krow_perm = swap_bits23(n);
  for (int t = 0; t < ntiles; ++t) {
    stage();
    __syncthreads();
    if (t + 1 < ntiles) issue(t + 1);
    if (computes) {
      const uint64_t okm = __ballot(s_ok[lane] != 0);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
        const int krow = 32 * kb + krow_perm;
#pragma unroll
        for (int ks = 0; ks < kNks; ++ks) {
          const int phys = (2 * ks + hh) ^ (krow % kCpr);
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&s_k[krow * D + phys * 8]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
        }
      }
      // register i of key block kb holds key 32kb + 16(i/8) + 8hh + (i%8)
      float mt = -__builtin_inff();
      if (okm == ~0ull) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            sacc[kb][i] *= p.scale_log2;
            mt = fmaxf(mt, sacc[kb][i]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
            const float x = ((okm >> key) & 1) ? sacc[kb][i] * p.scale_log2 : -__builtin_inff();
            sacc[kb][i] = x;
            mt = fmaxf(mt, x);
          }
      }
      mt = wave_max_pair(mt);
      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(sacc[kb][i] - m_use);
          sacc[kb][i] = pv;
          rs += pv;
        }
      rs = wave_sum_pair(rs);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < kNdb; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      f16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 pk{pack_f16(sacc[kb][8 * s2 + 0], sacc[kb][8 * s2 + 1]),
                   pack_f16(sacc[kb][8 * s2 + 2], sacc[kb][8 * s2 + 3]),
                   pack_f16(sacc[kb][8 * s2 + 4], sacc[kb][8 * s2 + 5]),
                   pack_f16(sacc[kb][8 * s2 + 6], sacc[kb][8 * s2 + 7])};
          pf[kb][s2] = __builtin_bit_cast(f16x8, pk);
        }
#pragma unroll
      for (int db = 0; db < kNdb; ++db) {
        const int d = 32 * db + n;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int kc = 4 * kb + 2 * s2 + hh;
            const f16x8 vf =
                *reinterpret_cast<const f16x8*>(&s_vt[d * kTileKeys + ((kc ^ (d & 7)) << 3)]);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kb][s2], oacc[db], 0, 0, 0);
          }
      }
    }
    __syncthreads();
  }

  if (kSparse && p.nchunk == 1) {
    if (computes) store_rows<D>(p, s, h, w, lane, m_run, l_run, oacc);
    return;
  }

  // partial result of this chunk
  const int64_t slot = static_cast<int64_t>(u) * p.nchunk + c;
  if (computes) {
#pragma unroll
    for (int db = 0; db < kNdb; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v{oacc[db][4 * i4], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]};
        *reinterpret_cast<f32x4*>(p.part_o + 4 * part_o_index<D>(slot, w, db, i4, lane)) = v;
      }
    if (hh == 0) {
      p.part_ml[(slot * kMaxRows + 32 * w + n) * 2 + 0] = m_run;
      p.part_ml[(slot * kMaxRows + 32 * w + n) * 2 + 1] = l_run;
    }
  }
  if (!kSparse) return;

  // sparse pass: the last chunk of a unit to finish merges all of them
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&p.counters[2 * u], 1u);
    __threadfence();
    s_last = prev == static_cast<unsigned>(p.nchunk - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid == 0) p.counters[2 * u] = 0u;
  if (!computes) return;
  const int r = 32 * w + n;
  const int64_t slot0 = static_cast<int64_t>(u) * p.nchunk;
  float M = -__builtin_inff();
  for (int cc = 0; cc < p.nchunk; ++cc) M = fmaxf(M, p.part_ml[((slot0 + cc) * kMaxRows + r) * 2]);
  const float Mu = M == -__builtin_inff() ? 0.f : M;
  float L = 0.f;
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  for (int cc = 0; cc < p.nchunk; ++cc) {
    const float mc = p.part_ml[((slot0 + cc) * kMaxRows + r) * 2];
    const float lc2 = p.part_ml[((slot0 + cc) * kMaxRows + r) * 2 + 1];
    const float wc = fast_exp2(mc - Mu);
    L += lc2 * wc;
#pragma unroll
    for (int db = 0; db < kNdb; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(p.part_o + 4 * part_o_index<D>(slot0 + cc, w, db, i4, lane));
        oacc[db][4 * i4 + 0] += wc * v[0];
        oacc[db][4 * i4 + 1] += wc * v[1];
        oacc[db][4 * i4 + 2] += wc * v[2];
        oacc[db][4 * i4 + 3] += wc * v[3];
      }
  }
  store_rows<D>(p, s, h, w, lane, M, L, oacc);
}

// Merge of the exact pass's split partials. One work-group per
// (unit, row block, d block); wave i4 handles accumulator registers 4*i4..4*i4+3.
// Also writes lse and the per-row max + log2(sum) that the score sweep needs.
template <int D>
__global__ __launch_bounds__(kThreads) void exact_merge_kernel(MergeParams p) {
  constexpr int kNdb = D / 32;
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
  float M = -__builtin_inff();
  for (int c = 0; c < nch; ++c) M = fmaxf(M, p.part_ml[((slot0 + c) * kMaxRows + r) * 2]);
  const float Mu = M == -__builtin_inff() ? 0.f : M;
  float L = 0.f;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    const float mc = p.part_ml[((slot0 + c) * kMaxRows + r) * 2];
    const float lc = p.part_ml[((slot0 + c) * kMaxRows + r) * 2 + 1];
    const float wc = fast_exp2(mc - Mu);
    L += lc * wc;
    const f32x4 v = *reinterpret_cast<const f32x4*>(
        p.part_o + 4 * part_o_index<D>(slot0 + c, w, db, i4, lane));
    acc[0] += wc * v[0];
    acc[1] += wc * v[1];
    acc[2] += wc * v[2];
    acc[3] += wc * v[3];
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
    p.rowstat[static_cast<int64_t>(u) * kMaxRows + r] = c2;
  }
}

}  // namespace mage
