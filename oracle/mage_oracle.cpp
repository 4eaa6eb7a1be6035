// CPU oracle for block-shared top-k sparse KV attention (MAGE).
//
// TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
// CPU-baseline leg may load this library. It shares no code, header or
// constant with the HIP library and must never be used as a fallback for it.
//
// What it computes (plain definitions, fp64 throughout, no blocking or fusion):
//
//  * Exact step-1 attention of the all-[MASK] block over the prefix KV cache
//    ("MAGE: All-[MASK] Block Already Knows Where to Look in Block Diffusion
//    LLM", atlas.scime.ai summary, opening summary and "Approach"). For query
//    head j the KV head is j / G (contiguous GQA groups). For every row
//    r = (b, g) of KV head h:
//        x[r][p] = scale * sum_i Q[b][hG+g][i] * K[h][p][i]
//        M[r] = max_p x[r][p],  L[r] = sum_p exp(x[r][p] - M[r])
//        P[r][p] = exp(x[r][p] - M[r]) / L[r]
//        O[b][hG+g][:] = sum_p P[r][p] V[h][p][:],  lse = M[r] + log L[r]
//  * The per-block score that picks the block-shared KV subset (same page,
//    "Problem": every token of a block shares one KV subset; "Approach": the
//    exact pass at step 1 reveals the per-block top-k): the softmax
//    probability averaged over the B block tokens and the G query heads of
//    the group,  score[h][p] = (1 / (B G)) sum_r P[r][p].
//  * Top-k of the score with ties broken by the lower position: a full sort
//    under the strict order (score descending, position ascending); the first
//    min(k, N) positions, returned in ascending order, -1 past the end.
//  * The later-step sparse attention (same page, "Approach": later steps reuse
//    the step-1 index set): gather the selected K and V rows into dense
//    arrays, then the same formulas over the gathered rows. Index entries
//    outside [0, N) are skipped; with no valid entry O = 0 and lse = -inf.
//  * Paged caches are first copied back to contiguous rows (logical position
//    p lives in page table[p / page] at slot p % page), then handled as above.
//  * Block attention, the op a block-diffusion layer calls: the queries of the
//    current block attend to the selected prefix rows (all of them, or the
//    idx set) together with all B rows of their own block, which the block's
//    tokens share (same page, "Problem": the block is denoised jointly and
//    only the prefix rows are selected). Written as its definition: one
//    softmax over the union of the two row sets, formulas as above.
//
// bf16 inputs are widened exactly (bits << 16 is the fp32 value).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#include <omp.h>

namespace {

inline double widen_bf16(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// Attention of R rows of one KV head over n rows of K/V (dense, row-major).
// q_rows[r] points at the d bf16 values of row r. Writes O rows (fp64), lse,
// and, if probs != nullptr, the probability matrix probs[r * n + p].
void dense_attention(int R, int n, int d, double scale,
                     const std::vector<const uint16_t*>& q_rows,
                     const std::vector<double>& Kd, const std::vector<double>& Vd,
                     const std::vector<double*>& o_rows, const std::vector<double*>& lse_rows,
                     double* probs) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) {
    std::vector<double> q(d), x(n);
    for (int i = 0; i < d; ++i) q[i] = widen_bf16(q_rows[r][i]);
    double* o = o_rows[r];
    if (n == 0) {
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      *lse_rows[r] = -std::numeric_limits<double>::infinity();
      continue;
    }
    double M = -std::numeric_limits<double>::infinity();
    for (int p = 0; p < n; ++p) {
      const double* kp = &Kd[static_cast<size_t>(p) * d];
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += q[i] * kp[i];
      x[p] = scale * acc;
      M = std::max(M, x[p]);
    }
    double L = 0.0;
    for (int p = 0; p < n; ++p) L += std::exp(x[p] - M);
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int p = 0; p < n; ++p) {
      const double P = std::exp(x[p] - M) / L;
      if (probs) probs[static_cast<size_t>(r) * n + p] = P;
      const double* vp = &Vd[static_cast<size_t>(p) * d];
      for (int i = 0; i < d; ++i) o[i] += P * vp[i];
    }
    *lse_rows[r] = M + std::log(L);
  }
}

void widen_rows(const uint16_t* src, int n, int d, std::vector<double>& dst) {
  dst.resize(static_cast<size_t>(n) * d);
  for (size_t i = 0; i < dst.size(); ++i) dst[i] = widen_bf16(src[i]);
}

}  // namespace

extern "C" {

// Threads an OpenMP region of the oracle uses.
int oracle_num_threads(void) { return omp_get_max_threads(); }

// One sequence. Q bf16 [B][Hq][d]; K, V bf16 [Hkv][N][d].
// Outputs: O fp64 [B][Hq][d], lse fp64 [B][Hq], score fp64 [Hkv][N] (nullable).
// Returns 0, or -1 on invalid sizes.
int oracle_exact_seq(int B, int Hq, int Hkv, int d, double scale,
                     const uint16_t* Q, const uint16_t* K, const uint16_t* V, int N,
                     double* O, double* lse, double* score) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || N < 0 || Hq % Hkv) return -1;
  const int G = Hq / Hkv, R = B * G;
  std::vector<double> Kd, Vd, probs;
  for (int h = 0; h < Hkv; ++h) {
    widen_rows(K + static_cast<size_t>(h) * N * d, N, d, Kd);
    widen_rows(V + static_cast<size_t>(h) * N * d, N, d, Vd);
    std::vector<const uint16_t*> qr(R);
    std::vector<double*> orow(R), lrow(R);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < G; ++g) {
        const int r = b * G + g, j = h * G + g;
        qr[r] = Q + (static_cast<size_t>(b) * Hq + j) * d;
        orow[r] = O + (static_cast<size_t>(b) * Hq + j) * d;
        lrow[r] = lse + static_cast<size_t>(b) * Hq + j;
      }
    probs.assign(score ? static_cast<size_t>(R) * N : 0, 0.0);
    dense_attention(R, N, d, scale, qr, Kd, Vd, orow, lrow, score ? probs.data() : nullptr);
    if (score) {
      double* sc = score + static_cast<size_t>(h) * N;
#pragma omp parallel for schedule(static)
      for (int p = 0; p < N; ++p) {
        double acc = 0.0;
        for (int r = 0; r < R; ++r) acc += probs[static_cast<size_t>(r) * N + p];
        sc[p] = acc / static_cast<double>(R);
      }
    }
  }
  return 0;
}

// Top-k of one score row under (score descending, position ascending).
// idx gets k entries: the first min(k, N) positions in ascending order, then -1.
int oracle_topk_row(const double* score, int N, int k, int32_t* idx) {
  if (N < 0 || k <= 0) return -1;
  std::vector<int32_t> order(N);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [score](int32_t a, int32_t b) {
    if (score[a] != score[b]) return score[a] > score[b];
    return a < b;
  });
  const int keff = std::min(k, N);
  std::sort(order.begin(), order.begin() + keff);
  for (int i = 0; i < k; ++i) idx[i] = i < keff ? order[i] : -1;
  return 0;
}

// Top-k of `rows` independent score rows of length N each (row-major).
int oracle_topk(const double* score, int rows, int N, int k, int32_t* idx) {
  if (rows < 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int r = 0; r < rows; ++r)
    bad |= oracle_topk_row(score + static_cast<size_t>(r) * N, N, k,
                           idx + static_cast<size_t>(r) * k) != 0;
  return bad ? -1 : 0;
}

// Sparse attention of one sequence over the gathered rows idx[h][0..k).
// Q bf16 [B][Hq][d]; K, V bf16 [Hkv][N][d]; idx int32 [Hkv][k].
int oracle_sparse_seq(int B, int Hq, int Hkv, int d, double scale,
                      const uint16_t* Q, const uint16_t* K, const uint16_t* V, int N,
                      const int32_t* idx, int k, double* O, double* lse) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || N < 0 || k < 0 || Hq % Hkv) return -1;
  const int G = Hq / Hkv, R = B * G;
  std::vector<double> Kd, Vd;
  for (int h = 0; h < Hkv; ++h) {
    // gather, then dense
    std::vector<int32_t> sel;
    for (int i = 0; i < k; ++i) {
      const int32_t p = idx[static_cast<size_t>(h) * k + i];
      if (p >= 0 && p < N) sel.push_back(p);
    }
    const int n = static_cast<int>(sel.size());
    Kd.assign(static_cast<size_t>(n) * d, 0.0);
    Vd.assign(static_cast<size_t>(n) * d, 0.0);
    for (int t = 0; t < n; ++t) {
      const uint16_t* kr = K + (static_cast<size_t>(h) * N + sel[t]) * d;
      const uint16_t* vr = V + (static_cast<size_t>(h) * N + sel[t]) * d;
      for (int i = 0; i < d; ++i) {
        Kd[static_cast<size_t>(t) * d + i] = widen_bf16(kr[i]);
        Vd[static_cast<size_t>(t) * d + i] = widen_bf16(vr[i]);
      }
    }
    std::vector<const uint16_t*> qr(R);
    std::vector<double*> orow(R), lrow(R);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < G; ++g) {
        const int r = b * G + g, j = h * G + g;
        qr[r] = Q + (static_cast<size_t>(b) * Hq + j) * d;
        orow[r] = O + (static_cast<size_t>(b) * Hq + j) * d;
        lrow[r] = lse + static_cast<size_t>(b) * Hq + j;
      }
    dense_attention(R, n, d, scale, qr, Kd, Vd, orow, lrow, nullptr);
  }
  return 0;
}

// Block attention of one sequence: softmax over the prefix rows idx[h][0..k)
// (idx null: all N rows; entries outside [0, N) skipped) followed by the B
// block rows Kb/Vb [Hkv][B][d]. Q bf16 [B][Hq][d]; K, V bf16 [Hkv][N][d].
// Outputs O fp64 [B][Hq][d], lse fp64 [B][Hq].
int oracle_block_seq(int B, int Hq, int Hkv, int d, double scale,
                     const uint16_t* Q, const uint16_t* K, const uint16_t* V, int N,
                     const int32_t* idx, int k, const uint16_t* Kb, const uint16_t* Vb,
                     double* O, double* lse) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || N < 0 || k < 0 || Hq % Hkv) return -1;
  const int G = Hq / Hkv, R = B * G;
  std::vector<double> Kd, Vd;
  for (int h = 0; h < Hkv; ++h) {
    std::vector<const uint16_t*> krow, vrow;   // the union, prefix rows first
    if (idx) {
      for (int i = 0; i < k; ++i) {
        const int32_t p = idx[static_cast<size_t>(h) * k + i];
        if (p >= 0 && p < N) {
          krow.push_back(K + (static_cast<size_t>(h) * N + p) * d);
          vrow.push_back(V + (static_cast<size_t>(h) * N + p) * d);
        }
      }
    } else {
      for (int p = 0; p < N; ++p) {
        krow.push_back(K + (static_cast<size_t>(h) * N + p) * d);
        vrow.push_back(V + (static_cast<size_t>(h) * N + p) * d);
      }
    }
    for (int t = 0; t < B; ++t) {
      krow.push_back(Kb + (static_cast<size_t>(h) * B + t) * d);
      vrow.push_back(Vb + (static_cast<size_t>(h) * B + t) * d);
    }
    const int n = static_cast<int>(krow.size());
    Kd.assign(static_cast<size_t>(n) * d, 0.0);
    Vd.assign(static_cast<size_t>(n) * d, 0.0);
    for (int t = 0; t < n; ++t)
      for (int i = 0; i < d; ++i) {
        Kd[static_cast<size_t>(t) * d + i] = widen_bf16(krow[t][i]);
        Vd[static_cast<size_t>(t) * d + i] = widen_bf16(vrow[t][i]);
      }
    std::vector<const uint16_t*> qr(R);
    std::vector<double*> orow(R), lrow(R);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < G; ++g) {
        const int r = b * G + g, j = h * G + g;
        qr[r] = Q + (static_cast<size_t>(b) * Hq + j) * d;
        orow[r] = O + (static_cast<size_t>(b) * Hq + j) * d;
        lrow[r] = lse + static_cast<size_t>(b) * Hq + j;
      }
    dense_attention(R, n, d, scale, qr, Kd, Vd, orow, lrow, nullptr);
  }
  return 0;
}

// Copy one sequence's rows out of a page pool [P][Hkv][page][d] into
// contiguous [Hkv][N][d]: logical position p is slot p % page of page
// table_row[p / page].
int oracle_depage(const uint16_t* pool, int Hkv, int page, int d,
                  const int32_t* table_row, int N, uint16_t* out) {
  if (Hkv <= 0 || page <= 0 || d <= 0 || N < 0) return -1;
  for (int h = 0; h < Hkv; ++h)
    for (int p = 0; p < N; ++p) {
      const int64_t pg = table_row[p / page];
      const uint16_t* src = pool + ((pg * Hkv + h) * page + p % page) * static_cast<int64_t>(d);
      std::memcpy(out + (static_cast<size_t>(h) * N + p) * d, src, sizeof(uint16_t) * d);
    }
  return 0;
}

}  // extern "C"
