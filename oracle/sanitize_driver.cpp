// Drives every exported function of the CPU oracle (mage_oracle.cpp) through
// small cases, including the edge cases (empty prefix, k > N, one row, skipped
// and repeated index entries, ragged pages), and checks the invariants that
// fix each result. Built together with mage_oracle.cpp under AddressSanitizer
// and UndefinedBehaviorSanitizer by the CPU test suite, so that an
// out-of-bounds access, a use after free or undefined arithmetic in the
// checker itself fails a test. TEST INFRASTRUCTURE ONLY, like the oracle.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int oracle_num_threads(void);
int oracle_exact_seq(int B, int Hq, int Hkv, int d, double scale, const uint16_t* Q, const uint16_t* K,
                     const uint16_t* V, int N, double* O, double* lse, double* score);
int oracle_topk_row(const double* score, int N, int k, int32_t* idx);
int oracle_topk(const double* score, int rows, int N, int k, int32_t* idx);
int oracle_sparse_seq(int B, int Hq, int Hkv, int d, double scale, const uint16_t* Q, const uint16_t* K,
                      const uint16_t* V, int N, const int32_t* idx, int k, double* O, double* lse);
int oracle_block_seq(int B, int Hq, int Hkv, int d, double scale, const uint16_t* Q, const uint16_t* K,
                     const uint16_t* V, int N, const int32_t* idx, int k, const uint16_t* Kb,
                     const uint16_t* Vb, double* O, double* lse);
int oracle_depage(const uint16_t* pool, int Hkv, int page, int d, const int32_t* table_row, int N,
                  uint16_t* out);
}

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::printf("FAIL line %d: %s\n", line, what);
    ++g_fail;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

uint16_t to_bf16(float f) {   // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

std::vector<uint16_t> randn_bf16(size_t n, std::mt19937& g, float sd) {
  std::normal_distribution<float> nd(0.f, sd);
  std::vector<uint16_t> v(n > 0 ? n : 1);   // never an empty (null) buffer
  for (auto& x : v) x = to_bf16(nd(g));
  return v;
}

double max_abs_diff(const std::vector<double>& a, const std::vector<double>& b) {
  double m = 0.0;
  for (size_t i = 0; i < a.size(); ++i) m = std::fmax(m, std::fabs(a[i] - b[i]));
  return m;
}

// Exact pass, scores, top-k and the later step on one random case; k may exceed N.
void case_select(int B, int Hq, int Hkv, int d, int N, int k, unsigned seed) {
  std::mt19937 g(seed);
  const double scale = 1.0 / std::sqrt(static_cast<double>(d));
  auto Q = randn_bf16(static_cast<size_t>(B) * Hq * d, g, 1.f);
  auto K = randn_bf16(static_cast<size_t>(Hkv) * N * d, g, 1.f);
  auto V = randn_bf16(static_cast<size_t>(Hkv) * N * d, g, 1.f);
  std::vector<double> O(static_cast<size_t>(B) * Hq * d), lse(static_cast<size_t>(B) * Hq),
      sc(static_cast<size_t>(Hkv) * N);
  EXPECT(oracle_exact_seq(B, Hq, Hkv, d, scale, Q.data(), K.data(), V.data(), N, O.data(), lse.data(),
                          sc.data()) == 0);
  for (int h = 0; h < Hkv && N > 0; ++h) {
    double s = 0.0;
    for (int p = 0; p < N; ++p) {
      EXPECT(sc[static_cast<size_t>(h) * N + p] >= 0.0);
      s += sc[static_cast<size_t>(h) * N + p];
    }
    EXPECT(std::fabs(s - 1.0) < 1e-12);
  }
  std::vector<int32_t> idx(static_cast<size_t>(Hkv) * k);
  EXPECT(oracle_topk(sc.data(), Hkv, N, k, idx.data()) == 0);
  const int keff = std::min(k, N);
  for (int h = 0; h < Hkv; ++h) {
    const int32_t* row = idx.data() + static_cast<size_t>(h) * k;
    for (int i = 0; i < k; ++i) {
      if (i < keff) {
        EXPECT(row[i] >= 0 && row[i] < N);
        if (i > 0) EXPECT(row[i] > row[i - 1]);
      } else {
        EXPECT(row[i] == -1);
      }
    }
    // rank of every selected position by brute-force counting is below keff
    const double* s = sc.data() + static_cast<size_t>(h) * N;
    for (int i = 0; i < keff; ++i) {
      const int p = row[i];
      int rank = 0;
      for (int q = 0; q < N; ++q) rank += s[q] > s[p] || (s[q] == s[p] && q < p);
      EXPECT(rank < keff);
    }
  }
  // later step over the selection; with k >= N it equals the exact pass
  std::vector<double> O2(O.size()), l2(lse.size());
  EXPECT(oracle_sparse_seq(B, Hq, Hkv, d, scale, Q.data(), K.data(), V.data(), N, idx.data(), k, O2.data(),
                           l2.data()) == 0);
  if (k >= N && N > 0) {
    EXPECT(max_abs_diff(O, O2) < 1e-12);
    EXPECT(max_abs_diff(lse, l2) < 1e-12);
  }
  // block attention with an empty prefix selection equals attention over the block rows alone
  auto Kb = randn_bf16(static_cast<size_t>(Hkv) * B * d, g, 1.f);
  auto Vb = randn_bf16(static_cast<size_t>(Hkv) * B * d, g, 1.f);
  std::vector<int32_t> none(static_cast<size_t>(Hkv) * 1, -1);
  std::vector<double> O3(O.size()), l3(lse.size()), O4(O.size()), l4(lse.size());
  EXPECT(oracle_block_seq(B, Hq, Hkv, d, scale, Q.data(), K.data(), V.data(), N, none.data(), 1, Kb.data(),
                          Vb.data(), O3.data(), l3.data()) == 0);
  EXPECT(oracle_exact_seq(B, Hq, Hkv, d, scale, Q.data(), Kb.data(), Vb.data(), B, O4.data(), l4.data(),
                          nullptr) == 0);
  EXPECT(max_abs_diff(O3, O4) < 1e-12);
  EXPECT(max_abs_diff(l3, l4) < 1e-12);
  // block attention over all prefix rows (idx null) and over an idx with repeats and junk
  EXPECT(oracle_block_seq(B, Hq, Hkv, d, scale, Q.data(), K.data(), V.data(), N, nullptr, 0, Kb.data(),
                          Vb.data(), O3.data(), l3.data()) == 0);
  std::vector<int32_t> junk(static_cast<size_t>(Hkv) * 4);
  for (int h = 0; h < Hkv; ++h) {
    junk[h * 4 + 0] = N > 0 ? 0 : -1;
    junk[h * 4 + 1] = N > 0 ? 0 : -1;
    junk[h * 4 + 2] = N;        // out of range: skipped
    junk[h * 4 + 3] = -7;       // negative: skipped
  }
  EXPECT(oracle_sparse_seq(B, Hq, Hkv, d, scale, Q.data(), K.data(), V.data(), N, junk.data(), 4, O2.data(),
                           l2.data()) == 0);
  if (N > 0) {   // two copies of row 0: O = V[0], lse = logit + log 2
    for (int b = 0; b < B; ++b)
      for (int j = 0; j < Hq; ++j) {
        const int h = j / (Hq / Hkv);
        double x = 0.0;
        for (int i = 0; i < d; ++i) {
          uint32_t uq = static_cast<uint32_t>(Q[(static_cast<size_t>(b) * Hq + j) * d + i]) << 16;
          uint32_t uk = static_cast<uint32_t>(K[(static_cast<size_t>(h) * N) * d + i]) << 16;
          float fq, fk;
          std::memcpy(&fq, &uq, 4);
          std::memcpy(&fk, &uk, 4);
          x += static_cast<double>(fq) * fk;
        }
        EXPECT(std::fabs(l2[static_cast<size_t>(b) * Hq + j] - (scale * x + std::log(2.0))) < 1e-12);
      }
  } else {
    for (double v : l2) EXPECT(std::isinf(v) && v < 0);
    for (double v : O2) EXPECT(v == 0.0);
  }
}

// A ragged paged sequence copied back to contiguous rows equals its source rows.
void case_depage(int Hkv, int page, int d, int N, unsigned seed) {
  std::mt19937 g(seed);
  const int pages = (N + page - 1) / page, P = pages + 3;
  auto pool = randn_bf16(static_cast<size_t>(P) * Hkv * page * d, g, 1.f);
  std::vector<int32_t> table(pages);
  for (int i = 0; i < pages; ++i) table[i] = (i * 5 + 2) % P;   // distinct: 5 is coprime to P here
  std::vector<uint16_t> out(static_cast<size_t>(Hkv) * N * d);
  EXPECT(oracle_depage(pool.data(), Hkv, page, d, table.data(), N, out.data()) == 0);
  for (int h = 0; h < Hkv; ++h)
    for (int p = 0; p < N; ++p)
      for (int i = 0; i < d; ++i)
        EXPECT(out[(static_cast<size_t>(h) * N + p) * d + i] ==
               pool[((static_cast<size_t>(table[p / page]) * Hkv + h) * page + p % page) * d + i]);
}

void case_ties() {
  std::vector<double> s(50, 0.02);
  std::vector<int32_t> idx(60);
  EXPECT(oracle_topk_row(s.data(), 50, 60, idx.data()) == 0);
  for (int i = 0; i < 60; ++i) EXPECT(idx[i] == (i < 50 ? i : -1));
  EXPECT(oracle_topk_row(s.data(), 50, 7, idx.data()) == 0);
  for (int i = 0; i < 7; ++i) EXPECT(idx[i] == i);
  EXPECT(oracle_topk_row(s.data(), 0, 3, idx.data()) == 0);
  for (int i = 0; i < 3; ++i) EXPECT(idx[i] == -1);
  EXPECT(oracle_topk_row(s.data(), 5, 0, idx.data()) == -1);
}

}  // namespace

int main() {
  EXPECT(oracle_num_threads() >= 1);
  case_select(3, 4, 2, 64, 17, 5, 1);
  case_select(1, 1, 1, 64, 1, 1, 2);      // one row, one key
  case_select(2, 2, 1, 128, 40, 64, 3);   // k > N: the later step equals the exact pass
  case_select(16, 1, 1, 64, 130, 16, 4);
  case_select(1, 4, 4, 32, 0, 3, 5);      // empty prefix: O = 0, lse = -inf
  case_ties();
  case_depage(2, 16, 8, 53, 6);           // ragged last page
  case_depage(3, 1, 4, 9, 7);
  std::printf("%s: %d failures\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
