// Host side of the C ABI declared in include/mage.h: argument checks, the
// launch plan, the workspace layout, and the two-stream issue order of step 1.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mage.h"
#include "attn_kernels.hpp"
#include "budget_kernels.hpp"
#include "diag_kernels.hpp"
#include "page_kernels.hpp"
#include "select_kernels.hpp"

namespace {

using namespace mage;

thread_local std::string g_last_error;

mage_status fail(mage_status st, const char* what) {
  g_last_error = what;
  return st;
}

mage_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return MAGE_ERR_HIP;
}

// ---- kernel launches and the optional kernel timers -----------------------
// Every launch goes through launch(): it records the kernel's name for
// mage_last_launches and, when the caller armed timers for this call, launches
// through hipExtLaunchKernel so that the armed events mark the kernel's start
// and end on the GPU.
struct LaunchLog {
  hipEvent_t start[MAGE_MAX_TIMED_LAUNCHES];
  hipEvent_t stop[MAGE_MAX_TIMED_LAUNCHES];
  int armed;
  int used;
  const char* names[MAGE_MAX_TIMED_LAUNCHES];
};
thread_local LaunchLog g_launches{};

// Scope of one compute entry point: starts a fresh launch log, disarms on exit.
struct CallScope {
  CallScope() { g_launches.used = 0; }
  ~CallScope() { g_launches.armed = 0; }
};

template <class P>
mage_status launch(const void* kernel, const char* name, int64_t grid, int block, hipStream_t s,
                   P params) {
  if (grid < 1 || grid > 0x7fffffff) return fail(MAGE_ERR_UNSUPPORTED, "launch grid out of range");
  void* args[] = {&params};
  const int i = g_launches.used++;
  if (i < MAGE_MAX_TIMED_LAUNCHES) g_launches.names[i] = name;
  hipError_t e;
  if (i < g_launches.armed)
    e = hipExtLaunchKernel(kernel, dim3(static_cast<unsigned>(grid)), dim3(block), args, 0, s,
                           g_launches.start[i], g_launches.stop[i], 0);
  else
    e = hipLaunchKernel(kernel, dim3(static_cast<unsigned>(grid)), dim3(block), args, 0, s);
  if (e == hipSuccess) e = hipGetLastError();
  return e == hipSuccess ? MAGE_OK : hip_fail(e, name);
}

template <class K>
const void* kfn(K* kernel) {
  return reinterpret_cast<const void*>(kernel);
}

struct Dims {
  int S, B, Hq, Hkv, G, R, D, nrb, units;
  float scale;
  int ng;        // sub-groups the head group runs in (1: not split)
  int gs, g0;    // query-head stride and first head of a sub-group (q_head); 0, 0 when unsplit
  int r_total;   // rows of the whole head group (the score's average)
};

// Sub-group grp of a split head group: G / ng query heads per KV head, at
// most kMaxRows rows, run like an unsplit call.
Dims group_dims(const Dims& d, int grp) {
  Dims g = d;
  g.G = d.G / d.ng;
  g.R = d.B * g.G;
  g.nrb = (g.R + 31) / 32;
  g.ng = 1;
  g.gs = d.G;
  g.g0 = grp * g.G;
  g.r_total = d.R;
  return g;
}

mage_status check_dims(const mage_dims* d, Dims& o) {
  if (!d) return fail(MAGE_ERR_INVALID_ARG, "dims is null");
  if (d->num_seqs < 1 || d->block < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(MAGE_ERR_INVALID_ARG, "num_seqs, block and head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(MAGE_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MAGE_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(std::isfinite(d->scale) && d->scale > 0.f))
    return fail(MAGE_ERR_INVALID_ARG, "scale must be finite and > 0");
  o.S = d->num_seqs;
  o.B = d->block;
  o.Hq = d->num_q_heads;
  o.Hkv = d->num_kv_heads;
  o.G = o.Hq / o.Hkv;
  if (o.B > MAGE_MAX_ROWS) return fail(MAGE_ERR_UNSUPPORTED, "block must be <= 128");
  // more than MAGE_MAX_ROWS rows per KV head: the fewest equal sub-groups of
  // heads that fit (ng = G always does)
  o.ng = 1;
  while (o.G % o.ng != 0 || static_cast<int64_t>(o.B) * (o.G / o.ng) > MAGE_MAX_ROWS) ++o.ng;
  if (static_cast<int64_t>(o.S) * o.Hkv > (1 << 20))
    return fail(MAGE_ERR_UNSUPPORTED, "num_seqs * num_kv_heads must be <= 2^20");
  o.R = o.B * o.G;
  o.D = d->head_dim;
  o.nrb = (o.R + 31) / 32;
  o.units = o.S * o.Hkv;
  o.scale = d->scale;
  o.gs = 0;
  o.g0 = 0;
  o.r_total = o.R;
  return MAGE_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

int env_int(const char* name, int dflt) {
#ifdef MAGE_TUNING
  const char* v = std::getenv(name);
  if (v && *v) return std::atoi(v);
#else
  (void)name;
#endif
  return dflt;
}

// ---- launch plan ----------------------------------------------------------
// Exact pass: split each (seq, KV head) prefix into chunks of `chunk` keys.
// One work-group fills a CU (LDS ring), so the chunk is chosen to make the
// work-group count whole rounds of kCus with at most kExactRoundKeys keys per
// work-group: one round of 4096-key chunks for 8 x 128K keys, two rounds of
// about 6.6K keys for the ragged 8-sequence batch (3.4M keys; against four
// rounds of 3.3K keys: 435 against 453 us and 449 against 451 us in two A/Bs;
// one round of 13K keys: 482 us). Never below the floor that bounds the
// partial-result workspace.
constexpr int kCus = 256;
constexpr int64_t kExactRoundKeys = 8192;
constexpr int kExactMinChunk = 512;
constexpr int kExactSlotBudget = 4096;

int exact_chunk_floor(int64_t units, int64_t max_n) {
  return static_cast<int>(std::max<int64_t>(kExactMinChunk,
                                            round_up(cdiv(units * max_n, kExactSlotBudget), 64)));
}

// Returns 0 when no chunk size satisfies both the workspace floor and the
// per-work-group page table limit (paged layout with tiny pages).
// seq_n: per-sequence prefix lengths (S of them, each repeated for Hkv
// units), or null when every unit has max_n keys. With unequal lengths the
// last chunk of each unit is partial, so the chunk is grown (in steps of 64)
// until the work-group count again fits the whole rounds.
int exact_chunk(int64_t units, int64_t max_n, int64_t total_keys, int page_size, const int32_t* seq_n, int S,
                int Hkv) {
  const int64_t rounds = std::max<int64_t>(1, cdiv(total_keys, kCus * kExactRoundKeys));
  const int64_t target = env_int("MAGE_EXACT_WGS", static_cast<int>(kCus * rounds));
  int64_t c = round_up(cdiv(total_keys, target), 64);
  auto wgs = [&](int64_t chunk) {
    if (!seq_n) return units * cdiv(max_n, chunk);
    int64_t w = 0;
    for (int s = 0; s < S; ++s) w += cdiv(seq_n[s], chunk);
    return w * Hkv;
  };
  while (wgs(c) > target && c < max_n) c += 64;
  const int64_t floor = exact_chunk_floor(units, max_n);
  c = std::max<int64_t>(c, floor);
  const int forced = env_int("MAGE_EXACT_CHUNK", 0);
  if (forced > 0) c = std::max<int64_t>(round_up(forced, 64), floor);
  if (page_size > 0) {
    // the chunk's pages plus the pages of the 64 rows before it
    const int64_t cap = ((kMaxChunkPages - 2 - cdiv(64, page_size)) * static_cast<int64_t>(page_size)) / 64 * 64;
    c = std::min(c, cap);
    if (c < floor || c < 64) return 0;
  }
  return static_cast<int>(c);
}

// Sparse step: work-group = (unit, 32-row block, chunk of the index list);
// chunks are multiples of 4 waves x 32 keys. With enough (unit, row block)
// pairs to fill the chip the index list is not split (one kernel, no merge);
// otherwise it is split into up to kSparseMaxChunks chunks aiming at one
// work-group per CU.
constexpr int kSparseMaxChunks = 32;
constexpr int kSparseChunkUnit = kSparseWaves * kSparseTileKeys;        // 128
constexpr int kSparseMaxChunk = kSparseWaves * kSparseMaxKpw;           // 4096

int sparse_chunk(int64_t units, int nrb, int k) {
  const int min_chunk =
      static_cast<int>(round_up(cdiv(k, kSparseMaxChunks), kSparseChunkUnit));   // <= 4096 for valid k
  const int forced = env_int("MAGE_SPARSE_CHUNK", 0);
  int c;
  if (forced > 0) {
    c = static_cast<int>(round_up(forced, kSparseChunkUnit));
  } else if (k <= 2 * kSparseChunkUnit) {
    // at most two 32-key tiles per wave, both in flight at once: no split
    // beats a split plus its in-launch merge (mha64k, k = 256: 10.4 against
    // 12.0 us with two 128-entry chunks)
    c = static_cast<int>(round_up(k, kSparseChunkUnit));
  } else {
    const int64_t pairs = units * nrb;
    const int64_t want = pairs >= kCus ? 1 : std::min<int64_t>(kSparseMaxChunks, cdiv(kCus, pairs));
    c = static_cast<int>(round_up(cdiv(k, want), kSparseChunkUnit));
  }
  return std::min(kSparseMaxChunk, std::max(min_chunk, c));
}

// LDS ring depth of the exact pass: 3 stages of K+V tiles (3 x 32 KiB at
// d = 128), with the tile loads issued by half the waves, for contiguous and
// paged caches alike. Once the steady loop issued full tiles from fixed
// per-lane offsets (contiguous) or one batch of page-list reads (paged), this
// took the paged ragged batch to 350.7 us, against 361.4 us with every wave
// issuing through a 4-stage ring (359.9 split with 4 stages, 352.2 every wave
// with 3; interleaved A/B, bit-identical); contiguous caches had measured
// 116.4 against 118.4 us at head128k for 3 against 4 stages. The score
// sweep streams K only, through 2 stages (2 x 16 KiB at d = 128): with 48 KiB of LDS per
// work-group three fit on a CU instead of two, which took the sweep from 57.1
// to 54.8 us at head128k, 23.2 to 21.3 at gqa32k and 218.6 to 188.1 us on the
// ragged batch (interleaved A/B; 3 stages: 56.0, 22.1, 217.8).
// Score work-groups per CU: the sweep holds 160 VGPRs (three waves per SIMD)
// and 39 KiB of LDS (46 KiB paged), so three fit. Filling all three with a
// chunk that is any multiple of 64 took the sweep from 58.4 to 56.4 us at
// head128k and 48.4 to 45.9 us at mha64k against power-of-two chunks at two
// per CU (interleaved A/B, bit-identical).
constexpr int kScoreWgsPerCu = 3;
constexpr int kExactStages = 3;
template <int D>
constexpr int kScoreStagesFor = 2;
constexpr int kSparseStages = 2;

// ---- workspace layout ------------------------------------------------------
struct Layout {
  size_t arrivals;       // sparse pass: per (unit, row block) arrival counters; first, at a fixed place
  size_t part_ml, part_o, cand_bits, cand_pos, cand_count, topk_arrivals, hist, scores;
  size_t qbar, qbar_o;   // mean-query selection: the mean query and its (unused) attention output
  size_t page_scores, page_idx;   // page-granular selection (pages of >= 1 positions; <= k page ids)
  size_t total;
  int64_t slots, cand_stride;
};

// Units (sequence, KV head) that a sparse launch can merge in-kernel; larger
// batches fall back to the merge launch.
constexpr int64_t kArrivalUnits = 16384;

Layout make_layout(const Dims& d, int64_t max_n, int64_t k) {
  Layout L{};
  const int64_t U = d.units;
  const int64_t exact_slots = U * cdiv(max_n, exact_chunk_floor(U, max_n));
  // sparse pass: up to kSparseMaxChunks chunks per unit, plus one per unit for
  // per-unit counts (each head's last chunk may be partly empty)
  const int64_t sparse_slots = U * (std::min<int64_t>(kSparseMaxChunks, cdiv(k, kSparseChunkUnit)) + 1);
  L.slots = std::max(exact_slots, sparse_slots);
  const int64_t nchunk = cdiv(max_n, kLocalChunk);
  L.cand_stride = round_up(max_n, kWideChunk);   // room for either candidate chunk
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  // The arrival counters sit at the start of every layout with a fixed
  // capacity, so no other region of any call shape overlaps them: a zeroed
  // workspace keeps them zero through every call.
  L.arrivals = take(kArrivalUnits * (kMaxRows / 32) * 4);
  L.part_ml = take(L.slots * kMaxRows * 2 * 4);
  L.part_o = take(L.slots * 4 * (d.D / 32) * 4 * kWave * 16);
  L.cand_bits = take(U * L.cand_stride * 4);
  L.cand_pos = take(U * L.cand_stride * 4);
  L.cand_count = take(U * nchunk * 4);
  L.topk_arrivals = take(U * 4);
  L.hist = take(U * kHistBins * 4);
  L.scores = take(U * max_n * 4);
  L.qbar = take(U * d.D * 2);
  L.qbar_o = take(U * d.D * 4);
  L.page_scores = take(U * max_n * 4);
  L.page_idx = take(U * k * 4);
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

hipEvent_t internal_event() {
  // one per thread and device: orders the select stream after the merge
  thread_local hipEvent_t ev[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!ev[dev] && hipEventCreateWithFlags(&ev[dev], hipEventDisableTiming) != hipSuccess)
    ev[dev] = nullptr;
  return ev[dev];
}

// ---- common argument bundle of the attention paths -------------------------
struct KvArgs {
  KvSource src;
  SeqLens lens;
  int64_t max_n;
  int64_t total_keys;  // sum over sequences of N_s, times Hkv
};

// Work-group numbering over (unit, chunk) pairs; `grid` receives the number
// of work-groups. Unequal lengths (paged layout) get the dense numbering.
ChunkMap chunk_map(const KvArgs& kv, const Dims& d, int chunk, int64_t& grid) {
  ChunkMap m;
  std::memset(&m, 0, sizeof m);
  if (!kv.src.page_table) {
    grid = d.units * cdiv(kv.max_n, chunk);
    return m;
  }
  m.on = 1;
  int64_t acc = 0;
  for (int s = 0; s < d.S; ++s) {
    m.first[s] = static_cast<int32_t>(acc);
    acc += cdiv(kv.lens.n[s], chunk) * d.Hkv;
  }
  m.first[d.S] = static_cast<int32_t>(acc);
  grid = acc;
  return m;
}

mage_status contiguous_kv(const Dims& d, const uint16_t* k, const uint16_t* v, int32_t n,
                          KvArgs& a) {
  if (!k || !v) return fail(MAGE_ERR_INVALID_ARG, "k_cache / v_cache is null");
  if (!aligned(k, 16) || !aligned(v, 16))
    return fail(MAGE_ERR_INVALID_ARG, "k_cache / v_cache must be 16-byte aligned");
  if (n < 1) return fail(MAGE_ERR_INVALID_ARG, "seq_len must be >= 1");
  a.src = KvSource{k, v, nullptr, 0, 0, n};
  std::memset(&a.lens, 0, sizeof a.lens);
  a.max_n = n;
  a.total_keys = static_cast<int64_t>(n) * d.units;
  return MAGE_OK;
}

mage_status paged_kv(const Dims& d, const mage_paged_kv* kv, KvArgs& a) {
  if (!kv) return fail(MAGE_ERR_INVALID_ARG, "kv is null");
  if (!kv->k_pool || !kv->v_pool || !kv->page_table || !kv->seq_lens)
    return fail(MAGE_ERR_INVALID_ARG, "paged kv has a null pointer");
  if (!aligned(kv->k_pool, 16) || !aligned(kv->v_pool, 16))
    return fail(MAGE_ERR_INVALID_ARG, "k_pool / v_pool must be 16-byte aligned");
  if (d.S > MAGE_MAX_SEQS) return fail(MAGE_ERR_UNSUPPORTED, "num_seqs > MAGE_MAX_SEQS for a paged call");
  const int ps = kv->page_size;
  if (ps < 1 || ps > 1024 || (ps & (ps - 1)))
    return fail(MAGE_ERR_INVALID_ARG, "page_size must be a power of two in [1, 1024]");
  if (kv->max_pages < 1) return fail(MAGE_ERR_INVALID_ARG, "max_pages must be >= 1");
  int shift = 0;
  while ((1 << shift) < ps) ++shift;
  a.src = KvSource{kv->k_pool, kv->v_pool, kv->page_table, kv->max_pages, shift, -1};
  std::memset(&a.lens, 0, sizeof a.lens);
  a.max_n = 0;
  a.total_keys = 0;
  for (int s = 0; s < d.S; ++s) {
    const int32_t n = kv->seq_lens[s];
    if (n < 1 || static_cast<int64_t>(n) > static_cast<int64_t>(kv->max_pages) * ps)
      return fail(MAGE_ERR_INVALID_ARG, "seq_lens[s] must be in [1, max_pages * page_size]");
    a.lens.n[s] = n;
    a.max_n = std::max<int64_t>(a.max_n, n);
    a.total_keys += static_cast<int64_t>(n) * d.Hkv;
  }
  return MAGE_OK;
}

// Sequences [s0, s0 + MAGE_MAX_SEQS) of a call (fewer for the last group).
Dims seq_group(const Dims& d, int s0) {
  Dims g = d;
  g.S = std::min(MAGE_MAX_SEQS, d.S - s0);
  g.units = g.S * d.Hkv;
  return g;
}

// A paged call's per-sequence lengths and chunk numbering travel in the
// kernel arguments, for at most MAGE_MAX_SEQS sequences, so a call over more
// sequences runs as consecutive groups of at most MAGE_MAX_SEQS, in stream
// order on one stream and with the same workspace, each with every
// per-sequence array offset to the group's first sequence s0. Every group is
// checked (check(g, kv)) before the first is launched (run(g, kv, s0)).
template <class Check, class Run>
mage_status paged_groups(const Dims& d, const mage_paged_kv* kvp, Check&& check, Run&& run) {
  if (!kvp) return fail(MAGE_ERR_INVALID_ARG, "kv is null");
  for (int pass = 0; pass < 2; ++pass)
    for (int s0 = 0; s0 < d.S; s0 += MAGE_MAX_SEQS) {
      const Dims g = seq_group(d, s0);
      mage_paged_kv gk = *kvp;
      if (gk.page_table) gk.page_table += static_cast<int64_t>(s0) * kvp->max_pages;
      if (gk.seq_lens) gk.seq_lens += s0;
      KvArgs kv;
      if (mage_status st = paged_kv(g, &gk, kv); st != MAGE_OK) return st;
      if (mage_status st = pass == 0 ? check(g, kv) : run(g, kv, s0); st != MAGE_OK) return st;
    }
  return MAGE_OK;
}

// The longest prefix of a paged call (the row length of its score output);
// only after paged_groups has checked the lengths.
int64_t paged_max_n(const Dims& d, const mage_paged_kv* kvp) {
  int64_t m = 0;
  for (int s = 0; s < d.S; ++s) m = std::max<int64_t>(m, kvp->seq_lens[s]);
  return m;
}

// A selection that ran entirely on attn: the select stream waits for it and
// idx_ready is recorded there, as when the selection runs on that stream.
mage_status join_select(hipStream_t attn, hipStream_t sel, hipEvent_t idx_ready) {
  if (sel && sel != attn) {
    hipEvent_t ev = internal_event();
    if (!ev) return fail(MAGE_ERR_HIP, "could not create the stream-ordering event");
    if (hipError_t e = hipEventRecord(ev, attn); e != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (hipError_t e = hipStreamWaitEvent(sel, ev, 0); e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  } else {
    sel = attn;
  }
  if (idx_ready) {
    if (hipError_t e = hipEventRecord(idx_ready, sel); e != hipSuccess) return hip_fail(e, "hipEventRecord(idx_ready)");
  }
  return MAGE_OK;
}

// Dense (row, chunk) numbering of the candidate pass when row lengths differ
// (tp.n_uniform < 0): seqs groups of tp.rows_per_seq rows.
ChunkMap topk_map(const TopkParams& tp, int seqs) {
  ChunkMap m;
  std::memset(&m, 0, sizeof m);
  if (tp.n_uniform >= 0) return m;
  m.on = 1;
  int64_t acc = 0;
  for (int s = 0; s < seqs; ++s) {
    m.first[s] = static_cast<int32_t>(acc);
    acc += cdiv(tp.lens.n[s], tp.chunk) * tp.rows_per_seq;
  }
  m.first[seqs] = static_cast<int32_t>(acc);
  return m;
}

// Rows longer than this are beyond the final pass's chunk table.
constexpr int64_t kMaxTopkLen = static_cast<int64_t>(kMaxLocalChunks) * kLocalChunk;

// Top-k of tp.rows rows. build_hist: the rows' histograms (and their arrival
// counters) are first zeroed and built from the scores (standalone top-k);
// else the score sweep has built them after the exact pass zeroed them.
mage_status launch_topk(const TopkParams& tp, hipStream_t stream, bool build_hist) {
  const int64_t wgs = tp.map.on ? tp.map.first[tp.rows / tp.rows_per_seq] : static_cast<int64_t>(tp.rows) * tp.nchunk;
  const bool wide_chunk = tp.chunk == kWideChunk;
  if (build_hist) {
    if (mage_status st = launch(kfn(topk_prep_kernel), "topk_prep_kernel", tp.rows, kHistThreads, stream, tp);
        st != MAGE_OK)
      return st;
    if (mage_status st = wide_chunk ? launch(kfn(topk_hist_kernel<kWideChunk>), "topk_hist_kernel", wgs,
                                             kHistThreads, stream, tp)
                                    : launch(kfn(topk_hist_kernel<kLocalChunk>), "topk_hist_kernel", wgs,
                                             kHistThreads, stream, tp);
        st != MAGE_OK)
      return st;
  }
  // the wide final pass for large k: more candidates stay on the register path
  const void* fn = tp.k > kFinalMax / 2
                       ? (wide_chunk ? kfn(topk_select_kernel<kFinalMaxWide, kWideChunk>)
                                     : kfn(topk_select_kernel<kFinalMaxWide, kLocalChunk>))
                       : (wide_chunk ? kfn(topk_select_kernel<kFinalMax, kWideChunk>)
                                     : kfn(topk_select_kernel<kFinalMax, kLocalChunk>));
  return launch(fn, "topk_select_kernel", wgs, kTopkThreads, stream, tp);
}

// The shared fields of a top-k over `rows` rows of the workspace's buffers.
TopkParams topk_params(void* ws, const Layout& L, const float* scores, int64_t stride, int32_t* idx, int32_t k,
                       int32_t rows, int32_t rows_per_seq, int32_t n_uniform, int64_t row_len_max,
                       const SeqLens& lens, int seqs) {
  TopkParams tp{};
  tp.scores = scores;
  tp.stride = stride;
  tp.idx = idx;
  tp.k = k;
  tp.hist = at<uint32_t>(ws, L.hist);
  tp.cand_bits = at<uint32_t>(ws, L.cand_bits);
  tp.cand_pos = at<int32_t>(ws, L.cand_pos);
  // candidate chunks of kLocalChunk positions, or of kWideChunk when those
  // would take more than one round of the CUs (ragged batch: 39.7 -> 29.1 us;
  // at one round the wider chunk was 2.5-3 us slower; interleaved, bit-identical)
  auto chunks = [&](int ch) {
    if (n_uniform >= 0) return static_cast<int64_t>(rows) * cdiv(row_len_max, ch);
    int64_t w = 0;
    for (int s = 0; s < seqs; ++s) w += cdiv(lens.n[s], ch) * rows_per_seq;
    return w;
  };
  tp.chunk = chunks(kLocalChunk) > kCus ? kWideChunk : kLocalChunk;
  tp.nchunk = static_cast<int>(cdiv(row_len_max, tp.chunk));
  tp.cand_stride = static_cast<int64_t>(tp.nchunk) * tp.chunk;
  tp.cand_count = at<int32_t>(ws, L.cand_count);
  tp.arrivals = at<uint32_t>(ws, L.topk_arrivals);
  tp.rows = rows;
  tp.rows_per_seq = rows_per_seq;
  tp.n_uniform = n_uniform;
  tp.lens = lens;
  tp.map = topk_map(tp, seqs);
  return tp;
}

struct PagePlan;
mage_status launch_page_topk(const Dims& d, const KvArgs& kv, const float* scores, int64_t stride,
                             const PagePlan& pp, int32_t* idx, void* ws, const Layout& L, hipStream_t stream);

// Head-adaptive budgets: k_per_head * Hkv positions per sequence; counts [S][Hkv].
struct BudgetPlan {
  int32_t k_per_head;
  int32_t* counts;
};
mage_status launch_budget_topk(const Dims& d, const KvArgs& kv, float* scores, int64_t stride,
                               const BudgetPlan& bp, int32_t* idx, void* ws, const Layout& L, hipStream_t stream);

// Page-granular selection: P positions per page and k_pages pages per row;
// page_idx may be null (then the workspace holds it).
struct PagePlan {
  int32_t page_tokens, k_pages;
  int32_t* page_idx;
};

// k == 0: exact attention only (no score sweep, no top-k). With a page plan,
// k = k_pages * page_tokens and the top-k runs over page scores.
template <int D>
mage_status launch_select(const Dims& d, const uint16_t* q, const KvArgs& kv, int32_t k, float* o,
                          float* lse, int32_t* idx, float* scores, int64_t score_stride, void* ws,
                          const Layout& L, hipStream_t attn, hipStream_t sel, hipEvent_t idx_ready,
                          const PagePlan* pages = nullptr, const BudgetPlan* budget = nullptr,
                          int group_pass = 0) {
  if (d.ng > 1) {
    // A head group of more than kMaxRows rows runs as sub-groups, one after
    // another on attn (each reuses the workspace's partials): every sub-group's
    // exact pass, merge and score sweep, the sweeps adding into one score row
    // per unit; the last one runs the top-k (positions, pages or budgets).
    for (int grp = 0; grp < d.ng; ++grp) {
      const int pass = (grp > 0 ? 1 : 0) | (grp == d.ng - 1 ? 2 : 0);
      if (mage_status st = launch_select<D>(group_dims(d, grp), q, kv, k, o, lse, idx, scores, score_stride, ws, L,
                                            attn, attn, nullptr, pages, budget, pass);
          st != MAGE_OK)
        return st;
    }
    return k > 0 ? join_select(attn, sel, idx_ready) : MAGE_OK;
  }
  // group_pass (sub-groups of a split head group): bit 0 = add to the stored
  // scores, bit 1 = the last sub-group (histogram and top-k); 0 = unsplit
  const bool add_scores = (group_pass & 1) != 0;
  const bool last_group = group_pass == 0 || (group_pass & 2) != 0;
  const int64_t U = d.units;
  const int chunk = exact_chunk(U, kv.max_n, kv.total_keys, kv.src.page_table ? (1 << kv.src.page_shift) : 0,
                                kv.src.page_table ? kv.lens.n : nullptr, d.S, d.Hkv);
  if (chunk == 0) return fail(MAGE_ERR_UNSUPPORTED, "page_size too small for this prefix length");
  if (k > 0 && kv.max_n > kMaxTopkLen) return fail(MAGE_ERR_UNSUPPORTED, "top-k of a prefix longer than 2^25");
  const int nch = static_cast<int>(cdiv(kv.max_n, chunk));
  const float scale_log2 = d.scale * kLog2e;

  AttnParams ap{};
  ap.q = q;
  ap.kv = kv.src;
  ap.idx = nullptr;
  ap.idx_k = 0;
  ap.o = o;
  ap.lse = lse;
  ap.part_o = at<float>(ws, L.part_o);
  ap.part_ml = at<float>(ws, L.part_ml);
  ap.S = d.S; ap.B = d.B; ap.Hq = d.Hq; ap.Hkv = d.Hkv; ap.G = d.G; ap.R = d.R;
  ap.gs = d.gs; ap.g0 = d.g0;
  ap.chunk = chunk;
  ap.nchunk = nch;
  ap.scale_log2 = scale_log2;
  ap.lens = kv.lens;
  int64_t exact_grid = 0;
  ap.map = chunk_map(kv, d, chunk, exact_grid);
  // the main selection adds its score histogram into zeroed rows: chunk 0 of
  // every unit zeroes its row and the row's top-k arrival counter
  const bool main_topk = k > 0 && !pages && !budget;
  ap.zero_hist = main_topk ? at<uint32_t>(ws, L.hist) : nullptr;
  ap.zero_count = main_topk ? at<uint32_t>(ws, L.topk_arrivals) : nullptr;
  // tile loads issued by half the waves through a 3-stage ring, contiguous and paged alike
  const void* exact_fn = kv.src.page_table ? kfn(exact_chunk_kernel<D, kExactStages, true, true>)
                                           : kfn(exact_chunk_kernel<D, kExactStages, true, false>);
#ifdef MAGE_TUNING
  switch (env_int("MAGE_EXACT_MODE", 0)) {   // every wave issues its own slices (4 or 3 stages)
    case 1: exact_fn = kv.src.page_table ? kfn(exact_chunk_kernel<D, 4, false, true>)
                                         : kfn(exact_chunk_kernel<D, 4, false, false>); break;
    case 2: exact_fn = kv.src.page_table ? kfn(exact_chunk_kernel<D, 3, false, true>)
                                         : kfn(exact_chunk_kernel<D, 3, false, false>); break;
    default: break;
  }
#endif
  if (mage_status st = launch(exact_fn, "exact_chunk_kernel", exact_grid, kAttnThreads, attn, ap); st != MAGE_OK)
    return st;

  // The select stream starts right after the exact pass: the score sweep
  // merges the row statistics it needs from the chunk partials itself, so the
  // merge of O below runs on attn_stream beside it.
  if (k > 0 && sel && sel != attn) {
    hipEvent_t ev = internal_event();
    if (!ev) return fail(MAGE_ERR_HIP, "could not create the stream-ordering event");
    if (hipError_t e = hipEventRecord(ev, attn); e != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (hipError_t e = hipStreamWaitEvent(sel, ev, 0); e != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
  } else {
    sel = attn;
  }

  MergeParams mp{};
  mp.part_o = ap.part_o;
  mp.part_ml = ap.part_ml;
  mp.o = o;
  mp.lse = lse;
  mp.S = d.S; mp.B = d.B; mp.Hq = d.Hq; mp.Hkv = d.Hkv; mp.G = d.G; mp.R = d.R; mp.nrb = d.nrb;
  mp.gs = d.gs; mp.g0 = d.g0;
  mp.chunk = chunk;
  mp.nchunk = nch;
  mp.n_uniform = kv.src.page_table ? -1 : kv.src.n_uniform;
  mp.lens = kv.lens;
  if (mage_status st = launch(kfn(exact_merge_kernel<D>), "exact_merge_kernel[exact]",
                              U * d.nrb * (D / 32), kThreads, attn, mp);
      st != MAGE_OK)
    return st;
  if (k == 0) return MAGE_OK;

  ScoreParams sp{};
  sp.q = q;
  sp.kv = kv.src;
  sp.part_ml = ap.part_ml;
  sp.exact_chunk = chunk;
  sp.exact_nchunk = nch;
  sp.hist = main_topk && last_group ? at<uint32_t>(ws, L.hist) : nullptr;
  sp.k = k;
  sp.scores = scores ? scores : at<float>(ws, L.scores);
  sp.stride = scores ? score_stride : kv.max_n;
  sp.S = d.S; sp.B = d.B; sp.Hq = d.Hq; sp.Hkv = d.Hkv; sp.G = d.G; sp.R = d.R;
  sp.gs = d.gs; sp.g0 = d.g0;
  sp.r_total = d.r_total;
  sp.accumulate = add_scores ? 1 : 0;
  // positions per work-group: the smallest multiple of 64 in [kScoreChunkMin,
  // kScoreChunk] whose grid fits kScoreWgsPerCu work-groups per CU, so the
  // sweep runs as one round with every CU holding as many as fit
  {
    int lo = kScoreChunkMin, hi = kScoreChunk;
    const int64_t target = static_cast<int64_t>(env_int("MAGE_SCORE_PER_CU", kScoreWgsPerCu)) * kCus;
    int64_t g = 0;
    chunk_map(kv, d, lo, g);
    if (g <= target) {
      hi = lo;
    } else {
      while (hi - lo > 64) {   // g(lo) > target
        const int mid = (lo + hi) / 2 / 64 * 64;
        chunk_map(kv, d, mid, g);
        (g > target ? lo : hi) = mid;
      }
    }
    sp.chunk = hi;
  }
  sp.nchunk = static_cast<int>(cdiv(kv.max_n, sp.chunk));
  sp.reverse = env_int("MAGE_SCORE_REVERSE", 1);
  sp.scale_log2 = scale_log2;
  sp.lens = kv.lens;
  int64_t score_grid = 0;
  sp.map = chunk_map(kv, d, sp.chunk, score_grid);
  const void* score_fn = kv.src.page_table ? kfn(score_kernel<D, kScoreStagesFor<D>, true>)
                                            : kfn(score_kernel<D, kScoreStagesFor<D>, false>);
  if (mage_status st = launch(score_fn, "score_kernel", score_grid, kThreads, sel, sp); st != MAGE_OK)
    return st;
  if (!last_group) return MAGE_OK;
  if (main_topk) {
    const TopkParams tp = topk_params(ws, L, sp.scores, sp.stride, idx, k, static_cast<int32_t>(U), d.Hkv,
                                      kv.src.page_table ? -1 : kv.src.n_uniform, kv.max_n, kv.lens, d.S);
    if (mage_status st = launch_topk(tp, sel, false); st != MAGE_OK) return st;
  } else {
    mage_status st = pages ? launch_page_topk(d, kv, sp.scores, sp.stride, *pages, idx, ws, L, sel)
                           : launch_budget_topk(d, kv, sp.scores, sp.stride, *budget, idx, ws, L, sel);
    if (st != MAGE_OK) return st;
  }
  if (idx_ready) {
    if (hipError_t e = hipEventRecord(idx_ready, sel); e != hipSuccess)
      return hip_fail(e, "hipEventRecord(idx_ready)");
  }
  return MAGE_OK;
}

// One top-k per sequence over its Hkv score rows taken as one row (entry
// h * stride + p), then the split into per-head rows and counts.
mage_status launch_budget_topk(const Dims& d, const KvArgs& kv, float* scores, int64_t stride,
                               const BudgetPlan& bp, int32_t* idx, void* ws, const Layout& L, hipStream_t stream) {
  const bool ragged = kv.src.page_table != nullptr;
  const int64_t row_len = stride * d.Hkv;
  if (row_len > kMaxTopkLen) return fail(MAGE_ERR_UNSUPPORTED, "num_kv_heads * prefix length must be <= 2^25");
  if (ragged) {
    GapZeroParams gz{};
    gz.scores = scores;
    gz.stride = stride;
    gz.rows = d.units;
    gz.rows_per_seq = d.Hkv;
    gz.lens = kv.lens;
    if (mage_status st = launch(kfn(gap_zero_kernel), "gap_zero_kernel", d.units, 256, stream, gz); st != MAGE_OK)
      return st;
  }
  const int32_t K = bp.k_per_head * d.Hkv;
  int32_t* gidx = at<int32_t>(ws, L.page_idx);   // [S][K]
  SeqLens none;
  std::memset(&none, 0, sizeof none);
  const TopkParams tp = topk_params(ws, L, scores, row_len, gidx, K, d.S, 1, static_cast<int32_t>(row_len),
                                    row_len, none, d.S);
  if (mage_status st = launch_topk(tp, stream, true); st != MAGE_OK) return st;
  BudgetSplitParams bs{};
  bs.gidx = gidx;
  bs.idx = idx;
  bs.counts = bp.counts;
  bs.stride = stride;
  bs.S = d.S;
  bs.Hkv = d.Hkv;
  bs.K = K;
  bs.n_uniform = ragged ? -1 : kv.src.n_uniform;
  bs.lens = kv.lens;
  return launch(kfn(budget_split_kernel), "budget_split_kernel", d.units, 256, stream, bs);
}

// Page scores, the top k_pages pages of every row (the standalone top-k path
// over the page scores) and their expansion into positions.
mage_status launch_page_topk(const Dims& d, const KvArgs& kv, const float* scores, int64_t stride,
                             const PagePlan& pp, int32_t* idx, void* ws, const Layout& L, hipStream_t stream) {
  const bool ragged = kv.src.page_table != nullptr;
  const int P = pp.page_tokens;
  const int64_t pages_max = cdiv(kv.max_n, P);
  SeqLens plens;
  std::memset(&plens, 0, sizeof plens);
  if (ragged)
    for (int s = 0; s < d.S; ++s) plens.n[s] = static_cast<int32_t>(cdiv(kv.lens.n[s], P));
  PageSumParams ps{};
  ps.scores = scores;
  ps.stride = stride;
  ps.page_scores = at<float>(ws, L.page_scores);
  ps.pstride = pages_max;
  ps.rows = d.units;
  ps.rows_per_seq = d.Hkv;
  ps.n_uniform = ragged ? -1 : kv.src.n_uniform;
  ps.page_tokens = P;
  ps.pages_max = static_cast<int32_t>(pages_max);
  ps.vec4 = P % 4 == 0 && stride % 4 == 0 && aligned(scores, 16);
  ps.lens = kv.lens;
  if (mage_status st = launch(kfn(page_sum_kernel), "page_sum_kernel", cdiv(d.units * pages_max, 256), 256,
                              stream, ps);
      st != MAGE_OK)
    return st;
  int32_t* page_idx = pp.page_idx ? pp.page_idx : at<int32_t>(ws, L.page_idx);
  const TopkParams tp = topk_params(ws, L, ps.page_scores, pages_max, page_idx, pp.k_pages, d.units, d.Hkv,
                                    ragged ? -1 : static_cast<int32_t>(pages_max), pages_max, plens, d.S);
  if (mage_status st = launch_topk(tp, stream, true); st != MAGE_OK) return st;
  PageExpandParams pe{};
  pe.page_idx = page_idx;
  pe.idx = idx;
  pe.rows = d.units;
  pe.rows_per_seq = d.Hkv;
  pe.n_uniform = ragged ? -1 : kv.src.n_uniform;
  pe.k_pages = pp.k_pages;
  pe.page_tokens = P;
  pe.lens = kv.lens;
  return launch(kfn(page_expand_kernel), "page_expand_kernel",
                cdiv(static_cast<int64_t>(d.units) * pp.k_pages * P, 256), 256, stream, pe);
}

template <int D>
mage_status launch_sparse(const Dims& d, const uint16_t* q, const KvArgs& kv, const int32_t* idx,
                          int32_t k, float* o, float* lse, void* ws, const Layout& L,
                          hipStream_t stream, const uint16_t* k_blk = nullptr,
                          const uint16_t* v_blk = nullptr, const int32_t* counts = nullptr, int32_t k_seq = 0) {
  if (d.ng > 1) {
    // a head group of more than kMaxRows rows: one launch per sub-group (in
    // stream order, each reusing the workspace), each with the KV head's
    // block rows and counts
    for (int grp = 0; grp < d.ng; ++grp)
      if (mage_status st = launch_sparse<D>(group_dims(d, grp), q, kv, idx, k, o, lse, ws, L, stream, k_blk, v_blk,
                                            counts, k_seq);
          st != MAGE_OK)
        return st;
    return MAGE_OK;
  }
  const int64_t U = d.units;
  int chunk = sparse_chunk(U, d.nrb, counts ? std::max(1, k_seq / d.Hkv) : k);
  int64_t seq_slots = 0;
  if (counts) {
    // per-unit counts: a sequence's chunks are numbered densely; its heads
    // hold at most k_seq entries, so cdiv(k_seq, chunk) + Hkv slots suffice.
    // The chunk doubles until the grid fits one round of the CUs, but not past
    // the average entries per head (a larger chunk hands a long head's entries
    // to one work-group); it grows further only if the workspace needs it. A
    // unit whose entries fit one chunk writes O itself.
    auto slots_for = [&](int ch) { return cdiv(k_seq, ch) + d.Hkv; };
    const int64_t avg = round_up(cdiv(k_seq, d.Hkv), kSparseChunkUnit);
    while (chunk < kSparseMaxChunk && 2 * chunk <= avg && d.S * slots_for(chunk) * d.nrb > kCus)
      chunk = std::min(kSparseMaxChunk, 2 * chunk);
    while (chunk < kSparseMaxChunk && d.S * slots_for(chunk) > L.slots) chunk = std::min(kSparseMaxChunk, 2 * chunk);
    if (d.S * slots_for(chunk) > L.slots) return fail(MAGE_ERR_UNSUPPORTED, "workspace plan too small for k_seq");
    seq_slots = slots_for(chunk);
  }
  const int nch = static_cast<int>(cdiv(k, chunk));   // block rows, if any, ride in the last chunk
  if (!counts && nch > 1 && U * nch > L.slots) return fail(MAGE_ERR_UNSUPPORTED, "workspace plan too small for the split");
  AttnParams ap{};
  ap.q = q;
  ap.kv = kv.src;
  ap.idx = idx;
  ap.idx_k = k;
  ap.o = o;
  ap.lse = lse;
  ap.part_o = at<float>(ws, L.part_o);
  ap.part_ml = at<float>(ws, L.part_ml);
  ap.S = d.S; ap.B = d.B; ap.Hq = d.Hq; ap.Hkv = d.Hkv; ap.G = d.G; ap.R = d.R;
  ap.gs = d.gs; ap.g0 = d.g0;
  ap.chunk = chunk;
  ap.nchunk = nch;
  ap.scale_log2 = d.scale * kLog2e;
  ap.lens = kv.lens;
  ap.k_blk = k_blk;
  ap.v_blk = v_blk;
  ap.counts = counts;
  ap.seq_slots = static_cast<int32_t>(seq_slots);
  // uniform chunks: the last work-group of each (unit, row block) merges its
  // chunks inside the launch (arrival counters); per-unit counts keep the
  // merge launch
  const bool handoff = !counts && nch > 1 && U <= kArrivalUnits && env_int("MAGE_SPARSE_HANDOFF", 1) != 0;
  ap.arrivals = handoff ? at<uint32_t>(ws, L.arrivals) : nullptr;
  const int64_t grid = round_up(counts ? d.S * seq_slots : U * nch, 8) * d.nrb;
  if (mage_status st = launch(kfn(sparse_attn_kernel<D, kSparseStages>), "sparse_attn_kernel", grid,
                              kSparseThreads, stream, ap);
      st != MAGE_OK)
    return st;
  if ((nch == 1 && !counts) || handoff) return MAGE_OK;  // O and lse written by the launch
  MergeParams mp{};
  mp.part_o = ap.part_o;
  mp.part_ml = ap.part_ml;
  mp.o = o;
  mp.lse = lse;
  mp.S = d.S; mp.B = d.B; mp.Hq = d.Hq; mp.Hkv = d.Hkv; mp.G = d.G; mp.R = d.R; mp.nrb = d.nrb;
  mp.gs = d.gs; mp.g0 = d.g0;
  mp.chunk = chunk;
  mp.nchunk = nch;
  mp.n_uniform = k;  // every unit has k index entries (per-unit counts: at most k)
  mp.counts = counts;
  mp.seq_slots = static_cast<int32_t>(seq_slots);
  std::memset(&mp.lens, 0, sizeof mp.lens);
  return launch(kfn(exact_merge_kernel<D>), "exact_merge_kernel[sparse]", U * d.nrb * (D / 32),
                kThreads, stream, mp);
}

// Selection by the probability under the block's mean query: the mean query
// (one bf16 row per KV head) goes through the step-1 selection as a block of
// one token with one query head per KV head. Its attention output lands in
// the workspace and is not used.
template <int D>
mage_status launch_mean_query_select(const Dims& d, const uint16_t* q, const KvArgs& kv, int32_t k,
                                     int32_t* idx, float* scores, int64_t score_stride, void* ws,
                                     const Layout& L, hipStream_t stream) {
  MeanQueryParams mq{};
  mq.q = q;
  mq.qbar = at<uint16_t>(ws, L.qbar);
  mq.S = d.S; mq.B = d.B; mq.Hq = d.Hq; mq.Hkv = d.Hkv; mq.G = d.G; mq.D = D;
  if (mage_status st = launch(kfn(mean_query_kernel), "mean_query_kernel",
                              cdiv(static_cast<int64_t>(d.units) * D, 256), 256, stream, mq);
      st != MAGE_OK)
    return st;
  Dims d1 = d;
  d1.B = 1;
  d1.Hq = d.Hkv;
  d1.G = 1;
  d1.R = 1;
  d1.nrb = 1;
  d1.r_total = 1;
  d1.ng = 1;   // one row per KV head, whatever the block's head group
  d1.gs = 0;
  d1.g0 = 0;
  return launch_select<D>(d1, mq.qbar, kv, k, at<float>(ws, L.qbar_o), nullptr, idx, scores, score_stride,
                          ws, L, stream, nullptr, nullptr);
}

mage_status check_ws(void* ws, size_t bytes, const Layout& L) {
  if (!ws) return fail(MAGE_ERR_INVALID_ARG, "workspace is null");
  if (!aligned(ws, 256)) return fail(MAGE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (bytes < L.total) return fail(MAGE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  return MAGE_OK;
}

mage_status common_select_checks(const uint16_t* q, int32_t k, float* o, float* lse, int32_t* idx,
                                 float* scores) {
  if (!q || !o || !idx) return fail(MAGE_ERR_INVALID_ARG, "q, o and idx must not be null");
  if (!aligned(q, 16) || !aligned(o, 16)) return fail(MAGE_ERR_INVALID_ARG, "q and o must be 16-byte aligned");
  if (!aligned(idx, 4) || (lse && !aligned(lse, 4)) || (scores && !aligned(scores, 4)))
    return fail(MAGE_ERR_INVALID_ARG, "idx, lse and scores must be 4-byte aligned");
  if (k < 1) return fail(MAGE_ERR_INVALID_ARG, "k must be >= 1");
  return MAGE_OK;
}

__global__ void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Number of non-zero words among the first `words` of p, written to *out (one
// work-group: no cross-group accumulation, no atomics).
constexpr int kCheckThreads = 1024;
__global__ __launch_bounds__(kCheckThreads) void count_nonzero_kernel(const uint32_t* p, int32_t words,
                                                                       int32_t* out) {
  __shared__ int32_t s_part[kCheckThreads / kWave];
  int32_t n = 0;
  for (int32_t i = threadIdx.x; i < words; i += kCheckThreads) n += p[i] != 0u;
  n = static_cast<int32_t>(sum_over_rows(static_cast<uint32_t>(n)));   // 4 rows of 16 lanes
  for (int off = 1; off < 16; off <<= 1) n += __shfl_xor(n, off, 16);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int w = 0; w < kCheckThreads / kWave; ++w) t += s_part[w];
    *out = t;
  }
}

// ---- the allocation-free later step -----------------------------------------
// mage_sparse_attn_noalloc keeps its scratch (the arrival counters, then the
// split partials, in the workspace layout of the later step) in this
// file-scope array: one copy per GPU, held until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in); it passes the device address that hipGetSymbolAddress returns,
// kept per device.
constexpr size_t kScratchCounterBytes = kArrivalUnits * (kMaxRows / 32) * 4;   // 256 KiB
constexpr size_t kScratchBytes = kScratchCounterBytes + (size_t(8) << 20);    // + 8 MiB of partials
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The scratch's device address on the current device. The first call on a
// device looks it up (with that device current) and zeroes its counters with
// a fill kernel on `stream` (the array starts zeroed when the code object is
// loaded; every call leaves the counters at zero again).
mage_status scratch_on_device(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MAGE_ERR_UNSUPPORTED, "device index beyond the scratch table");
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (slot.err != hipSuccess) return;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(cdiv(kScratchCounterBytes / 4, 256))),
                       dim3(256), 0, stream, static_cast<uint32_t*>(p), kScratchCounterBytes / 4);
    slot.err = hipGetLastError();
    if (slot.err == hipSuccess) slot.ptr = p;
  });
  if (slot.err != hipSuccess) return hip_fail(slot.err, "scratch set-up (hipGetSymbolAddress / zero fill)");
  *out = slot.ptr;
  return MAGE_OK;
}

// head-dimension dispatch of the launch plans
template <class... A>
mage_status select_d(const Dims& d, A&&... a) {
  return d.D == 128 ? launch_select<128>(d, a...) : launch_select<64>(d, a...);
}
template <class... A>
mage_status sparse_d(const Dims& d, A&&... a) {
  return d.D == 128 ? launch_sparse<128>(d, a...) : launch_sparse<64>(d, a...);
}

}  // namespace

extern "C" {

size_t mage_workspace_bytes(const mage_dims* dims, int32_t max_seq_len, int32_t k) {
  Dims d;
  if (check_dims(dims, d) != MAGE_OK || max_seq_len < 1 || k < 1) return 0;
  // also enough for a paged call's groups of MAGE_MAX_SEQS sequences
  size_t t = make_layout(d, max_seq_len, k).total;
  for (int s0 = 0; s0 < d.S; s0 += MAGE_MAX_SEQS) t = std::max(t, make_layout(seq_group(d, s0), max_seq_len, k).total);
  return t;
}

mage_status mage_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || !aligned(workspace, 4) || workspace_bytes % 4)
    return fail(MAGE_ERR_INVALID_ARG, "workspace must be non-null, 4-byte aligned, a multiple of 4 bytes");
  const size_t words = workspace_bytes / 4;
  if (words == 0) return MAGE_OK;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>(4096, cdiv(words, 256)));
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(workspace), words);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_fail(e, "workspace init launch");
  return MAGE_OK;
}

mage_status mage_workspace_check(const void* workspace, size_t workspace_bytes, int32_t* nonzero,
                                 hipStream_t stream) {
  if (!workspace || !nonzero || !aligned(workspace, 4) || !aligned(nonzero, 4))
    return fail(MAGE_ERR_INVALID_ARG, "workspace and nonzero must be non-null and 4-byte aligned");
  const size_t counter_bytes = kArrivalUnits * (kMaxRows / 32) * 4;
  if (workspace_bytes < counter_bytes)
    return fail(MAGE_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than its arrival-counter region");
  hipLaunchKernelGGL(count_nonzero_kernel, dim3(1), dim3(kCheckThreads), 0, stream,
                     static_cast<const uint32_t*>(workspace), static_cast<int32_t>(counter_bytes / 4), nonzero);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return hip_fail(e, "workspace check launch");
  return MAGE_OK;
}

mage_status mage_select_exact(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                              const uint16_t* v_cache, int32_t seq_len, int32_t k, float* o,
                              float* lse, int32_t* idx, float* scores, void* workspace,
                              size_t workspace_bytes, hipStream_t attn_stream,
                              hipStream_t select_stream, hipEvent_t idx_ready) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = common_select_checks(q, k, o, lse, idx, scores); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const Layout L = make_layout(d, kv.max_n, k);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  return d.D == 128 ? launch_select<128>(d, q, kv, k, o, lse, idx, scores, seq_len, workspace, L,
                                         attn_stream, select_stream, idx_ready)
                    : launch_select<64>(d, q, kv, k, o, lse, idx, scores, seq_len, workspace, L,
                                        attn_stream, select_stream, idx_ready);
}

mage_status mage_select_exact_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                    int32_t k, float* o, float* lse, int32_t* idx, float* scores,
                                    void* workspace, size_t workspace_bytes, hipStream_t attn_stream,
                                    hipStream_t select_stream, hipEvent_t idx_ready) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = common_select_checks(q, k, o, lse, idx, scores); st != MAGE_OK) return st;
  const bool grouped = d.S > MAGE_MAX_SEQS;
  int64_t stride = 0;
  mage_status st = paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, k)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        if (stride == 0) stride = paged_max_n(d, kvp);
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        return select_d(g, q + sq * d.D, kv, k, o + sq * d.D, lse ? lse + sq : nullptr, idx + su * k,
                        scores ? scores + su * stride : nullptr, stride, workspace, make_layout(g, kv.max_n, k),
                        attn_stream, grouped ? attn_stream : select_stream, grouped ? nullptr : idx_ready);
      });
  if (st != MAGE_OK || !grouped) return st;
  return join_select(attn_stream, select_stream, idx_ready);
}

mage_status mage_exact_attn(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, int32_t seq_len, float* o, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  int32_t dummy_idx = 0;
  if (mage_status st = common_select_checks(q, 1, o, lse, &dummy_idx, nullptr); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const Layout L = make_layout(d, kv.max_n, 1);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  return d.D == 128 ? launch_select<128>(d, q, kv, 0, o, lse, nullptr, nullptr, 0, workspace, L,
                                         stream, nullptr, nullptr)
                    : launch_select<64>(d, q, kv, 0, o, lse, nullptr, nullptr, 0, workspace, L,
                                        stream, nullptr, nullptr);
}

mage_status mage_exact_attn_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                  float* o, float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  int32_t dummy_idx = 0;
  if (mage_status st = common_select_checks(q, 1, o, lse, &dummy_idx, nullptr); st != MAGE_OK) return st;
  return paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, 1)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq;
        return select_d(g, q + sq * d.D, kv, 0, o + sq * d.D, lse ? lse + sq : nullptr, nullptr, nullptr, 0,
                        workspace, make_layout(g, kv.max_n, 1), stream, nullptr, nullptr);
      });
}

static mage_status mean_query_checks(const uint16_t* q, int32_t k, int32_t* idx, float* scores) {
  if (!q || !idx) return fail(MAGE_ERR_INVALID_ARG, "q and idx must not be null");
  if (!aligned(q, 16)) return fail(MAGE_ERR_INVALID_ARG, "q must be 16-byte aligned");
  if (!aligned(idx, 4) || (scores && !aligned(scores, 4)))
    return fail(MAGE_ERR_INVALID_ARG, "idx and scores must be 4-byte aligned");
  if (k < 1) return fail(MAGE_ERR_INVALID_ARG, "k must be >= 1");
  return MAGE_OK;
}

mage_status mage_select_mean_query(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int32_t seq_len, int32_t k, int32_t* idx,
                                   float* scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = mean_query_checks(q, k, idx, scores); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const Layout L = make_layout(d, kv.max_n, k);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  return d.D == 128 ? launch_mean_query_select<128>(d, q, kv, k, idx, scores, seq_len, workspace, L, stream)
                    : launch_mean_query_select<64>(d, q, kv, k, idx, scores, seq_len, workspace, L, stream);
}

mage_status mage_select_mean_query_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                         int32_t k, int32_t* idx, float* scores, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = mean_query_checks(q, k, idx, scores); st != MAGE_OK) return st;
  int64_t stride = 0;
  return paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, k)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        if (stride == 0) stride = paged_max_n(d, kvp);
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        const Layout L = make_layout(g, kv.max_n, k);
        float* sc = scores ? scores + su * stride : nullptr;
        return d.D == 128
                   ? launch_mean_query_select<128>(g, q + sq * d.D, kv, k, idx + su * k, sc, stride, workspace, L, stream)
                   : launch_mean_query_select<64>(g, q + sq * d.D, kv, k, idx + su * k, sc, stride, workspace, L, stream);
      });
}

static mage_status page_checks(const uint16_t* q, int32_t page_tokens, int32_t k_pages, float* o, float* lse,
                               int32_t* idx, int32_t* page_idx, float* scores) {
  if (page_tokens < 1 || page_tokens > 4096) return fail(MAGE_ERR_INVALID_ARG, "page_tokens must be in [1, 4096]");
  if (k_pages < 1) return fail(MAGE_ERR_INVALID_ARG, "k_pages must be >= 1");
  if (static_cast<int64_t>(k_pages) * page_tokens > MAGE_MAX_SPARSE_K)
    return fail(MAGE_ERR_UNSUPPORTED, "k_pages * page_tokens must be <= MAGE_MAX_SPARSE_K");
  if (page_idx && !aligned(page_idx, 4)) return fail(MAGE_ERR_INVALID_ARG, "page_idx must be 4-byte aligned");
  return common_select_checks(q, k_pages * page_tokens, o, lse, idx, scores);
}

mage_status mage_select_pages(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                              const uint16_t* v_cache, int32_t seq_len, int32_t page_tokens, int32_t k_pages,
                              float* o, float* lse, int32_t* idx, int32_t* page_idx, float* scores,
                              void* workspace, size_t workspace_bytes, hipStream_t attn_stream,
                              hipStream_t select_stream, hipEvent_t idx_ready) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = page_checks(q, page_tokens, k_pages, o, lse, idx, page_idx, scores); st != MAGE_OK)
    return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const int32_t k = k_pages * page_tokens;
  const Layout L = make_layout(d, kv.max_n, k);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  const PagePlan pp{page_tokens, k_pages, page_idx};
  return d.D == 128 ? launch_select<128>(d, q, kv, k, o, lse, idx, scores, seq_len, workspace, L, attn_stream,
                                         select_stream, idx_ready, &pp)
                    : launch_select<64>(d, q, kv, k, o, lse, idx, scores, seq_len, workspace, L, attn_stream,
                                        select_stream, idx_ready, &pp);
}

mage_status mage_select_pages_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                    int32_t page_tokens, int32_t k_pages, float* o, float* lse, int32_t* idx,
                                    int32_t* page_idx, float* scores, void* workspace, size_t workspace_bytes,
                                    hipStream_t attn_stream, hipStream_t select_stream, hipEvent_t idx_ready) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = page_checks(q, page_tokens, k_pages, o, lse, idx, page_idx, scores); st != MAGE_OK)
    return st;
  const int32_t k = k_pages * page_tokens;
  const bool grouped = d.S > MAGE_MAX_SEQS;
  int64_t stride = 0;
  mage_status st = paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, k)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        if (stride == 0) stride = paged_max_n(d, kvp);
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        const PagePlan pp{page_tokens, k_pages, page_idx ? page_idx + su * k_pages : nullptr};
        return select_d(g, q + sq * d.D, kv, k, o + sq * d.D, lse ? lse + sq : nullptr, idx + su * k,
                        scores ? scores + su * stride : nullptr, stride, workspace, make_layout(g, kv.max_n, k),
                        attn_stream, grouped ? attn_stream : select_stream, grouped ? nullptr : idx_ready, &pp);
      });
  if (st != MAGE_OK || !grouped) return st;
  return join_select(attn_stream, select_stream, idx_ready);
}

mage_status mage_select_adaptive(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, int32_t seq_len, int32_t k, float* o, float* lse,
                                 int32_t* idx, int32_t* counts, void* workspace, size_t workspace_bytes,
                                 hipStream_t attn_stream, hipStream_t select_stream, hipEvent_t idx_ready) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = common_select_checks(q, k, o, lse, idx, nullptr); st != MAGE_OK) return st;
  if (!counts || !aligned(counts, 4)) return fail(MAGE_ERR_INVALID_ARG, "counts must be non-null and 4-byte aligned");
  if (static_cast<int64_t>(k) * d.Hkv > MAGE_MAX_SPARSE_K)
    return fail(MAGE_ERR_UNSUPPORTED, "k * num_kv_heads must be <= MAGE_MAX_SPARSE_K");
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const int32_t K = k * d.Hkv;
  const Layout L = make_layout(d, kv.max_n, K);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  const BudgetPlan bp{k, counts};
  return d.D == 128 ? launch_select<128>(d, q, kv, K, o, lse, idx, nullptr, 0, workspace, L, attn_stream,
                                         select_stream, idx_ready, nullptr, &bp)
                    : launch_select<64>(d, q, kv, K, o, lse, idx, nullptr, 0, workspace, L, attn_stream,
                                        select_stream, idx_ready, nullptr, &bp);
}

mage_status mage_select_adaptive_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                       int32_t k, float* o, float* lse, int32_t* idx, int32_t* counts,
                                       void* workspace, size_t workspace_bytes, hipStream_t attn_stream,
                                       hipStream_t select_stream, hipEvent_t idx_ready) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (mage_status st = common_select_checks(q, k, o, lse, idx, nullptr); st != MAGE_OK) return st;
  if (!counts || !aligned(counts, 4)) return fail(MAGE_ERR_INVALID_ARG, "counts must be non-null and 4-byte aligned");
  if (static_cast<int64_t>(k) * d.Hkv > MAGE_MAX_SPARSE_K)
    return fail(MAGE_ERR_UNSUPPORTED, "k * num_kv_heads must be <= MAGE_MAX_SPARSE_K");
  const int32_t K = k * d.Hkv;
  const bool grouped = d.S > MAGE_MAX_SEQS;
  mage_status st = paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, K)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        const BudgetPlan bp{k, counts + su};
        return select_d(g, q + sq * d.D, kv, K, o + sq * d.D, lse ? lse + sq : nullptr, idx + su * K, nullptr, 0,
                        workspace, make_layout(g, kv.max_n, K), attn_stream,
                        grouped ? attn_stream : select_stream, grouped ? nullptr : idx_ready, nullptr, &bp);
      });
  if (st != MAGE_OK || !grouped) return st;
  return join_select(attn_stream, select_stream, idx_ready);
}

mage_status mage_mean_query(const mage_dims* dims, const uint16_t* q, uint16_t* qbar, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (!q || !qbar) return fail(MAGE_ERR_INVALID_ARG, "q and qbar must not be null");
  if (!aligned(q, 2) || !aligned(qbar, 2)) return fail(MAGE_ERR_INVALID_ARG, "q and qbar must be 2-byte aligned");
  MeanQueryParams mq{};
  mq.q = q;
  mq.qbar = qbar;
  mq.S = d.S; mq.B = d.B; mq.Hq = d.Hq; mq.Hkv = d.Hkv; mq.G = d.G; mq.D = d.D;
  return launch(kfn(mean_query_kernel), "mean_query_kernel", cdiv(static_cast<int64_t>(d.units) * d.D, 256),
                256, stream, mq);
}

mage_status mage_idx_overlap(int32_t rows, int32_t k, const int32_t* a, const int32_t* b, int32_t* common,
                             int32_t* count_a, int32_t* count_b, hipStream_t stream) {
  CallScope scope;
  if (rows < 1 || k < 1) return fail(MAGE_ERR_INVALID_ARG, "rows and k must be >= 1");
  if (!a || !b || !common) return fail(MAGE_ERR_INVALID_ARG, "a, b and common must not be null");
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(common, 4) || (count_a && !aligned(count_a, 4)) ||
      (count_b && !aligned(count_b, 4)))
    return fail(MAGE_ERR_INVALID_ARG, "index and count arrays must be 4-byte aligned");
  OverlapParams op{a, b, common, count_a, count_b, rows, k};
  return launch(kfn(idx_overlap_kernel), "idx_overlap_kernel", rows, kOverlapThreads, stream, op);
}

static mage_status sparse_common(const mage_dims* dims, const uint16_t* q, const int32_t* idx,
                                 int32_t k, float* o, float* lse, Dims& d) {
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (!q || !o || !idx) return fail(MAGE_ERR_INVALID_ARG, "q, o and idx must not be null");
  if (!aligned(q, 16) || !aligned(o, 16)) return fail(MAGE_ERR_INVALID_ARG, "q and o must be 16-byte aligned");
  if (!aligned(idx, 4) || (lse && !aligned(lse, 4)))
    return fail(MAGE_ERR_INVALID_ARG, "idx and lse must be 4-byte aligned");
  if (k < 1) return fail(MAGE_ERR_INVALID_ARG, "k must be >= 1");
  static_assert(MAGE_MAX_SPARSE_K <= kSparseMaxChunks * kSparseMaxChunk, "sparse plan limit");
  if (k > MAGE_MAX_SPARSE_K)
    return fail(MAGE_ERR_UNSUPPORTED, "sparse steps take k <= MAGE_MAX_SPARSE_K index entries");
  return MAGE_OK;
}

mage_status mage_sparse_attn(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                             const uint16_t* v_cache, int32_t seq_len, const int32_t* idx, int32_t k,
                             float* o, float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k, o, lse, d); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const Layout L = make_layout(d, kv.max_n, k);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  return d.D == 128 ? launch_sparse<128>(d, q, kv, idx, k, o, lse, workspace, L, stream)
                    : launch_sparse<64>(d, q, kv, idx, k, o, lse, workspace, L, stream);
}

mage_status mage_sparse_attn_noalloc(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                                     const uint16_t* v_cache, int32_t seq_len, const int32_t* idx, int32_t k,
                                     float* o, float* lse, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k, o, lse, d); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  // the later step's part of the workspace layout, sized for this call's plan
  // (that of each sub-group when the head group is split)
  const Dims g0 = d.ng > 1 ? group_dims(d, 0) : d;
  const int64_t nch = cdiv(k, sparse_chunk(g0.units, g0.nrb, k));
  Layout L{};
  L.slots = nch > 1 ? d.units * nch : 0;
  L.arrivals = 0;
  L.part_ml = round_up(kScratchCounterBytes, 256);
  L.part_o = round_up(L.part_ml + L.slots * kMaxRows * 2 * 4, 256);
  L.total = L.part_o + L.slots * 4 * (d.D / 32) * 4 * kWave * 16;
  if (L.total > kScratchBytes)
    return fail(MAGE_ERR_UNSUPPORTED, "this later step's split partials exceed the fixed scratch (8 MiB)");
  void* ws = nullptr;
  if (mage_status st = scratch_on_device(stream, &ws); st != MAGE_OK) return st;
  return d.D == 128 ? launch_sparse<128>(d, q, kv, idx, k, o, lse, ws, L, stream)
                    : launch_sparse<64>(d, q, kv, idx, k, o, lse, ws, L, stream);
}

mage_status mage_sparse_attn_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                   const int32_t* idx, int32_t k, float* o, float* lse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k, o, lse, d); st != MAGE_OK) return st;
  return paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, k)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        return sparse_d(g, q + sq * d.D, kv, idx + su * k, k, o + sq * d.D, lse ? lse + sq : nullptr, workspace,
                        make_layout(g, kv.max_n, k), stream);
      });
}

static mage_status block_rows_checks(const uint16_t* k_blk, const uint16_t* v_blk) {
  if (!k_blk || !v_blk) return fail(MAGE_ERR_INVALID_ARG, "k_blk and v_blk must not be null");
  if (!aligned(k_blk, 16) || !aligned(v_blk, 16))
    return fail(MAGE_ERR_INVALID_ARG, "k_blk and v_blk must be 16-byte aligned");
  return MAGE_OK;
}

mage_status mage_sparse_block_attn(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int32_t seq_len, const int32_t* idx, int32_t k,
                                   const uint16_t* k_blk, const uint16_t* v_blk, float* o, float* lse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k, o, lse, d); st != MAGE_OK) return st;
  if (mage_status st = block_rows_checks(k_blk, v_blk); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const Layout L = make_layout(d, kv.max_n, k);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  return d.D == 128 ? launch_sparse<128>(d, q, kv, idx, k, o, lse, workspace, L, stream, k_blk, v_blk)
                    : launch_sparse<64>(d, q, kv, idx, k, o, lse, workspace, L, stream, k_blk, v_blk);
}

mage_status mage_sparse_block_attn_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                         const int32_t* idx, int32_t k, const uint16_t* k_blk,
                                         const uint16_t* v_blk, float* o, float* lse, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k, o, lse, d); st != MAGE_OK) return st;
  if (mage_status st = block_rows_checks(k_blk, v_blk); st != MAGE_OK) return st;
  return paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, k)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        const int64_t sb = su * d.B * d.D;   // block rows before the group
        return sparse_d(g, q + sq * d.D, kv, idx + su * k, k, o + sq * d.D, lse ? lse + sq : nullptr, workspace,
                        make_layout(g, kv.max_n, k), stream, k_blk + sb, v_blk + sb);
      });
}

static mage_status counts_checks(const int32_t* counts, int32_t k_seq) {
  if (!counts || !aligned(counts, 4)) return fail(MAGE_ERR_INVALID_ARG, "counts must be non-null and 4-byte aligned");
  if (k_seq < 1) return fail(MAGE_ERR_INVALID_ARG, "k_seq must be >= 1");
  return MAGE_OK;
}

mage_status mage_sparse_attn_counts(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                                    const uint16_t* v_cache, int32_t seq_len, const int32_t* idx, int32_t k_row,
                                    const int32_t* counts, int32_t k_seq, float* o, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k_row, o, lse, d); st != MAGE_OK) return st;
  if (mage_status st = counts_checks(counts, k_seq); st != MAGE_OK) return st;
  KvArgs kv;
  if (mage_status st = contiguous_kv(d, k_cache, v_cache, seq_len, kv); st != MAGE_OK) return st;
  const Layout L = make_layout(d, kv.max_n, k_row);
  if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
  return d.D == 128
             ? launch_sparse<128>(d, q, kv, idx, k_row, o, lse, workspace, L, stream, nullptr, nullptr, counts, k_seq)
             : launch_sparse<64>(d, q, kv, idx, k_row, o, lse, workspace, L, stream, nullptr, nullptr, counts, k_seq);
}

mage_status mage_sparse_attn_counts_paged(const mage_dims* dims, const uint16_t* q, const mage_paged_kv* kvp,
                                          const int32_t* idx, int32_t k_row, const int32_t* counts, int32_t k_seq,
                                          float* o, float* lse, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = sparse_common(dims, q, idx, k_row, o, lse, d); st != MAGE_OK) return st;
  if (mage_status st = counts_checks(counts, k_seq); st != MAGE_OK) return st;
  return paged_groups(
      d, kvp,
      [&](const Dims& g, const KvArgs& kv) { return check_ws(workspace, workspace_bytes, make_layout(g, kv.max_n, k_row)); },
      [&](const Dims& g, const KvArgs& kv, int s0) {
        const int64_t sq = static_cast<int64_t>(s0) * d.B * d.Hq, su = static_cast<int64_t>(s0) * d.Hkv;
        return sparse_d(g, q + sq * d.D, kv, idx + su * k_row, k_row, o + sq * d.D, lse ? lse + sq : nullptr,
                        workspace, make_layout(g, kv.max_n, k_row), stream, nullptr, nullptr, counts + su, k_seq);
      });
}

mage_status mage_block_attn(const mage_dims* dims, const uint16_t* q, const uint16_t* k_blk,
                            const uint16_t* v_blk, const float* o_prefix, const float* lse_prefix, float* o,
                            float* lse, hipStream_t stream) {
  CallScope scope;
  Dims d;
  if (mage_status st = check_dims(dims, d); st != MAGE_OK) return st;
  if (!q || !k_blk || !v_blk || !o_prefix || !lse_prefix || !o)
    return fail(MAGE_ERR_INVALID_ARG, "q, k_blk, v_blk, o_prefix, lse_prefix and o must not be null");
  if (!aligned(q, 16) || !aligned(k_blk, 16) || !aligned(v_blk, 16) || !aligned(o_prefix, 16) || !aligned(o, 16))
    return fail(MAGE_ERR_INVALID_ARG, "q, k_blk, v_blk, o_prefix and o must be 16-byte aligned");
  if (!aligned(lse_prefix, 4) || (lse && !aligned(lse, 4)))
    return fail(MAGE_ERR_INVALID_ARG, "lse_prefix and lse must be 4-byte aligned");
  BlockParams bp{};
  bp.q = q;
  bp.k_blk = k_blk;
  bp.v_blk = v_blk;
  bp.o_pre = o_prefix;
  bp.lse_pre = lse_prefix;
  bp.o = o;
  bp.lse = lse;
  bp.S = d.S; bp.B = d.B; bp.Hq = d.Hq; bp.Hkv = d.Hkv;
  bp.scale_log2 = d.scale * kLog2e;
  // more than MAGE_MAX_ROWS rows per KV head: one launch per sub-group of heads
  for (int grp = 0; grp < d.ng; ++grp) {
    const Dims g = d.ng > 1 ? group_dims(d, grp) : d;
    bp.G = g.G; bp.R = g.R; bp.gs = g.gs; bp.g0 = g.g0;
    const int64_t grid = g.units * g.nrb;
    if (mage_status st = d.D == 128 ? launch(kfn(block_attn_kernel<128>), "block_attn_kernel", grid, kWave, stream, bp)
                                    : launch(kfn(block_attn_kernel<64>), "block_attn_kernel", grid, kWave, stream, bp);
        st != MAGE_OK)
      return st;
  }
  return MAGE_OK;
}

mage_status mage_topk(int32_t rows, const float* scores, int64_t row_stride, const int32_t* lens,
                      int32_t n, int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  CallScope scope;
  if (rows < 1 || n < 1 || k < 1) return fail(MAGE_ERR_INVALID_ARG, "rows, n and k must be >= 1");
  if (!scores || !idx) return fail(MAGE_ERR_INVALID_ARG, "scores and idx must not be null");
  if (!aligned(scores, 4) || !aligned(idx, 4)) return fail(MAGE_ERR_INVALID_ARG, "scores and idx must be 4-byte aligned");
  if (row_stride < n) return fail(MAGE_ERR_INVALID_ARG, "row_stride must be >= n");
  if (lens) {
    for (int r = 0; r < rows; ++r)
      if (lens[r] < 1 || lens[r] > n) return fail(MAGE_ERR_INVALID_ARG, "lens[r] must be in [1, n]");
  }
  if (rows > (1 << 20)) return fail(MAGE_ERR_UNSUPPORTED, "rows must be <= 2^20");
  if (n > kMaxTopkLen) return fail(MAGE_ERR_UNSUPPORTED, "rows longer than 2^25 entries");
  // workspace: the full layout for one KV head per row. Per-row lengths travel
  // in the kernel arguments, so with lens the rows run in stream-ordered
  // groups of at most MAGE_MAX_SEQS.
  Dims d{};
  d.S = rows; d.B = 1; d.Hq = 1; d.Hkv = 1; d.G = 1; d.R = 1; d.D = 64; d.nrb = 1; d.units = rows;
  d.ng = 1; d.gs = 0; d.g0 = 0; d.r_total = 1;
  d.scale = 1.f;
  const int group = lens ? MAGE_MAX_SEQS : rows;
  for (int pass = 0; pass < 2; ++pass)
    for (int r0 = 0; r0 < rows; r0 += group) {
      const Dims g = lens ? seq_group(d, r0) : d;
      const Layout L = make_layout(g, n, k);
      if (pass == 0) {
        if (mage_status st = check_ws(workspace, workspace_bytes, L); st != MAGE_OK) return st;
        continue;
      }
      SeqLens sl;
      std::memset(&sl, 0, sizeof sl);
      if (lens)
        for (int r = 0; r < g.S; ++r) sl.n[r] = lens[r0 + r];
      const TopkParams tp = topk_params(workspace, L, scores + r0 * row_stride, row_stride, idx + static_cast<int64_t>(r0) * k,
                                        k, g.S, 1, lens ? -1 : n, n, sl, g.S);
      if (mage_status st = launch_topk(tp, stream, true); st != MAGE_OK) return st;
    }
  return MAGE_OK;
}

const char* mage_status_string(mage_status status) {
  switch (status) {
    case MAGE_OK: return "ok";
    case MAGE_ERR_INVALID_ARG: return "invalid argument";
    case MAGE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MAGE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MAGE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mage_last_error(void) { return g_last_error.c_str(); }

mage_status mage_arm_kernel_timers(const hipEvent_t* start, const hipEvent_t* stop, int32_t n) {
  if (n < 0 || n > MAGE_MAX_TIMED_LAUNCHES)
    return fail(MAGE_ERR_INVALID_ARG, "n must be in [0, MAGE_MAX_TIMED_LAUNCHES]");
  if (n > 0 && (!start || !stop)) return fail(MAGE_ERR_INVALID_ARG, "event arrays must not be null");
  for (int i = 0; i < n; ++i) {
    g_launches.start[i] = start[i];
    g_launches.stop[i] = stop[i];
  }
  g_launches.armed = n;
  return MAGE_OK;
}

int32_t mage_last_launches(const char** names, int32_t max_names) {
  const int n = g_launches.used;
  if (names)
    for (int i = 0; i < max_names && i < n && i < MAGE_MAX_TIMED_LAUNCHES; ++i) names[i] = g_launches.names[i];
  return n;
}

#ifdef MAGE_TRACE
// Debug builds only: copy the per-work-group phase timestamps to host memory.
int mage_debug_trace(void* host, size_t bytes) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(mage::g_trace), std::min(bytes, sizeof(mage::g_trace))) == hipSuccess ? 0 : -1;
}
int mage_debug_trace_clear(void) {
  static uint64_t zeros[8192][8];
  return hipMemcpyToSymbol(HIP_SYMBOL(mage::g_trace), zeros, sizeof(zeros)) == hipSuccess ? 0 : -1;
}
#endif

}  // extern "C"
