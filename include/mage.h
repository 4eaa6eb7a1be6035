/*
 * mage.h -- C ABI of the MI355X (gfx950) library for block-shared top-k sparse
 * KV attention in block-diffusion decoding (the MAGE scheme).
 *
 * Method: "MAGE: All-[MASK] Block Already Knows Where to Look in Block
 * Diffusion LLM" (atlas.scime.ai summary page).
 *   - At denoising step 1 one exact attention pass runs for the all-[MASK]
 *     block over the prefix KV cache; it also yields, per (sequence, KV head),
 *     the top-k prefix positions that the whole block then shares
 *     (summary paragraph and "Approach").
 *   - All B tokens of a block share one KV subset ("Problem").
 *   - Every later step attends only to that subset ("Approach").
 *   - Selection runs on a second stream, overlapped with the step-1 output
 *     (summary paragraph; first-step overhead under "Key results").
 * The score that ranks positions is the softmax probability averaged over the
 * B block tokens and the G query heads that share the KV head; ties are
 * broken by the lower position.
 *
 * Notation: S sequences, B block tokens, Hq query heads, Hkv KV heads,
 * G = Hq / Hkv, d head dim, R = B * G query rows per KV head, N (N_s) prefix
 * length, k top-k budget, k_eff = min(k, N_s). Query head j reads KV head
 * j / G. Row r = b * G + g of KV head h is query (token b, head h * G + g).
 *
 * Layouts (all row-major, all buffers device memory unless stated):
 *   Q        bf16 [S][B][Hq][d]        (bf16 passed as uint16_t bit patterns)
 *   K, V     bf16 [S][Hkv][N][d]       contiguous cache, one N for all seqs
 *   pools    bf16 [P][Hkv][page][d]    paged cache; position p of sequence s
 *                                      is slot p % page of page
 *                                      page_table[s * max_pages + p / page]
 *   O        fp32 [S][B][Hq][d]
 *   lse      fp32 [S][B][Hq]           natural-log log-sum-exp of scale*q.k
 *   scores   fp32 [S][Hkv][stride]     stride = N (contiguous) or
 *                                      max_seq_len (paged); entries at
 *                                      p >= N_s are left untouched
 *   idx      int32 [S][Hkv][k]         ascending positions, -1 past k_eff
 *
 * Ownership: the caller owns every buffer, stream and event. The library
 * never allocates device memory in these calls; all scratch lives in the
 * caller's workspace (size from mage_workspace_bytes). Calls are
 * asynchronous and stream-ordered; host-side argument checks happen before
 * any launch, and a failed check launches nothing.
 *
 * Workspace contract: zero-fill a new workspace once with
 * mage_workspace_init before its first call (again only if the caller writes
 * over it). Its first 256 KiB hold arrival counters that the later-step calls
 * (mage_sparse_attn, mage_sparse_block_attn and their paged forms) use to
 * merge split work inside one launch; every call leaves them at zero, and no
 * other part of any call's layout overlaps them. The rest of the workspace is
 * scratch that no call expects to hold anything. Calls that may run
 * concurrently need distinct workspaces; a workspace may be reused once the
 * previous call's work (including its select stream) is ordered before the
 * new call. A workspace with non-zero counters makes a later step return
 * wrong values (it does not fault or hang); mage_workspace_check detects that
 * state.
 *
 * Errors: every entry point returns a mage_status and never aborts.
 * MAGE_ERR_HIP carries the runtime's message in mage_last_error() (thread
 * local). Content preconditions (finite values, valid page ids, unique idx
 * entries) are documented, not checked: idx entries outside [0, N_s) are
 * skipped by the sparse step, never dereferenced.
 */
#ifndef MAGE_H_
#define MAGE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mage_status {
  MAGE_OK = 0,
  MAGE_ERR_INVALID_ARG = 1,          /* null pointer, bad size, Hq % Hkv != 0 */
  MAGE_ERR_UNSUPPORTED = 2,          /* d not in {64, 128}, B > 128, sizes beyond a
                                        stated maximum (MAGE_MAX_SPARSE_K, ...) */
  MAGE_ERR_WORKSPACE_TOO_SMALL = 3,
  MAGE_ERR_HIP = 4                   /* launch or runtime failure; see mage_last_error() */
} mage_status;

/* Sequences per launch of a paged call (their lengths and chunk numbering
 * travel in the kernel arguments). A paged call over more sequences runs as
 * consecutive groups of at most MAGE_MAX_SEQS sequences, in stream order on
 * the call's stream with the same workspace; its results are those of one
 * call per group. Every group's arguments are checked before the first
 * launch. A grouped step-1 call runs its selection on attn_stream too; the
 * select stream, when given, waits for the end and records idx_ready there.
 * The standalone top-k runs rows with per-row lengths the same way. */
#define MAGE_MAX_SEQS 256
/* Largest R = B * G rows per KV head that one pass of the kernels takes.
 * Every call takes larger head groups: it runs the G query heads of each KV
 * head in the fewest equal sub-groups of at most MAGE_MAX_ROWS rows, one
 * after another on the call's stream (every kernel of the call on that
 * stream; the select stream, when given, waits for the end), with the score
 * averaged over all R rows before the top-k (positions, pages or budgets).
 * The mean query averages all R rows in one pass. B <= MAGE_MAX_ROWS always. */
#define MAGE_MAX_ROWS 128

typedef struct mage_dims {
  int32_t num_seqs;      /* S >= 1 */
  int32_t block;         /* B >= 1, query tokens per block */
  int32_t num_q_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0 (R = B * Hq / Hkv: see MAGE_MAX_ROWS) */
  int32_t head_dim;      /* d in {64, 128} */
  float scale;           /* softmax scale applied to q.k (finite, > 0) */
} mage_dims;

/* A paged KV cache. seq_lens is HOST memory (read during the call). */
typedef struct mage_paged_kv {
  const uint16_t* k_pool;     /* bf16 [P][Hkv][page_size][d] */
  const uint16_t* v_pool;     /* bf16 [P][Hkv][page_size][d] */
  const int32_t* page_table;  /* device int32 [S][max_pages] physical page ids */
  int32_t max_pages;          /* row stride of page_table */
  int32_t page_size;          /* power of two, 1..1024 */
  const int32_t* seq_lens;    /* HOST int32 [S], 1 <= N_s <= max_pages * page_size */
} mage_paged_kv;

/* Bytes of workspace that every entry point below needs for these dims, any
 * prefix length <= max_seq_len and any top-k budget <= k (including a paged
 * call's groups of MAGE_MAX_SEQS sequences). */
size_t mage_workspace_bytes(const mage_dims* dims, int32_t max_seq_len, int32_t k);

/* Zero-fill a workspace on `stream` with a fill kernel (no memset node).
 * Required once on a new workspace: the later-step calls keep arrival
 * counters in it, which must start at zero (every call leaves them at zero).
 * workspace 4-byte aligned, workspace_bytes a multiple of 4, else
 * MAGE_ERR_INVALID_ARG. */
mage_status mage_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Count the non-zero arrival counters of a workspace (the first 256 KiB) on
 * `stream`: *nonzero (device int32, 4-byte aligned) receives their number once
 * the stream reaches this point. Every call leaves them at zero, so a
 * non-zero count means the workspace was not zeroed with mage_workspace_init,
 * was written over, or saw a call overlap another on a second stream; a later
 * step on it would return wrong values. Null or misaligned pointers give
 * MAGE_ERR_INVALID_ARG, a workspace smaller than the counter region
 * MAGE_ERR_WORKSPACE_TOO_SMALL. */
mage_status mage_workspace_check(const void* workspace, size_t workspace_bytes, int32_t* nonzero,
                                 hipStream_t stream);

/*
 * Step 1 of a block (MAGE page, summary and "Approach"): exact attention of
 * the block's queries over the whole prefix, the block-averaged score of every
 * prefix position, and the top-k positions per (sequence, KV head).
 *
 * Exact pass (split over N, MFMA, online softmax) then the split merge run on
 * attn_stream; O and lse are final when attn_stream reaches that point. The
 * score sweep (which merges the row statistics it needs from the exact pass's
 * partials itself) and top-k run on select_stream after waiting for the exact
 * pass, beside the merge; idx and scores are final when select_stream
 * completes, and idx_ready (if non-null) is recorded there. select_stream may
 * be null (= attn_stream). lse and scores may be null.
 */
mage_status mage_select_exact(const mage_dims* dims, const uint16_t* q,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              int32_t seq_len, int32_t k, float* o, float* lse,
                              int32_t* idx, float* scores, void* workspace,
                              size_t workspace_bytes, hipStream_t attn_stream,
                              hipStream_t select_stream, hipEvent_t idx_ready);

mage_status mage_select_exact_paged(const mage_dims* dims, const uint16_t* q,
                                    const mage_paged_kv* kv, int32_t k, float* o,
                                    float* lse, int32_t* idx, float* scores,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t attn_stream, hipStream_t select_stream,
                                    hipEvent_t idx_ready);

/*
 * Exact attention only (the step-1 pass without selection; also the
 * exact-attention-at-every-step baseline the MAGE page compares against under
 * "Key results"). Runs the split exact pass and merge on `stream`.
 * lse may be null.
 */
mage_status mage_exact_attn(const mage_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, int32_t seq_len, float* o, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

mage_status mage_exact_attn_paged(const mage_dims* dims, const uint16_t* q,
                                  const mage_paged_kv* kv, float* o, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * A later denoising step (MAGE page, "Approach": later steps reuse the step-1
 * subset): for every (sequence, KV head), gather the K/V rows named by
 * idx[s][h][0..k) and compute attention of the block's queries over them.
 * idx may be in any order; entries outside [0, N_s) are skipped (a head with
 * no valid entry gets O = 0, lse = -inf). lse may be null. k (the index row
 * length) must be in [1, MAGE_MAX_SPARSE_K], else MAGE_ERR_INVALID_ARG (k < 1)
 * or MAGE_ERR_UNSUPPORTED (k too large).
 * One launch: when the index rows are split over several work-groups, the
 * last of them to finish for a (unit, 32-row block) merges the split results,
 * counted through the workspace's arrival counters (zeroed once by
 * mage_workspace_init).
 */
#define MAGE_MAX_SPARSE_K 131072
mage_status mage_sparse_attn(const mage_dims* dims, const uint16_t* q,
                             const uint16_t* k_cache, const uint16_t* v_cache,
                             int32_t seq_len, const int32_t* idx, int32_t k, float* o,
                             float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

mage_status mage_sparse_attn_paged(const mage_dims* dims, const uint16_t* q,
                                   const mage_paged_kv* kv, const int32_t* idx, int32_t k,
                                   float* o, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * mage_sparse_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc). Same arguments and results as mage_sparse_attn
 * (the same kernels and launch plan, so the same bits) minus the workspace.
 * Its scratch (arrival counters and split partials) is a fixed array in the
 * library's code object: 256 KiB of counters plus 8 MiB of partials per GPU,
 * held until the process ends. A call whose split partials need more (for
 * example more than 126 (sequence, KV head) x chunk slots at d = 128) returns
 * MAGE_ERR_UNSUPPORTED before any launch. The call allocates nothing; its
 * first use on a device looks up the array's address and zeroes its counters
 * on `stream`. Every call on one GPU shares that array and leaves the
 * counters at zero: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 */
mage_status mage_sparse_attn_noalloc(const mage_dims* dims, const uint16_t* q,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     int32_t seq_len, const int32_t* idx, int32_t k, float* o,
                                     float* lse, hipStream_t stream);

/*
 * Block attention (the op a block-diffusion layer calls after the prefix
 * pass): every query of the current block attends to the selected prefix
 * rows and to all B rows of its own block, which the block's tokens share
 * (they are denoised jointly; MAGE page, "Problem" and "Approach" select
 * prefix rows only). The prefix part is given as the normalised output and
 * natural log-sum-exp of mage_select_exact / mage_exact_attn /
 * mage_sparse_attn; the block part is computed here, and the two are merged:
 *   O = (e^{lse_p} O_p + e^{lse_b} O_b) / (e^{lse_p} + e^{lse_b}),
 *   lse = log(e^{lse_p} + e^{lse_b}), with lse_p = -inf for rows that had no
 *   prefix entry.
 * q: bf16 [S][B][Hq][d] (as for the other entry points); k_blk, v_blk: bf16
 * [S][Hkv][B][d], the block's own keys and values; o_prefix: fp32
 * [S][B][Hq][d]; lse_prefix: fp32 [S][B][Hq]. Outputs o: fp32 [S][B][Hq][d]
 * and lse: fp32 [S][B][Hq] (nullable). o may be o_prefix and lse may be
 * lse_prefix (in place). All pointers are device memory, q/k_blk/v_blk/
 * o_prefix/o 16-byte aligned, the lse arrays 4-byte aligned, else
 * MAGE_ERR_INVALID_ARG; dims are checked as for the other entry points. No
 * workspace.
 */
mage_status mage_block_attn(const mage_dims* dims, const uint16_t* q, const uint16_t* k_blk,
                            const uint16_t* v_blk, const float* o_prefix, const float* lse_prefix,
                            float* o, float* lse, hipStream_t stream);

/*
 * A later denoising step with the block's own rows, in one pass: the result
 * mage_sparse_attn followed by mage_block_attn would give (attention of the
 * block's queries over the k gathered prefix rows together with the block's B
 * rows, MAGE page, "Approach", with the block rows read as above), but the
 * block rows are one more 32-row tile for each wave of the last split of the
 * sparse pass, so they fold into the same online softmax and split merge: no
 * separate launch and no prefix O round trip. Arguments as for mage_sparse_attn / mage_sparse_attn_paged,
 * plus k_blk, v_blk: bf16 [S][Hkv][B][d] device memory, 16-byte aligned, not
 * null, else MAGE_ERR_INVALID_ARG. The workspace is the same as for
 * mage_sparse_attn. A head with no valid index entry still sees its block
 * rows.
 */
mage_status mage_sparse_block_attn(const mage_dims* dims, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   int32_t seq_len, const int32_t* idx, int32_t k,
                                   const uint16_t* k_blk, const uint16_t* v_blk, float* o,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

mage_status mage_sparse_block_attn_paged(const mage_dims* dims, const uint16_t* q,
                                         const mage_paged_kv* kv, const int32_t* idx, int32_t k,
                                         const uint16_t* k_blk, const uint16_t* v_blk, float* o,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * Top-k of `rows` non-negative fp32 score rows (the selection step on its own):
 * row r has lens[r] valid entries (lens is HOST memory; null means all rows
 * have n entries) at scores + r * row_stride. Output idx [rows][k]: the
 * k_eff = min(k, lens[r]) positions with the largest scores, ties to the lower
 * position, in ascending order, then -1. Scores must be >= +0 and not NaN.
 * The workspace must come from mage_workspace_bytes with a max_seq_len >= n
 * and num_seqs * num_kv_heads >= rows.
 */
mage_status mage_topk(int32_t rows, const float* scores, int64_t row_stride,
                      const int32_t* lens, int32_t n, int32_t k, int32_t* idx,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Page-granular selection (the block-sparse form of step 1): positions are
 * grouped into pages of page_tokens consecutive positions (the last page of a
 * prefix holds what is left), a page's score is the sum of its positions'
 * block-averaged scores, and the k_pages pages with the largest scores per
 * (sequence, KV head) are kept whole (ties to the lower page). Step-dLLM page
 * (abstract): a block-sparse mask; pages of a paged cache are the natural
 * unit of a gather. Outputs: idx int32 [S][Hkv][k_pages * page_tokens], the
 * chosen pages' positions page by page in ascending order, -1 past N_s and
 * for missing pages (k_pages > pages in the prefix) -- a valid idx for
 * mage_sparse_attn with k = k_pages * page_tokens; page_idx (nullable) int32
 * [S][Hkv][k_pages], the ascending page ids, -1 padded. o, lse, scores,
 * streams and idx_ready as for mage_select_exact. page_tokens in [1, 4096]
 * (it need not match a paged cache's page size), k_pages >= 1, else
 * MAGE_ERR_INVALID_ARG; k_pages * page_tokens <= MAGE_MAX_SPARSE_K, else
 * MAGE_ERR_UNSUPPORTED. Workspace: mage_workspace_bytes(dims, max_seq_len,
 * k_pages * page_tokens).
 */
mage_status mage_select_pages(const mage_dims* dims, const uint16_t* q,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              int32_t seq_len, int32_t page_tokens, int32_t k_pages, float* o,
                              float* lse, int32_t* idx, int32_t* page_idx, float* scores,
                              void* workspace, size_t workspace_bytes, hipStream_t attn_stream,
                              hipStream_t select_stream, hipEvent_t idx_ready);

mage_status mage_select_pages_paged(const mage_dims* dims, const uint16_t* q,
                                    const mage_paged_kv* kv, int32_t page_tokens, int32_t k_pages,
                                    float* o, float* lse, int32_t* idx, int32_t* page_idx,
                                    float* scores, void* workspace, size_t workspace_bytes,
                                    hipStream_t attn_stream, hipStream_t select_stream,
                                    hipEvent_t idx_ready);

/*
 * Head-adaptive budgets (Step-dLLM page, abstract: one global budget shared
 * by the heads, compressing heads with concentrated attention harder). Step 1
 * as mage_select_exact, except that each sequence keeps the K = k * Hkv
 * largest block-averaged scores over all of its (KV head, position) pairs,
 * ties to the lower head, then the lower position: head h keeps counts[s][h]
 * positions (a head whose scores sit on few positions keeps few, a diffuse
 * head many; the counts of a sequence sum to min(K, Hkv * N_s)). Outputs
 * idx int32 [S][Hkv][K], each row ascending then -1, and counts int32
 * [S][Hkv] (device, not null, 4-byte aligned). o/lse/streams/idx_ready as
 * for mage_select_exact; no scores output. k * Hkv <= MAGE_MAX_SPARSE_K and
 * Hkv * N <= 2^25, else MAGE_ERR_UNSUPPORTED. Workspace:
 * mage_workspace_bytes(dims, max_seq_len, k * num_kv_heads).
 */
mage_status mage_select_adaptive(const mage_dims* dims, const uint16_t* q,
                                 const uint16_t* k_cache, const uint16_t* v_cache,
                                 int32_t seq_len, int32_t k, float* o, float* lse, int32_t* idx,
                                 int32_t* counts, void* workspace, size_t workspace_bytes,
                                 hipStream_t attn_stream, hipStream_t select_stream,
                                 hipEvent_t idx_ready);

mage_status mage_select_adaptive_paged(const mage_dims* dims, const uint16_t* q,
                                       const mage_paged_kv* kv, int32_t k, float* o, float* lse,
                                       int32_t* idx, int32_t* counts, void* workspace,
                                       size_t workspace_bytes, hipStream_t attn_stream,
                                       hipStream_t select_stream, hipEvent_t idx_ready);

/*
 * A later step with per-head entry counts (the index rows of
 * mage_select_adaptive): unit (s, h) attends over idx[s][h][0 .. min(counts,
 * k_row)), where k_row is the row length of idx (entries outside [0, N_s)
 * are skipped as in mage_sparse_attn). Work scales with the counts, not with
 * k_row: a sequence's chunks are numbered densely, planned for at most k_seq
 * entries per sequence (sum over its heads of min(counts, k_row)); chunks
 * beyond that plan are not computed. counts: device int32 [S][Hkv], not null,
 * 4-byte aligned; k_seq >= 1; other arguments and the workspace as for
 * mage_sparse_attn with k = k_row. A head with count 0 gets O = 0, lse = -inf.
 */
mage_status mage_sparse_attn_counts(const mage_dims* dims, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    int32_t seq_len, const int32_t* idx, int32_t k_row,
                                    const int32_t* counts, int32_t k_seq, float* o, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

mage_status mage_sparse_attn_counts_paged(const mage_dims* dims, const uint16_t* q,
                                          const mage_paged_kv* kv, const int32_t* idx,
                                          int32_t k_row, const int32_t* counts, int32_t k_seq,
                                          float* o, float* lse, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/*
 * Anchor re-selection diagnostics. The Step-dLLM page (abstract) refreshes the
 * sparse set at anchor steps and reuses it in between; re-running
 * mage_select_exact with an anchor step's queries is that refresh, and the
 * two calls below measure what it buys.
 *
 * mage_mean_query: the mean query alone, written to qbar, bf16 [S][Hkv][d]
 * (the q of a one-token block with one query head per KV head); q and qbar
 * are device memory, 2-byte aligned, not null, else MAGE_ERR_INVALID_ARG.
 *
 * mage_select_mean_query: top-k by the probability under the block's mean
 * query instead of the probability averaged over the block's rows (the other
 * reading of the MAGE page's block-average query, "Approach"). The mean query
 * of KV head h is the exact mean of its R = B*G query rows, rounded once to
 * bf16 (nearest, ties to even; exact whenever those rows' magnitudes span
 * less than about 2^38). It then goes through the step-1 selection as a
 * one-token block with one query head per KV head. Arguments as for
 * mage_select_exact without o/lse (scores nullable, [S][Hkv][N] or
 * [S][Hkv][max N_s] paged); everything runs on `stream`. Same workspace as
 * mage_select_exact.
 */
mage_status mage_mean_query(const mage_dims* dims, const uint16_t* q, uint16_t* qbar,
                            hipStream_t stream);

mage_status mage_select_mean_query(const mage_dims* dims, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   int32_t seq_len, int32_t k, int32_t* idx, float* scores,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

mage_status mage_select_mean_query_paged(const mage_dims* dims, const uint16_t* q,
                                         const mage_paged_kv* kv, int32_t k, int32_t* idx,
                                         float* scores, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * mage_idx_overlap: for `rows` pairs of index rows a[r], b[r] (int32 [rows][k],
 * each in idx form: ascending non-negative entries, then negative padding),
 * common[r] = the number of valid entries present in both; count_a[r] and
 * count_b[r] (nullable) = the number of valid entries of each. The recall of
 * a against the reference b is common / count_b. Device memory, 4-byte
 * aligned; rows, k >= 1, else MAGE_ERR_INVALID_ARG. Rows that are not in idx
 * form give unspecified counts (every read stays inside its row).
 */
mage_status mage_idx_overlap(int32_t rows, int32_t k, const int32_t* a, const int32_t* b,
                             int32_t* common, int32_t* count_a, int32_t* count_b,
                             hipStream_t stream);

const char* mage_status_string(mage_status status);
const char* mage_last_error(void);

/*
 * Kernel timing for benchmarks and profilers (not part of the method).
 *
 * mage_arm_kernel_timers arms up to MAGE_MAX_TIMED_LAUNCHES pairs of HIP
 * events for the NEXT compute entry point called on this thread: its i-th
 * kernel launch (launch order, i < n) is made with hipExtLaunchKernel so that
 * start[i] / stop[i] record when that kernel begins and ends on the GPU. The
 * events belong to the caller (created with timing enabled, on the device of
 * the call); the arrays are copied, so they may be freed after the call. Any
 * compute entry point disarms the timers when it returns. n = 0 disarms.
 * Returns MAGE_ERR_INVALID_ARG for n outside [0, MAGE_MAX_TIMED_LAUNCHES] or
 * a null array with n > 0.
 *
 * mage_last_launches reports the kernels that the last compute entry point on
 * this thread launched, armed or not: it returns their number and stores up
 * to max_names static, NUL-terminated kernel names into names (may be null).
 */
#define MAGE_MAX_TIMED_LAUNCHES 12
mage_status mage_arm_kernel_timers(const hipEvent_t* start, const hipEvent_t* stop, int32_t n);
int32_t mage_last_launches(const char** names, int32_t max_names);

#ifdef __cplusplus
}
#endif

#endif /* MAGE_H_ */
