/*
 * pa.h -- C ABI of the MI355X (gfx950) deterministic paged-KV GQA attention library.
 *
 * The library computes, for every row b, query head h and query i,
 *
 *   q^  = bf16( RoPE( RMSNorm(q) * w_q , query_position_ids[b][i] ) )
 *   k^j = bf16( RoPE( RMSNorm(k_j) * w_k , j ) )            j = logical key index of row b
 *   s_j = (q^ . k^j) / sqrt(head_dim)                        for keys with j <= query position
 *   lse = log( sum_j exp(s_j) )                              natural log, FP32
 *   out = bf16( sum_j exp(s_j - lse) * v_j )
 *
 * with FP32 accumulation and a reduction order that depends only on the row's own
 * length: never on the batch it runs in, on the plan's capacity ("plan width") or on
 * where its pages sit in the pool.  Sources (web pages, cited by title and section):
 *
 *   [PR279]  "[WS2][PR7][Attention] Add FlashInfer RoPE-fused paged attention scaffold",
 *            section "Scope" (boundary table: logical K/V order materialised before
 *            arithmetic, Split-KV disabled, FP32 attention-domain LSE, GQA packing from
 *            the head layout, same post-RoPE boundary on both sides, Q/K RMSNorm).
 *   [PR7]    "WS2 PR7 Fused Attention Backend Alignment", sections "Original PR7
 *            Requirements" (LSE shaped [B, Hq, Sq]; metadata validated before execution),
 *            "Current Implementation" (validation steps; out [B, Hq, Sq, D]),
 *            "FlashInfer RoPE Fusion" (Llama rotate-half RoPE, theta 1e6, scale 1.0,
 *            rotary_dim = head_dim; pre-RoPE Q and K cache; cache_position ==
 *            query_position_ids; trailing contiguous query positions),
 *            "Split-KV Policy" (disabled / fixed:<N> / auto, auto rejected).
 *   [PR162]  "flashinfer_fa2 backend for NVIDIA Ada (SM89)", sections "Summary" (BF16,
 *            page size 16, head_dim 128, NHD), "Design notes" (CSR indptr / compact
 *            indices / last_page_len; Split-KV disabled so a row's result does not depend
 *            on plan width or batch), "Code audit" (empty rows have last_page_len 1;
 *            unsupported head ratios and row-count mismatches are rejected).
 *   [XCFG]   "WS2 Attention Cross-Configuration Integration", sections "H100 Attention
 *            input and projection boundary" (order: Q/K RMSNorm, then RoPE) and "Fail
 *            closed, never substitute" (FP32 accumulation, downcast only at the final
 *            write, unsupported requests are errors).
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device addresses of caller-owned buffers; the library
 *     keeps no pointer after a call returns.  `stream` is a hipStream_t (NULL = the
 *     default stream).
 *   - BF16 tensors are raw 16-bit patterns.  All tensors are dense, row-major, with the
 *     layouts stated below.
 *   - Errors are negative pa_status codes; nothing falls back to another algorithm.
 *   - pa_decode / pa_prefill never allocate, never synchronise and never read device
 *     memory from the host, so they may be recorded into a HIP graph.  They check host
 *     scalars only.  The kernels additionally check every metadata value they read and
 *     never access memory through an out-of-range value; broken metadata fails closed with
 *     NaN instead ([XCFG] "Fail closed, never substitute"; [PR162] "Code audit"):
 *       - a row whose indptr extent or last_page_len is out of range, or (prefill) whose
 *         extent is not part of a non-decreasing indptr prefix, gets NaN in all its out and
 *         lse;
 *       - an out-of-range page index, a query position outside [0, table rows) or a
 *         cache_position that differs from its query_position_ids entry gets NaN in every
 *         output computed from it (decode: the whole row; prefill: each block of 32 queries
 *         that reads that page or holds that query);
 *       - a key whose key_position_ids entry is not its logical index gets NaN in every
 *         output that attends to it (decode: the whole row; prefill: every query that sees
 *         the key).
 *     The launch still succeeds.  Call pa_validate_metadata first to get a precise error
 *     instead.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = -1,  /* null pointer, non-positive size, bad plan handle          */
  PA_ERR_UNSUPPORTED = -2,       /* head_dim != 128, page_size != 16, theta != 1e6,
                                    rope_scale != 1, unknown or "auto" split policy            */
  PA_ERR_CAPACITY = -3,          /* batch, q_len or pages per row beyond the plan            */
  PA_ERR_HEAD_RATIO = -4,        /* Hq not a positive multiple of Hkv, or Hq/Hkv > 16         */
  PA_ERR_INDPTR = -5,            /* indptr[0] != 0, decreasing, or indptr[B] != num_indices   */
  PA_ERR_PAGE_OOB = -6,          /* a page index outside [0, num_pages)                      */
  PA_ERR_DUPLICATE_PAGE = -7,    /* a physical page used twice in the batch                  */
  PA_ERR_LAST_PAGE_LEN = -8,     /* outside [1, page_size], or != 1 for a row with no pages  */
  PA_ERR_KEY_POSITION = -9,      /* key_position_ids not 0, 1, ..., L_b - 1 in logical order */
  PA_ERR_QUERY_POSITION = -10,   /* query positions not contiguous, negative, or not ending
                                    at L_b - 1 or L_b                                        */
  PA_ERR_CACHE_POSITION = -11,   /* cache_position != query_position_ids                     */
  PA_ERR_WORKSPACE = -12,        /* a workspace too small (decode), or missing (prefill)      */
  PA_ERR_HIP = -13               /* a HIP runtime call failed                                */
};

/* Split-KV policy ([PR7] "Split-KV Policy": disabled, fixed:<N> with N in logical KV
 * tokens divisible by the page size, auto).
 *   PA_SPLIT_DISABLED  the default: decode's fixed 16-stream tree, prefill's one pass.
 *   PA_SPLIT_FIXED     decode only: each row's keys are cut into chunks of N tokens at
 *                      positions 0, N, 2N, ... (a length-only partition: [PR162] "Code
 *                      audit", the Triton backend whose partition depends only on a row's
 *                      own length); every chunk is one online softmax over its pages in
 *                      ascending order, and the chunk states are folded in ascending chunk
 *                      order in FP32.  The tree depends only on the row's length and N, so
 *                      results stay batch- and plan-width-invariant; the bits differ from
 *                      PA_SPLIT_DISABLED's.
 *   PA_SPLIT_AUTO      rejected: it makes a row's reduction depend on the batch. */
enum { PA_SPLIT_DISABLED = 0, PA_SPLIT_FIXED = 1, PA_SPLIT_AUTO = 2 };

typedef struct pa_plan_s* pa_plan_t;

/* Result of pa_validate_metadata: the first violated rule, in the order PA_ERR_INDPTR,
 * PA_ERR_CAPACITY (pages per row), PA_ERR_PAGE_OOB, PA_ERR_DUPLICATE_PAGE,
 * PA_ERR_LAST_PAGE_LEN, PA_ERR_KEY_POSITION, PA_ERR_QUERY_POSITION, PA_ERR_CACHE_POSITION,
 * and within that rule the lowest offending element. */
typedef struct {
  pa_status code;   /* PA_OK or the violated rule                                   */
  int32_t row;      /* batch row of the violation, -1 if not row-specific            */
  int64_t index;    /* element index in the offending array, -1 if not applicable   */
  int64_t value;    /* the offending value (or the expected one for count checks)    */
} pa_validation_report;

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);

/* Create a plan: fixed shapes, capacities, the split policy and the RoPE cos/sin table.
 *   num_q_heads, num_kv_heads  Hq, Hkv of one GPU's head share; Hq % Hkv == 0, Hq/Hkv <= 16
 *                              ([PR279] "Scope": GQA packing fixed from the head layout).
 *   head_dim, page_size        must be 128 and 16 ([PR162] "Summary").
 *   max_batch, max_q_len       capacity for B and Sq.
 *   max_pages_per_row          capacity for pages per row.  Capacity only: it never
 *                              changes the arithmetic ([PR162] "Design notes").
 *   rope_theta, rope_scale     must be 1e6 and 1.0; rms_eps > 0 ([PR7] "FlashInfer RoPE
 *                              Fusion").
 *   split_policy               PA_SPLIT_DISABLED or PA_SPLIT_FIXED (else
 *                              PA_ERR_UNSUPPORTED).
 *   split_chunk_tokens         PA_SPLIT_FIXED: the chunk size N, a positive multiple of 16
 *                              (else PA_ERR_UNSUPPORTED); ignored otherwise.  A row may hold
 *                              at most 4096 chunks: max_pages_per_row * 16 / N above 4096
 *                              returns PA_ERR_CAPACITY.
 * Allocates device memory for the cos/sin table (max_pages_per_row * page_size + 1
 * positions, 512 bytes each) and synchronises the current device once.  The plan is
 * immutable afterwards and may serve several streams at once.  *plan_out is written
 * only on success. */
pa_status pa_plan(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                  int32_t max_batch, int32_t max_q_len, int32_t max_pages_per_row,
                  float rope_theta, float rope_scale, float rms_eps, int32_t split_policy,
                  int32_t split_chunk_tokens, pa_plan_t* plan_out);

/* Free a plan and its device table.  NULL is accepted.  No call using the plan may be in
 * flight on any stream. */
pa_status pa_plan_destroy(pa_plan_t plan);

/* Check the paged-KV metadata on the device before execution ([PR7] "Original PR7
 * Requirements": page table, cache_position, query_position_ids, key_position_ids and
 * logical token order are validated before execution; "Current Implementation": page
 * bounds, logical order, key positions, duplicate pages, non-canonical inactive rows,
 * cache_position == query_position_ids, trailing query positions; [PR162] "Code audit":
 * empty rows carry last_page_len 1).
 *   batch, q_len               B and Sq (host scalars, checked against the plan).
 *   num_pages                  pages in the K/V pool.
 *   num_indices                nnz, the length of kv_indices.
 *   kv_indptr        int32 [B+1]       row b owns kv_indices[kv_indptr[b] .. kv_indptr[b+1]).
 *   kv_indices       int32 [nnz]       physical page ids, logical page order.
 *   kv_last_page_len int32 [B]         keys in each row's last page.
 *   cache_position, query_position_ids int32 [B, Sq].
 *   key_position_ids int32 [nnz * 16]  logical key j of row b at kv_indptr[b] * 16 + j;
 *                                      entries past a row's length are ignored.
 * Launches validation kernels on `stream`, copies a small report back and synchronises
 * `stream`; allocates and frees a scratch buffer of num_pages * 4 bytes.  Returns the
 * report's code (PA_OK if every rule holds); `report` (optional) receives the details. */
pa_status pa_validate_metadata(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages,
                               int32_t num_indices, const int32_t* kv_indptr,
                               const int32_t* kv_indices, const int32_t* kv_last_page_len,
                               const int32_t* cache_position, const int32_t* query_position_ids,
                               const int32_t* key_position_ids, void* stream,
                               pa_validation_report* report);

/* Paged decode (Sq = 1): the G = Hq/Hkv query heads of each (row, KV head) against every key
 * of the row, with the page gather, the RMSNorm + RoPE + BF16 prologue of q and of every key,
 * an FP32 online softmax and the P.V product fused, and no Split-KV ([PR279] "Scope"; [PR7]
 * "FlashInfer RoPE Fusion", "Split-KV Policy"; [PR162] "Design notes").
 *   q                bf16 [B, Hq, 1, 128]   pre-norm, pre-RoPE.
 *   k_cache, v_cache bf16 [num_pages, 16, Hkv, 128] (NHD); K pre-norm, pre-RoPE.
 *   q_norm_weight, k_norm_weight  fp32 [128], or NULL to skip that RMSNorm.
 *   kv_indptr, kv_indices, kv_last_page_len, cache_position, query_position_ids,
 *   key_position_ids   the metadata as for pa_validate_metadata, with Sq = 1 ([PR7]
 *                    "Original PR7 Requirements": the page table, cache_position,
 *                    query_position_ids and key_position_ids are the adapter's inputs).  The
 *                    query sits at query_position_ids[b]; key j of row b sits at
 *                    key_position_ids[kv_indptr[b] * 16 + j], which must be j (logical
 *                    order, [PR7] "Current Implementation"): RoPE rotates key j by j and the
 *                    kernels check the entry (see the conventions above).
 *   out              bf16 [B, Hq, 1, 128]   written.
 *   lse              fp32 [B, Hq, 1]        written; natural log of the sum of
 *                                           exp(scaled scores) ([PR7] "Original PR7
 *                                           Requirements").  Rows with no keys get
 *                                           out = 0 and lse = -inf.
 *   workspace        NULL, or device memory of at least pa_decode_workspace_size() bytes.
 * Reduction order: each (row, KV head)'s pages are dealt to 16 streams (stream s takes pages
 * s, s+16, s+32, ...), each stream is an online softmax over its pages in ascending order,
 * and the 16 stream states are combined in stream order.  The order depends only on the row
 * itself.  With workspace == NULL one workgroup runs all 16 streams; with a workspace each
 * stream runs on its own compute unit and writes its state there, and a second kernel
 * combines the states, which spreads a long row over 16 compute units.  Both give
 * bit-identical results.  Under a PA_SPLIT_FIXED plan the chunks of N tokens replace the 16
 * streams: one wavefront per (row, KV head, chunk) writes the chunk's state to the workspace
 * and a second kernel folds the states in ascending chunk order; the workspace is then
 * required (PA_ERR_WORKSPACE without one).  The workspace needs no initialisation (every call
 * writes what it reads).  Calls that overlap in time need separate workspaces.
 * Asynchronous on `stream`; requires q_len == 1 and batch <= plan capacity. */
pa_status pa_decode(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages,
                    int32_t num_indices, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* kv_last_page_len, const int32_t* cache_position,
                    const int32_t* query_position_ids, const int32_t* key_position_ids,
                    const void* q, const void* k_cache, const void* v_cache,
                    const float* q_norm_weight, const float* k_norm_weight,
                    void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode's multi-compute-unit schedule (or, under a PA_SPLIT_FIXED plan, its fixed-chunk
 * schedule) without a caller workspace and without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, results and bits as pa_decode with a workspace; the
 * stream states live in a library-owned scratch array of 16 MiB per device instead (set up on
 * the device by pa_plan, held until the process ends).  A batch whose workspace
 * (pa_decode_workspace_size) exceeds 16 MiB returns PA_ERR_CAPACITY; for Hq = 16, Hkv = 4 under
 * PA_SPLIT_DISABLED that is any batch above 125 rows.  The scratch needs no initialisation
 * (every call writes what it reads), but all calls on one device share it: calls that overlap
 * in time on the same device (several streams, several threads) race and must not be issued.
 * No allocation, no synchronisation, no memset: asynchronous on `stream`. */
pa_status pa_decode_no_alloc(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages,
                             int32_t num_indices, const int32_t* kv_indptr, const int32_t* kv_indices,
                             const int32_t* kv_last_page_len, const int32_t* cache_position,
                             const int32_t* query_position_ids, const int32_t* key_position_ids,
                             const void* q, const void* k_cache, const void* v_cache,
                             const float* q_norm_weight, const float* k_norm_weight,
                             void* out, float* lse, void* stream);

/* Workspace bytes of pa_decode's multi-compute-unit schedule for `batch` rows under this
 * plan's split policy (host arithmetic only; a PA_SPLIT_FIXED plan needs room for
 * ceil(max_pages_per_row * 16 / N) chunk states per (row, KV head)). */
pa_status pa_decode_workspace_size(pa_plan_t plan, int32_t batch, size_t* bytes);

/* Workspace bytes pa_prefill needs for these sizes (host arithmetic only). */
pa_status pa_prefill_workspace_size(pa_plan_t plan, int32_t batch, int32_t q_len,
                                    int32_t num_indices, size_t* bytes);

/* Chunked paged prefill: Sq >= 1 trailing queries per row attend causally (key j visible
 * to the query at position p iff j <= p, on logical positions) to the row's cached keys,
 * which include the chunk's own keys ([PR7] "Current Implementation", "FlashInfer RoPE
 * Fusion").  Same arguments and layouts as pa_decode with Sq = q_len, plus a caller-owned
 * device workspace of at least pa_prefill_workspace_size() bytes that holds the
 * normalised, rotated BF16 k^ of every cached key between the two kernels of the call.  Asynchronous
 * on `stream`.  Concurrent calls need separate workspaces.  Prefill runs one pass per
 * (query block, head); a plan whose policy is not PA_SPLIT_DISABLED gets PA_ERR_UNSUPPORTED. */
pa_status pa_prefill(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages,
                     int32_t num_indices, const int32_t* kv_indptr, const int32_t* kv_indices,
                     const int32_t* kv_last_page_len, const int32_t* cache_position,
                     const int32_t* query_position_ids, const int32_t* key_position_ids,
                     const void* q, const void* k_cache, const void* v_cache,
                     const float* q_norm_weight, const float* k_norm_weight,
                     void* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Workspace bytes of pa_prefill_backward for these sizes (host arithmetic only). */
pa_status pa_prefill_backward_workspace_size(pa_plan_t plan, int32_t batch, int32_t seq_len, size_t* bytes);

/* Deterministic backward of full-prefill attention, the training layout ([PR279] "Scope":
 * the strict path requires a deterministic backward, dropout 0; [PR7] "Goal", "Original PR7
 * Requirements": the training forward is full prefill, dq/dk/dv belong to its backward).
 * The forward it differentiates is pa_prefill's arithmetic on dense inputs: row b's keys are
 * its own seq_len tokens, token i has its query and its key at positions[b][i], key j is
 * visible to query i iff positions[b][j] <= positions[b][i].  The BF16 roundings of q^, k^
 * (the post-RoPE boundary) and of out pass gradients through unchanged.
 *   positions          int32 [B, S]        in [0, table_rows); a token out of range gets NaN
 *                                          gradients.
 *   q                  bf16 [B, Hq, S, 128]   pre-norm, pre-RoPE.
 *   k, v               bf16 [B, Hkv, S, 128]  k pre-norm, pre-RoPE.
 *   q_norm_weight, k_norm_weight  fp32 [128] or NULL (no RMSNorm on that side).
 *   out, lse           the forward's results: bf16 [B, Hq, S, 128], fp32 [B, Hq, S].
 *   dout               bf16 [B, Hq, S, 128]   gradient of out.
 *   dq                 fp32 [B, Hq, S, 128]   written.
 *   dk, dv             fp32 [B, Hkv, S, 128]  written.
 *   dq_norm_weight, dk_norm_weight  fp32 [128], written when the matching norm weight is
 *                      given (required then), else ignored.
 *   workspace          at least pa_prefill_backward_workspace_size() bytes, any contents.
 * Every sum runs in a fixed order with no atomics: dk and dv of a key sum over the group's
 * query heads in ascending order and over query tiles in ascending order, dq over key tiles in
 * ascending order, the weight gradients over fixed shares in a fixed order; results are
 * bitwise repeatable.  Kernels on `stream` only (three, then a few small ones that sum the
 * weight gradients), no allocation, no synchronisation, no memset.  Requires
 * a PA_SPLIT_DISABLED plan with batch <= max_batch and seq_len <= max_q_len. */
pa_status pa_prefill_backward(pa_plan_t plan, int32_t batch, int32_t seq_len, const int32_t* positions,
                              const void* q, const void* k, const void* v, const float* q_norm_weight,
                              const float* k_norm_weight, const void* out, const float* lse, const void* dout,
                              float* dq, float* dk, float* dv, float* dq_norm_weight, float* dk_norm_weight,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Build the CSR block table on the device from a dense one ([PR162] "Design notes": CSR
 * metadata built once per traversal, fixed-shape and device-only; "Code audit", "Data
 * flows checked": indptr = running sum of ceil(len / 16), compact indices by a fixed-shape
 * scatter, rows without keys get last_page_len 1, no host synchronisation).
 *   batch, width       B >= 0 rows of a table `width` >= 1 pages wide (B * width and
 *                      width * 16 must fit in int32).
 *   block_table        int32 [B, width]   row b's physical pages in logical order; entries
 *                                         past the row's pages are ignored (-1 by
 *                                         convention).
 *   kv_lens            int32 [B]          keys in the cache per row (L_b).
 *   kv_indptr          int32 [B + 1]      written: kv_indptr[b + 1] - kv_indptr[b] =
 *                                         ceil(L_b / 16).
 *   kv_indices         int32 [B * width]  written: the first ceil(L_b / 16) table entries of
 *                                         each row, rows back to back; slots from
 *                                         kv_indptr[B] on are set to -1.
 *   kv_last_page_len   int32 [B]          written: L_b - 16 (ceil(L_b / 16) - 1), or 1 for
 *                                         a row with no keys.
 * A length outside [0, 16 * width] cannot be represented: that row takes its whole table row
 * and last_page_len 0, which pa_validate_metadata reports (PA_ERR_LAST_PAGE_LEN) and which
 * pa_decode / pa_prefill turn into NaN for the row.  The outputs fit the other entry points
 * directly, with num_indices = B * width (the compact count kv_indptr[B] stays on the
 * device; pa_validate_metadata needs it exactly).  Two kernels on `stream`, no allocation,
 * no synchronisation, no memset: capturable in a HIP graph.  Errors: PA_ERR_INVALID_ARGUMENT
 * for sizes out of range or a NULL pointer (kv_indptr is always written, so it may not be
 * NULL even for B = 0). */
pa_status pa_build_csr(int32_t batch, int32_t width, const int32_t* block_table, const int32_t* kv_lens,
                       int32_t* kv_indptr, int32_t* kv_indices, int32_t* kv_last_page_len, void* stream);

/* The table width a plan should be made for: the smallest power of two >= width ([PR162]
 * "Design notes": plans keyed by a power-of-two width bucket, so a growing context makes
 * few plans).  Host arithmetic only; width in [1, 2^30], else PA_ERR_INVALID_ARGUMENT. */
pa_status pa_width_bucket(int32_t width, int32_t* bucket);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
