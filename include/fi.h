/*
 * fi.h -- C ABI of a gfx950 (MI355X) library for batched attention over a
 * paged KV cache viewed as a block-sparse-row (BSR) matrix.
 *
 * Source of the operations: the FlashInfer (MLSys 2025) pages.
 *   - Serving-engine page (infra.bea.ai guide), section 2 "Page-Level
 *     Attention" and "Ragged Batching", section 3 "Cascade Attention for
 *     Shared Prefixes" and "FlashDecoding: Parallel KV Split", section 4 "The
 *     Interface": the paged KV cache, the index arrays kv_indptr / kv_indices
 *     / kv_last_page_len, batch decode, causal batch prefill, the shared-prefix
 *     cascade with merge_state.
 *   - Paper page (fdeinterviews.com), "One format for every KV layout" (BSR,
 *     composable formats), "Customizable attention" (logits soft-cap, query
 *     tile size from the average query length), "Load balancing that survives
 *     CUDA graphs" (CPU-side plan, equal KV chunks, partial-result slots,
 *     fixed-grid persistent kernels, log-sum-exp merge).
 *   - Talk page (greptalks.com), "Runtime Scheduler for Dynamic Problem
 *     Shapes" (inspector-executor: plan, then run) and "Head Group Packing".
 *
 * Conventions for every call.
 *   - Pointers marked "host" are CPU memory; "device" are GPU memory.  The
 *     caller owns every buffer; the library allocates no device memory.
 *     Run calls never synchronise: they only enqueue work on `stream` (a
 *     hipStream_t passed as void*; NULL means the null stream).  Only
 *     fi_read_status waits.
 *   - The KV pool has shape [pool_pages, 2, page_size, num_kv_heads,
 *     head_dim] (axis 1: 0 = K, 1 = V); row-major, contiguous.
 *   - Request i owns pages kv_indices[kv_indptr[i] .. kv_indptr[i+1]) in
 *     logical order; its last page holds kv_last_page_len[i] valid tokens
 *     (1..page_size; ignored when the request has no page), so
 *     kv_len_i = (pages_i - 1) * page_size + kv_last_page_len[i], or 0.
 *   - Query head h reads KV head h / (num_qo_heads / num_kv_heads).
 *   - Causal alignment is bottom-right: query token t of a request with
 *     qo_len queries sees keys j <= kv_len - qo_len + t.
 *   - Logits: s = sm_scale * q.k, then s = cap * tanh(s / cap) when the cap
 *     is positive.  lse is the natural-log log-sum-exp of the logits a query
 *     row saw; a row that sees no key gets o = 0 and lse = -inf.
 *   - Return value: FI_OK or a negative FI_ERR_* code.  On error nothing is
 *     launched and outputs are untouched; fi_last_error() returns a
 *     thread-local message.  No C++ exception crosses this ABI.
 */
#ifndef FI_H_
#define FI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FI_OK 0
#define FI_ERR_INVALID_ARG (-1)        /* malformed sizes, index arrays or pointers */
#define FI_ERR_UNSUPPORTED (-2)        /* dtype / head_dim / group size not built */
#define FI_ERR_WORKSPACE_TOO_SMALL (-3) /* plan buffer or float workspace too small */
#define FI_ERR_PLAN_MISMATCH (-4)      /* plan built for other shapes or corrupted */
#define FI_ERR_HIP (-5)                /* a HIP runtime call failed */

typedef enum fi_dtype { FI_F32 = 0, FI_BF16 = 1 } fi_dtype;

/* Stream selector of fi_default_workers. */
#define FI_KIND_DECODE 0
#define FI_KIND_PREFILL 1

/*
 * fi_plan inputs.  Defines the work partition of one generation step
 * (paper page, "Load balancing that survives CUDA graphs"; talk page, the
 * plan function of the scheduler abstraction).
 *   batch_size        B >= 0
 *   qo_indptr         host int32 [B+1], or NULL: every request has one query
 *                     (decode).  qo_len 0 = no query, 1 = decode row,
 *                     >= 2 = prefill tiles.
 *   kv_indptr         host int32 [B+1], kv_indptr[0] == 0, non-decreasing
 *   kv_last_page_len  host int32 [B]
 *   page_size         >= 1
 *   num_qo_heads, num_kv_heads: num_qo_heads % num_kv_heads == 0 and the
 *                     group size G = num_qo_heads / num_kv_heads in {1,2,4,8}
 *   head_dim          64 or 128
 *   causal            0 or 1 (binds requests with qo_len >= 2)
 *   workers_decode, workers_prefill: persistent workers per KV head of the
 *                     decode and prefill kernels (grid = workers x KV heads)
 *   min_seg_pages     >= 1, pages past its fixed cost in the smallest segment
 *                     of a stream one worker owns.  Cost units: a work item
 *                     (a row's pages on one worker) costs its pages plus
 *                     ceil(32 / page_size) for a decode row, ceil(512 /
 *                     page_size) for a prefill tile
 *   br_override       0 (tile rows from the mean query length) or 16/32/64/128
 *   no_split          1: one item per row, no partial slots (unsplit reference)
 *   window_left       -1: no window.  >= 0: sliding-window attention, the
 *                     query at position p = kv_len - qo_len + t sees no key
 *                     before p - window_left (paper page: sliding windows
 *                     among the attention variants of its opening paragraph;
 *                     "Customizable attention": a variant is a logits mask).
 *                     The plan drops every page no query of a row can see and
 *                     records the window; the run calls apply it.  Every
 *                     request needs kv_len + qo_len < 2^30 (else
 *                     FI_ERR_UNSUPPORTED).  The cascade call takes no
 *                     windowed plan.
 */
typedef struct fi_plan_in {
  int32_t batch_size;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_last_page_len;
  int32_t page_size;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t causal;
  int32_t workers_decode;
  int32_t workers_prefill;
  int32_t min_seg_pages;
  int32_t br_override;
  int32_t no_split;
  int32_t window_left;
} fi_plan_in;

/* Summary of a plan (also recorded inside the plan buffer). */
typedef struct fi_plan_info {
  int64_t plan_ints;        /* int32 words written to the plan buffer */
  int64_t float_ws_bytes;   /* float workspace the run calls need */
  int32_t decode_rows, decode_items, decode_slots, decode_segment_pages;
  int32_t prefill_rows, prefill_items, prefill_slots, prefill_segment_pages; /* segments in cost units */
  int32_t prefill_tile_rows; /* BR: packed (token, head) rows per prefill tile */
} fi_plan_info;

/*
 * Build the plan on the host (no HIP call).  `plan` is a host int32 buffer
 * of `plan_capacity` words, owned by the caller; size it with
 * fi_plan_bounds.  The caller copies plan[0 .. info.plan_ints) to a device
 * buffer before the run calls; one plan serves every layer of a step.
 * `info` may be NULL.  Errors: FI_ERR_INVALID_ARG, FI_ERR_UNSUPPORTED,
 * FI_ERR_WORKSPACE_TOO_SMALL (capacity).
 */
int fi_plan(const fi_plan_in* in, int32_t* plan, int64_t plan_capacity, fi_plan_info* info);

/*
 * Upper bounds, from shapes and worker counts only, of the plan buffer
 * (int32 words) and of the float workspace (bytes) for any batch of at most
 * `batch_size` requests and `total_qo` queries.  Buffers sized this way stay
 * valid for every later step, so device pointers can stay fixed.
 */
int fi_plan_bounds(int32_t batch_size, int64_t total_qo, int32_t num_qo_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t workers_decode,
                   int32_t workers_prefill, int64_t* plan_ints, int64_t* float_ws_bytes);

/*
 * Attention parameters of the run calls.
 *   dtype      storage type of q and kv_pool (FI_F32 or FI_BF16)
 *   out_dtype  storage type of o (FI_F32 or FI_BF16; bf16 rounds to nearest even)
 *   sm_scale   logit scale; <= 0 selects 1/sqrt(head_dim)
 *   logits_soft_cap  cap of s = cap * tanh(s / cap); 0 disables it
 *   graph_safe nonzero: every kernel of the call is launched whether or not
 *              this plan gives it work (kernels without work exit at once),
 *              so a call captured into a HIP graph stays valid when replayed
 *              with any later plan of the same shapes and worker counts
 *              (paper page, "Load balancing that survives CUDA graphs":
 *              persistent kernels with fixed grids replayed inside a
 *              captured graph).  0: kernels without work are not launched.
 *   rope_theta > 0: fused rotary embedding of q and k inside the kernels
 *              (paper page: fused rotary embeddings among the attention
 *              variants of its opening paragraph; "Customizable attention":
 *              a query / key transform).  Rotate-half form: for d < D/2 the
 *              pair (x[d], x[d + D/2]) turns by pos / rope_scale *
 *              rope_theta^(-2d/D); key j of a request sits at position j,
 *              query t at kv_len - qo_len + t.  The cache holds keys before
 *              rotation; v is not rotated.  With bf16 storage the rotated
 *              q and k are rounded to fp16 (round to nearest even,
 *              components saturating at +-65504) for the QK^T product;
 *              fp32 stays fp32.  <= 0: off.
 *   rope_scale position divisor of the rotary embedding; <= 0 means 1.
 *              The cascade call takes no rotary embedding (its levels do not
 *              carry the keys' positions): FI_ERR_UNSUPPORTED.
 */
typedef struct fi_attn_params {
  fi_dtype dtype;
  fi_dtype out_dtype;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  float sm_scale;
  float logits_soft_cap;
  int32_t graph_safe;
  float rope_theta;
  float rope_scale;
  /* Tree mask of speculative decoding (paper page, opening paragraph: trees
   * of guesses verified by speculative decoding; serving-engine page, token
   * trees among the KV layouts), fi_batch_prefill_paged only; NULL = none.
   * The qo_len query tokens of request i are its draft tokens, stored as its
   * last qo_len keys (the bottom-right alignment of the causal mask).  Bit
   * t * qo_len + u of the request's block, which starts at bit
   * mask_indptr[i] of the stream, lets draft token t see draft token u.  A
   * query always sees the keys before the draft and its own key, never a
   * later draft token (bits with u > t are ignored); a request with one
   * query ignores its bit.  Needs a causal plan without a sliding window and
   * no rotary embedding (else FI_ERR_UNSUPPORTED).
   *   tree_mask    device uint32 words; bit n of the stream is bit n % 32 of
   *                word n / 32 (the little-endian bit order of a byte array
   *                padded to whole words); holds ceil(mask_bits / 32) words
   *   mask_indptr  device int32 [batch + 1]: mask_indptr[0] = 0 and
   *                mask_indptr[i + 1] - mask_indptr[i] = qo_len_i^2 (not
   *                checked on the device; bits past mask_bits are not read)
   *   mask_bits    total bits, mask_indptr[batch]; 1 <= mask_bits < 2^31 */
  const uint32_t* tree_mask;
  const int32_t* mask_indptr;
  int64_t mask_bits;
} fi_attn_params;

/*
 * The float workspace (float_ws) of the run calls.  Its first
 * fi_plan_info.float_ws_bytes bytes (fi_cascade_workspace_bytes for the
 * cascade) hold a control region -- the status word and reserved words, 256
 * bytes at the start whatever the plan -- then the partial results of split
 * rows.  Zero-fill the control region once, when the workspace is allocated;
 * one workspace then serves any number of later calls and plans, in stream
 * order.  Calls that run at the same time must not share a workspace.
 *
 * Status word (word 0 of the workspace; of the cascade's workspace for both
 * of its levels): bit flags the kernels OR in and never clear.
 *   FI_STATUS_BAD_PAGE  a page id at or past pool_pages was read; the kernels
 *                       read page 0 in its place (never outside the pool), so
 *                       the rows that saw it hold wrong values.
 */
#define FI_STATUS_BAD_PAGE 1

/*
 * Batch decode over the paged KV cache: one query token per request
 * (serving-engine page, "The Interface", batch_decode_with_paged_kv_cache;
 * GQA head group packing; FlashDecoding split of long requests merged by
 * log-sum-exp composition).
 *   plan_host / plan_dev  the same plan, built with qo_indptr == NULL, on the
 *                         host and its device copy
 *   q           device [B, num_qo_heads, head_dim] (dtype)
 *   kv_pool     device [pool_pages, 2, page_size, num_kv_heads, head_dim]
 *   kv_indptr, kv_indices, kv_last_page_len: device int32 copies of the index
 *               arrays the plan was built from (kv_indices ids < pool_pages)
 *   o           device [B, num_qo_heads, head_dim] (out_dtype)
 *   lse         device float [B, num_qo_heads], or NULL
 *   float_ws    device workspace of at least float_ws_bytes (fi_plan_info),
 *               zero-filled when first used (see above)
 *   pool_pages  >= 1 whenever some row of the plan sees a KV page; kv_pool
 *               and kv_indices may be NULL only when none does
 * Launches the persistent decode kernel (grid workers_decode x num_kv_heads)
 * and the partial-merge kernel on `stream`.
 */
int fi_batch_decode_paged(const int32_t* plan_host, const int32_t* plan_dev,
                          const fi_attn_params* params, const void* q, const void* kv_pool,
                          int64_t pool_pages, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_last_page_len, void* o,
                          float* lse, void* float_ws, int64_t float_ws_bytes, void* stream);

/*
 * Ragged batch prefill over the paged KV cache (serving-engine page, "The
 * Interface", batch_prefill_with_paged_kv_cache(..., causal=True); "Ragged
 * Batching"; "Prefill-Decode Mixing").  Requests with one query run in the
 * decode kernel, requests with two or more in the MFMA prefill kernel, inside
 * this one call; the causal flag is the plan's.
 *   qo_indptr   device int32 [B+1], the array the plan was built from
 *   q, o        device [total_qo, num_qo_heads, head_dim]; lse [total_qo, num_qo_heads] or NULL
 * Other arguments as fi_batch_decode_paged.
 * Numeric range of the prefill kernel (requests with two or more queries;
 * also fi_cascade's level 0): V takes part in the P.V product as fp16, so
 * bf16 values of V are exact for 2^-17 <= |v| <= 65504 and zero; smaller
 * ones are rounded to fp16's subnormal step (2^-24, far below the output
 * tolerance), and larger ones are clamped to +-65504.  Keep |V| <= 65504 on
 * this path.  q and k are not narrowed (bf16 products, fp32 sums) unless the
 * rotary embedding is on (see rope_theta).
 * With a page_size that is not a power of two >= 16, the prefill kernel
 * needs 2 * pool_pages * page_size < 2^32 (a pool below 2^31 tokens), else
 * FI_ERR_UNSUPPORTED before anything runs.
 */
int fi_batch_prefill_paged(const int32_t* plan_host, const int32_t* plan_dev,
                           const fi_attn_params* params, const void* q, const void* kv_pool,
                           int64_t pool_pages, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           const int32_t* kv_last_page_len, void* o, float* lse,
                           void* float_ws, int64_t float_ws_bytes, void* stream);

/*
 * Two-way log-sum-exp merge of attention states of the same query rows
 * (serving-engine page, cascade code block, merge_state; paper page,
 * "log-sum-exp composition").  With M = max(s_a, s_b):
 *   s_out = M + ln(e^(s_a - M) + e^(s_b - M)),
 *   v_out = (e^(s_a - M) v_a + e^(s_b - M) v_b) / (e^(s_a - M) + e^(s_b - M));
 * both -inf gives (0, -inf).
 *   v_a, v_b, v_out  device [n_tokens, n_heads, head_dim] of `dtype`
 *   s_a, s_b, s_out  device float [n_tokens, n_heads] (natural log)
 * v_out may alias v_a or v_b, s_out may alias s_a or s_b.
 */
int fi_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                   void* v_out, float* s_out, int64_t n_tokens, int32_t n_heads,
                   int32_t head_dim, fi_dtype dtype, void* stream);

/*
 * Cascade (composable-format) attention (serving-engine page, "Cascade
 * Attention for Shared Prefixes"; paper page, composable formats: a shared
 * prefix viewed with a large row block, each request's own tokens with
 * single-row blocks; no data moves, only the index arrays differ).
 *   Level 0: the queries of a group, stacked as one ragged request, attend
 *            non-causally to the group's shared pages.  plan0 is built with
 *            qo_indptr0 (groups over the query rows of q) and causal = 0.
 *   Level 1: each request's queries attend to its own pages (plan1, built
 *            with qo_indptr1 or NULL for one query per request).
 *   The two states are merged into o / lse.
 *   q     device [total_qo, num_qo_heads, head_dim]; level 0 and level 1 index
 *         the same query rows (level-0 group k holds rows qo_indptr0[k] ..
 *         qo_indptr0[k+1])
 *   o     device [total_qo, num_qo_heads, head_dim] (out_dtype); lse may be NULL
 *   float_ws  at least fi_cascade_workspace_bytes(...)
 */
int fi_cascade(const int32_t* plan0_host, const int32_t* plan0_dev, const int32_t* qo_indptr0,
               const int32_t* kv_indptr0, const int32_t* kv_indices0,
               const int32_t* kv_last_page_len0, const int32_t* plan1_host,
               const int32_t* plan1_dev, const int32_t* qo_indptr1,
               const int32_t* kv_indptr1, const int32_t* kv_indices1,
               const int32_t* kv_last_page_len1, const fi_attn_params* params, const void* q,
               const void* kv_pool, int64_t pool_pages, void* o, float* lse, void* float_ws,
               int64_t float_ws_bytes, void* stream);

/* Float workspace fi_cascade needs for these two plans (bytes, or < 0 on error). */
int64_t fi_cascade_workspace_bytes(const int32_t* plan0_host, const int32_t* plan1_host);

/*
 * Paged KV append: write a step's new K/V tokens into their pages (talk page,
 * Background, "Dynamic Problem Shapes": the append stage, adding new tokens
 * to the KV cache; serving-engine page, "Page-Level Attention": a request's
 * tokens fill the pages of its page table in order, page_size tokens per
 * page).
 * The index arrays describe each request's pages after the append: request
 * i holds kv_len_i = (pages_i - 1) * page_size + kv_last_page_len[i] tokens
 * (0 without pages), and its n_i = append_indptr[i+1] - append_indptr[i] new
 * tokens are the last n_i of them.  New token t goes to position
 * p = kv_len_i - n_i + t: page kv_indices[kv_indptr[i] + p / page_size],
 * slot p % page_size, K at index 0 and V at index 1 of the pool's axis 1.
 *   append_k, append_v  device [n_tokens, num_kv_heads, head_dim] (dtype)
 *   append_indptr       device int32 [batch_size + 1], append_indptr[0] = 0,
 *                       append_indptr[batch_size] = n_tokens, non-decreasing
 *   kv_pool             device [pool_pages, 2, page_size, num_kv_heads,
 *                       head_dim] (dtype), written in place
 *   kv_indptr, kv_indices (kv_indices_len entries), kv_last_page_len:
 *                       device int32 arrays of the page table
 * Library contract beyond the pages (which define no such input): on the
 * device, a token whose position would be negative (more new tokens than
 * the request holds), whose page-table entry lies outside kv_indices, or
 * whose page id is not below pool_pages is not written, and nothing else of
 * the pool changes.  Returns
 * FI_ERR_INVALID_ARG for negative sizes, null pointers with tokens to write,
 * or buffers that are not 16-byte aligned; FI_ERR_UNSUPPORTED for a dtype
 * other than FI_F32 / FI_BF16 or a token row (num_kv_heads * head_dim
 * elements) that is not a multiple of 16 bytes.  Nothing is launched on
 * error, nor when n_tokens is 0.
 */
int fi_append_paged_kv(const void* append_k, const void* append_v, fi_dtype dtype,
                       const int32_t* append_indptr, int32_t batch_size, int64_t n_tokens,
                       void* kv_pool, int64_t pool_pages, int32_t page_size, int32_t num_kv_heads,
                       int32_t head_dim, const int32_t* kv_indptr, const int32_t* kv_indices,
                       int64_t kv_indices_len, const int32_t* kv_last_page_len, void* stream);

/*
 * Batch decode that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  As fi_batch_decode_paged, except that
 * the float workspace is a static device array of the library, one per GPU,
 * FI_NOALLOC_SCRATCH_BYTES long, held from load to process end.  A plan whose
 * decode stream needs more (its control region plus 2 (workers_decode - 1)
 * partial slots of num_qo_heads x head_dim floats and their lse) is refused
 * with FI_ERR_WORKSPACE_TOO_SMALL before anything runs.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU race, so keep them
 * in one stream order.  Its status word is read with fi_read_status(NULL,
 * ...) on the same device.  Never calls hipMalloc, hipFree or an allocating
 * routine.
 */
#define FI_NOALLOC_SCRATCH_BYTES (16 << 20)
int fi_batch_decode_paged_noalloc(const int32_t* plan_host, const int32_t* plan_dev,
                                  const fi_attn_params* params, const void* q,
                                  const void* kv_pool, int64_t pool_pages,
                                  const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* kv_last_page_len, void* o, float* lse,
                                  void* stream);

/*
 * Read the status word of a float workspace into *status (host int32), and
 * reset it to 0 afterwards if `clear` is nonzero.  Unlike the run calls this
 * one waits: it synchronises `stream`, so call it after the run calls whose
 * status is wanted, with none in flight on another stream.  float_ws NULL
 * reads the static scratch of fi_batch_decode_paged_noalloc on the current
 * device.  Errors: FI_ERR_INVALID_ARG (null status), FI_ERR_HIP.
 */
int fi_read_status(const void* float_ws, int32_t* status, int32_t clear, void* stream);

/* Thread-local message of the last error of this thread ("" if none). */
const char* fi_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int fi_version(void);

/*
 * Suggested workers per KV head for a kind (FI_KIND_DECODE / FI_KIND_PREFILL)
 * on a GPU with `num_cus` compute units, so that the fixed grid
 * workers x num_kv_heads fills the chip in one wave of workgroups.
 */
int fi_default_workers(int kind, int num_cus, int num_kv_heads);

#ifdef __cplusplus
}
#endif

#endif /* FI_H_ */
