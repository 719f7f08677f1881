/*
 * attn_ref.c -- plain fp64 CPU oracle for batched attention over a paged KV
 * cache viewed as a block-sparse-row matrix.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header or helper with the GPU
 * path.
 *
 * What it computes (FlashInfer MLSys 2025 pages):
 *   - page table walk: request i's logical token j lives in physical page
 *     kv_indices[kv_indptr[i] + j / P] at slot j % P ("Page-Level Attention",
 *     the request 0 / request 1 page-table example on the serving-engine page);
 *     the last page holds kv_last_page_len[i] valid tokens (index arrays named
 *     in "The Interface" code block);
 *   - exact attention softmax(s) V over the visible keys, with s = scale * q.k,
 *     an optional logits soft-cap transform s <- cap * tanh(s / cap) (paper
 *     page, "Customizable attention, compiled just in time": soft-capping is
 *     one of its logits transforms), GQA head
 *     grouping (query head h reads KV head h / G, "Head Group Packing"), and the
 *     causal mask of batch prefill (causal=True in "The Interface");
 *   - the (output, log-sum-exp) state of each query row, the quantity that
 *     FlashDecoding partials and merge_state combine ("FlashDecoding: Parallel
 *     KV Split"; paper page, "Load balancing that survives CUDA graphs": the
 *     partial results are combined by log-sum-exp composition).
 *
 * Method: naive per-token page gather and a plain two-pass softmax (max, then
 * exp-sum), all in double precision.  No tiling, no online rescaling.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - KV head of query head h is h / G with G = Hq / Hk (contiguous groups);
 *   - causal alignment is bottom-right: query token t of a request with
 *     qo_len queries and kv_len keys sees keys j <= kv_len - qo_len + t;
 *   - the soft-cap applies to the already-scaled logit;
 *   - a row with no visible key has o = 0 and lse = -inf;
 *   - lse is the natural-log log-sum-exp of the (capped) logits;
 *   - sliding window (paper page, opening paragraph: sliding windows among the
 *     attention variants; "Customizable attention": a variant is a mask):
 *     with window_left >= 0 the query at position kv_len - qo_len + t sees no
 *     key more than window_left positions before it (window_left < 0: no
 *     window).
 *   - fused rotary embedding (paper page, opening paragraph: fused rotary
 *     embeddings among the attention variants; "Customizable attention": a
 *     query / key transform such as RoPE): with rope_theta > 0, q and k are
 *     rotated before the dot product, v is not.  The pages give no formula;
 *     the reading is the rotate-half form: for d < D/2 the pair
 *     (x[d], x[d + D/2]) turns by the angle (pos / rope_scale) *
 *     rope_theta^(-2d/D), where the key j of a request sits at position j and
 *     the query t at kv_len - qo_len + t (the same alignment as the causal
 *     mask).  rope_scale <= 0 means 1.
 *   - tree mask (paper page, opening paragraph: speculative decoding verifies
 *     trees of guesses; "Customizable attention": a variant is a mask; the
 *     token trees of speculative decoding on the talk page, Background and
 *     "Block Sparse Matrix"): with a
 *     mask given, the qo_len query tokens of a request are its draft tokens,
 *     stored as its last qo_len keys (the bottom-right alignment of the
 *     causal mask), and bit t * qo_len + u of the request's bit block
 *     (starting at bit mask_indptr[i], row-major, bit b of byte k is bit
 *     8 k + b) says whether draft token t sees draft token u.  Every query
 *     sees all keys before the draft, always sees itself, and never sees a
 *     later draft token (bits with u > t are ignored), so the mask only
 *     narrows the causal one.  Needs causal = 1; requests with one query
 *     ignore their bit.
 *
 * Parity pins: see the oracle tests (dense brute force, library SDPA, closed
 * forms, the pages' page-table example, page-permutation invariance,
 * split+merge == unsplit, cascade == flat).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define OREF_OK 0
#define OREF_EINVAL -1
#define OREF_ENOMEM -2

static char g_err[256];

const char *oref_last_error(void) { return g_err; }

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the oracle's parallel loops use. */
int oref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the threads of the later parallel loops (n >= 1). */
void oref_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

static int fail(const char *msg, long long a, long long b) {
  snprintf(g_err, sizeof(g_err), "%s (%lld, %lld)", msg, a, b);
  return OREF_EINVAL;
}

/* Number of valid keys of request i: (pages - 1) * P + last_page_len, or 0. */
static int64_t kv_len_of(const int32_t *kv_indptr, const int32_t *last, int i, int P) {
  int64_t np = (int64_t)kv_indptr[i + 1] - kv_indptr[i];
  if (np == 0) return 0;
  return (np - 1) * P + last[i];
}

static int64_t qo_len_of(const int32_t *qo_indptr, int i) {
  return qo_indptr ? (int64_t)qo_indptr[i + 1] - qo_indptr[i] : 1;
}

static int64_t qo_start_of(const int32_t *qo_indptr, int i) {
  return qo_indptr ? (int64_t)qo_indptr[i] : (int64_t)i;
}

/*
 * Validate the index arrays (written separately from the library's own checks).
 * Rules: B >= 0; indptr[0] == 0 and non-decreasing; 1 <= last <= P for a
 * request with pages; page ids in [0, pool_pages); Hq % Hk == 0; causal needs
 * qo_len <= kv_len for a request with two or more queries (a single-query
 * request may have an empty cache: its row then sees no key).
 */
int oref_validate(int B, const int32_t *qo_indptr, const int32_t *kv_indptr,
                  const int32_t *kv_indices, const int32_t *kv_last_page_len, int P,
                  int Hq, int Hk, int D, int causal, int64_t pool_pages) {
  if (B < 0) return fail("negative batch", B, 0);
  if (P < 1) return fail("page_size < 1", P, 0);
  if (Hq < 1 || Hk < 1 || Hq % Hk != 0) return fail("bad head counts", Hq, Hk);
  if (D < 1) return fail("bad head_dim", D, 0);
  if (kv_indptr[0] != 0) return fail("kv_indptr[0] != 0", kv_indptr[0], 0);
  if (qo_indptr && qo_indptr[0] != 0) return fail("qo_indptr[0] != 0", qo_indptr[0], 0);
  for (int i = 0; i < B; ++i) {
    if (kv_indptr[i + 1] < kv_indptr[i]) return fail("kv_indptr decreases", i, kv_indptr[i + 1]);
    if (qo_indptr && qo_indptr[i + 1] < qo_indptr[i]) return fail("qo_indptr decreases", i, qo_indptr[i + 1]);
    int64_t np = (int64_t)kv_indptr[i + 1] - kv_indptr[i];
    if (np > 0 && (kv_last_page_len[i] < 1 || kv_last_page_len[i] > P))
      return fail("last_page_len out of [1, P]", i, kv_last_page_len[i]);
    for (int64_t p = kv_indptr[i]; p < kv_indptr[i + 1]; ++p)
      if (kv_indices[p] < 0 || kv_indices[p] >= pool_pages) return fail("page id out of pool", i, kv_indices[p]);
    if (causal && qo_len_of(qo_indptr, i) >= 2 &&
        qo_len_of(qo_indptr, i) > kv_len_of(kv_indptr, kv_last_page_len, i, P))
      return fail("causal with qo_len > kv_len", i, qo_len_of(qo_indptr, i));
  }
  return OREF_OK;
}

/* Physical location of logical token j of request i: page id and slot. */
int oref_token_location(const int32_t *kv_indptr, const int32_t *kv_indices, int P, int i,
                        int64_t j, int32_t *page, int32_t *slot) {
  int64_t np = (int64_t)kv_indptr[i + 1] - kv_indptr[i];
  if (j < 0 || j / P >= np) return fail("token beyond the request's pages", i, j);
  *page = kv_indices[kv_indptr[i] + j / P];
  *slot = (int32_t)(j % P);
  return OREF_OK;
}

/*
 * Rotary embedding of one head vector x (length D, even) at position pos:
 * for d < D/2 the pair (x[d], x[d + D/2]) is rotated by the angle
 * pos / scale * theta^(-2d/D).  Writes y; x and y do not overlap.
 */
static void rope_rotate(const double *x, double *y, int D, double pos, double theta,
                        double scale) {
  const int h = D / 2;
  for (int d = 0; d < h; ++d) {
    const double ang = pos / scale * pow(theta, -2.0 * d / D);
    const double c = cos(ang), s = sin(ang);
    y[d] = x[d] * c - x[d + h] * s;
    y[d + h] = x[d + h] * c + x[d] * s;
  }
}

/* Element (page, kv, slot, head, d) of the pool [pages, 2, P, Hk, D]. */
static inline double pool_at(const double *pool, int64_t page, int kv, int64_t slot, int g,
                             int d, int P, int Hk, int D) {
  return pool[((((page * 2 + kv) * P + slot) * Hk) + g) * (int64_t)D + d];
}

/*
 * Attention for an explicit list of query rows (request, token-in-request,
 * query head).  o is [n_rows, D], lse is [n_rows].  q is [total_qo, Hq, D].
 */
/* Whether draft token t of request i sees draft token u under the tree mask. */
static int tree_bit(const uint8_t *mask, const int32_t *mask_indptr, int i, int64_t qo_len,
                    int64_t t, int64_t u) {
  if (u == t) return 1;
  if (u > t) return 0;
  const int64_t b = (int64_t)mask_indptr[i] + t * qo_len + u;
  return (mask[b >> 3] >> (b & 7)) & 1;
}

/* Checks of the tree-mask arrays: causal, and qo_len^2 bits per request. */
static int validate_mask(int B, const int32_t *qo_indptr, int causal, const int32_t *mask_indptr) {
  if (!causal) return fail("a tree mask needs causal attention", 0, 0);
  if (mask_indptr[0] != 0) return fail("mask_indptr[0] != 0", mask_indptr[0], 0);
  for (int i = 0; i < B; ++i) {
    const int64_t n = qo_len_of(qo_indptr, i);
    if ((int64_t)mask_indptr[i + 1] - mask_indptr[i] != n * n)
      return fail("mask_indptr step != qo_len^2", i, (int64_t)mask_indptr[i + 1] - mask_indptr[i]);
  }
  return OREF_OK;
}

int oref_attention_rows(int B, const int32_t *qo_indptr, const int32_t *kv_indptr,
                        const int32_t *kv_indices, const int32_t *kv_last_page_len, int P,
                        int Hq, int Hk, int D, int causal, double sm_scale, double soft_cap,
                        int window_left, double rope_theta, double rope_scale,
                        const uint8_t *tree_mask, const int32_t *mask_indptr,
                        const double *q, const double *pool, int64_t pool_pages,
                        int64_t n_rows, const int32_t *row_req, const int32_t *row_tok,
                        const int32_t *row_head, double *o, double *lse) {
  int rc = oref_validate(B, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, P, Hq, Hk, D,
                         causal, pool_pages);
  if (rc) return rc;
  if (tree_mask && (rc = validate_mask(B, qo_indptr, causal, mask_indptr))) return rc;
  const int rope = rope_theta > 0.0;
  if (rope && D % 2) return fail("rotary embedding needs an even head_dim", D, 0);
  if (rope_scale <= 0.0) rope_scale = 1.0;
  for (int64_t r = 0; r < n_rows; ++r) {
    int i = row_req[r];
    if (i < 0 || i >= B) return fail("row request out of range", r, i);
    if (row_tok[r] < 0 || row_tok[r] >= qo_len_of(qo_indptr, i)) return fail("row token out of range", r, row_tok[r]);
    if (row_head[r] < 0 || row_head[r] >= Hq) return fail("row head out of range", r, row_head[r]);
  }
  const int G = Hq / Hk;
  int rc_all = OREF_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int i = row_req[r];
    const int t = row_tok[r];
    const int h = row_head[r];
    const int g = h / G;
    const int64_t kv_len = kv_len_of(kv_indptr, kv_last_page_len, i, P);
    const int64_t qo_len = qo_len_of(qo_indptr, i);
    const int64_t limit = causal ? kv_len - qo_len + t + 1 : kv_len;
    /* sliding window: the query sits at position kv_len - qo_len + t and
       sees no key more than window_left positions before it */
    int64_t first = 0;
    if (window_left >= 0 && kv_len - qo_len + t - window_left > 0) first = kv_len - qo_len + t - window_left;
    const double *qrow = q + ((qo_start_of(qo_indptr, i) + t) * (int64_t)Hq + h) * D;
    double *orow = o + r * (int64_t)D;
    if (limit <= first) {
      for (int d = 0; d < D; ++d) orow[d] = 0.0;
      lse[r] = -INFINITY;
      continue;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)(limit - first));
    double *qrot = (double *)malloc(sizeof(double) * (size_t)D * 3);
    if (!s || !qrot) {
      free(s);
      free(qrot);
#pragma omp critical
      rc_all = OREF_ENOMEM;
      continue;
    }
    /* rotary embedding: the query at its position, each key at its own */
    double *kraw = qrot + D, *krot = qrot + 2 * D;
    if (rope) rope_rotate(qrow, qrot, D, (double)(kv_len - qo_len + t), rope_theta, rope_scale);
    const double *qv = rope ? qrot : qrow;
    /* tree mask: draft keys (the last qo_len) outside the query's branch */
    const int64_t draft0 = kv_len - qo_len;
    const int masked = tree_mask && qo_len >= 2;
#define OREF_HIDDEN(j) (masked && (j) >= draft0 && !tree_bit(tree_mask, mask_indptr, i, qo_len, t, (j) - draft0))
    /* pass 1: logits of every visible key, gathered one token at a time */
    double m = -INFINITY;
    for (int64_t j = first; j < limit; ++j) {
      if (OREF_HIDDEN(j)) continue;
      int64_t page = kv_indices[kv_indptr[i] + j / P];
      int64_t slot = j % P;
      for (int d = 0; d < D; ++d) kraw[d] = pool_at(pool, page, 0, slot, g, d, P, Hk, D);
      if (rope) rope_rotate(kraw, krot, D, (double)j, rope_theta, rope_scale);
      const double *kv = rope ? krot : kraw;
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qv[d] * kv[d];
      acc *= sm_scale;
      if (soft_cap > 0.0) acc = soft_cap * tanh(acc / soft_cap);
      s[j - first] = acc;
      if (acc > m) m = acc;
    }
    /* pass 2: normaliser and weighted sum of values */
    double z = 0.0;
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    for (int64_t j = first; j < limit; ++j) {
      if (OREF_HIDDEN(j)) continue;
      int64_t page = kv_indices[kv_indptr[i] + j / P];
      int64_t slot = j % P;
      double w = exp(s[j - first] - m);
      z += w;
      for (int d = 0; d < D; ++d) orow[d] += w * pool_at(pool, page, 1, slot, g, d, P, Hk, D);
    }
    for (int d = 0; d < D; ++d) orow[d] /= z;
    lse[r] = m + log(z);
#undef OREF_HIDDEN
    free(s);
    free(qrot);
  }
  return rc_all;
}

/*
 * Every query row of the batch: o is [total_qo, Hq, D], lse is [total_qo, Hq].
 */
int oref_attention(int B, const int32_t *qo_indptr, const int32_t *kv_indptr,
                   const int32_t *kv_indices, const int32_t *kv_last_page_len, int P, int Hq,
                   int Hk, int D, int causal, double sm_scale, double soft_cap, int window_left,
                   double rope_theta, double rope_scale, const uint8_t *tree_mask,
                   const int32_t *mask_indptr, const double *q, const double *pool,
                   int64_t pool_pages, double *o, double *lse) {
  int64_t total = 0;
  for (int i = 0; i < B; ++i) total += qo_len_of(qo_indptr, i);
  int64_t n = total * Hq;
  int32_t *rq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
  int32_t *rt = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
  int32_t *rh = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
  if (!rq || !rt || !rh) {
    free(rq); free(rt); free(rh);
    return OREF_ENOMEM;
  }
  int64_t r = 0;
  for (int i = 0; i < B; ++i)
    for (int64_t t = 0; t < qo_len_of(qo_indptr, i); ++t)
      for (int h = 0; h < Hq; ++h) {
        rq[r] = i; rt[r] = (int32_t)t; rh[r] = h; ++r;
      }
  int rc = oref_attention_rows(B, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, P, Hq, Hk,
                               D, causal, sm_scale, soft_cap, window_left, rope_theta, rope_scale,
                               tree_mask, mask_indptr, q, pool, pool_pages, n,
                               rq, rt, rh, o, lse);
  free(rq); free(rt); free(rh);
  return rc;
}

/*
 * Combine k attention states of the same query rows by log-sum-exp
 * composition ("merge_state" in the cascade code block; the FlashDecoding
 * merge step).  o_parts is [k, n, D], lse_parts is [k, n]; results are
 * [n, D] and [n].  With M = max lse_k:
 *   lse = M + ln sum_k exp(lse_k - M),  o = sum_k exp(lse_k - lse) o_k.
 * If every lse_k is -inf the result is (0, -inf).
 */
int oref_merge_states(int k, int64_t n, int D, const double *o_parts, const double *lse_parts,
                      double *o_out, double *lse_out) {
  if (k < 1 || n < 0 || D < 1) return fail("bad merge sizes", k, n);
  for (int64_t r = 0; r < n; ++r) {
    double M = -INFINITY;
    for (int c = 0; c < k; ++c) {
      double v = lse_parts[(int64_t)c * n + r];
      if (v > M) M = v;
    }
    double *orow = o_out + r * (int64_t)D;
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (M == -INFINITY) {
      lse_out[r] = -INFINITY;
      continue;
    }
    double z = 0.0;
    for (int c = 0; c < k; ++c) z += exp(lse_parts[(int64_t)c * n + r] - M);
    double L = M + log(z);
    for (int c = 0; c < k; ++c) {
      double w = exp(lse_parts[(int64_t)c * n + r] - L);
      const double *src = o_parts + ((int64_t)c * n + r) * D;
      for (int d = 0; d < D; ++d) orow[d] += w * src[d];
    }
    lse_out[r] = L;
  }
  return OREF_OK;
}
