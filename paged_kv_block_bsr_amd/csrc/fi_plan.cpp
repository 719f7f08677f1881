// fi_plan.cpp -- the CPU-side inspector: splits each step's work into
// segments of equal cost, one per persistent worker, and records where partial
// results go (FlashInfer paper page, "Load balancing that survives CUDA
// graphs"; talk page, "Runtime Scheduler for Dynamic Problem Shapes": a cost
// model inspected ahead of time, deterministic balance, no tail wave).
//
// Cost model: one unit per visible KV page of a work item, plus a fixed
// charge in keys, rounded up to pages, for the work an item does whatever its
// length (loading its queries, writing its output rows or partial results):
// kTileCostKeys for an item of a prefill tile, kDecodeItemCostKeys for one
// of a decode row.  Rows are decode rows (one query token, the G heads
// of a KV head packed together) and prefill tiles of BR packed (token, head)
// rows; BR follows the batch's mean packed query length (paper page, the query
// tile size of the JIT paragraph).  The two kinds form separate streams
// because they run in different kernels.
//
// Host only: no HIP call.  O(B + rows + items + W) time.
#include <climits>
#include <cstdint>
#include <cstring>
#include <vector>

#include "fi.h"
#include "fi_internal.h"
#include "plan_format.h"

namespace fi {
namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int32_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return (int32_t)p;
}

inline int64_t align64(int64_t n) { return ceil_div(n, 64) * 64; }

// Fixed cost of a prefill work item, in keys (rounded up to pages).  On the
// 16 causal prefills of the mixed ragged step (page 16) the prefill kernel
// takes 0.139 ms with no charge, 0.127-0.129 ms at 512 keys (32 pages), 0.133
// at 256 and 0.128-0.131 from 384 to 1024.
constexpr int64_t kTileCostKeys = 512;
// Fixed cost of a decode work item, in keys: on llama8b_decode the call takes
// 1.5% less time at 32 keys (2 pages of 16) than with pages only, and the same
// at 16 or 64 keys.
constexpr int64_t kDecodeItemCostKeys = 32;

struct Row {
  int32_t req, rb, re, vis;
  int32_t fp;  // first visible page (not part of the rows array)
};

struct StreamPlan {
  int32_t W = 1, S = 1, tile = 0;
  std::vector<Row> rows;
  // items in final order
  std::vector<int32_t> item_row, item_pb, item_pe, item_slot, wip, merge, split;
};

// Greedy fill with segment size S: rows in order go to worker 0 until its
// cost reaches S, then to worker 1, and so on.  Each item (a row's pages on
// one worker) costs h plus its pages.  A worker with S - h or more already
// used takes nothing more; a row that does not fit is cut where the worker
// is full and continues on the next worker, which pays h again.  The last
// worker takes whatever is left.  Returns whether the last worker's cost
// stays within S.  With `emit`, records items (sorted by worker, then row,
// because workers never decrease) and their count per row.
bool fill(StreamPlan& st, int64_t S, int64_t h, bool emit, std::vector<int32_t>& nitems_row) {
  const int32_t W = st.W;
  int64_t w = 0, u = 0;  // current worker and its cost so far
  auto add = [&](int64_t r, int64_t pb, int64_t pe) {
    u += h + (pe - pb);
    if (!emit) return;
    st.item_row.push_back((int32_t)r);
    st.item_pb.push_back((int32_t)pb);
    st.item_pe.push_back((int32_t)pe);
    st.wip[w + 1] += 1;
    nitems_row[r] += 1;
  };
  for (int64_t r = 0; r < (int64_t)st.rows.size(); ++r) {
    const int64_t vis = st.rows[r].vis;
    if (w < W - 1 && S - u <= h) w += 1, u = 0;
    if (vis == 0) {
      add(r, 0, 0);
      continue;
    }
    int64_t pb = 0;
    for (;;) {
      const int64_t take = (w == W - 1) ? vis - pb : std::min<int64_t>(vis - pb, S - u - h);
      add(r, pb, pb + take);
      pb += take;
      if (pb == vis) break;
      w += 1, u = 0;
    }
  }
  return u <= S;
}

// P6 - P8 for one stream.  S is the smallest segment, at least min_seg pages
// past the fixed cost and at least the mean cost per worker, at which the
// greedy fill fits W workers.  lo + 2 h always fits: each worker but the last
// is left holding at least S - h, of which at most h repeats the fixed cost
// of a cut row, so the last one gets at most C - (W - 1)(S - 2 h) + h <= S.
int partition(StreamPlan& st, int32_t min_seg, bool no_split, int64_t h) {
  const int32_t W = st.W;
  const int64_t nrows = (int64_t)st.rows.size();
  int64_t C = 0;
  for (const Row& r : st.rows) C += h + r.vis;
  int64_t lo = std::max<int64_t>(h + min_seg, ceil_div(C, W)), hi = lo + 2 * h;
  std::vector<int32_t> nitems_row(nrows, 0);
  if (!no_split) {
    while (lo < hi) {  // feasibility only grows with S
      const int64_t mid = lo + (hi - lo) / 2;
      if (fill(st, mid, h, false, nitems_row))
        hi = mid;
      else
        lo = mid + 1;
    }
  }
  if (lo > INT32_MAX)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan: segment of %lld cost units too large", (long long)lo);
  st.S = (int32_t)lo;
  const int64_t S = lo;
  st.wip.assign(W + 1, 0);
  st.merge.assign(nrows + 1, 0);

  if (no_split) {
    // one item per row on worker r mod W: counting sort by worker keeps rows ascending
    for (int64_t r = 0; r < nrows; ++r) st.wip[r % W + 1] += 1;
    for (int32_t w = 0; w < W; ++w) st.wip[w + 1] += st.wip[w];
    const int64_t n = nrows;
    st.item_row.assign(n, 0);
    st.item_pb.assign(n, 0);
    st.item_pe.assign(n, 0);
    st.item_slot.assign(n, -1);
    std::vector<int32_t> at(st.wip.begin(), st.wip.end() - 1);
    for (int64_t r = 0; r < nrows; ++r) {
      int32_t k = at[r % W]++;
      st.item_row[k] = (int32_t)r;
      st.item_pe[k] = st.rows[r].vis;
    }
    return FI_OK;  // merge stays all-zero, no split rows
  }

  fill(st, S, h, true, nitems_row);
  for (int32_t w = 0; w < W; ++w) st.wip[w + 1] += st.wip[w];
  // slots: rows with k >= 2 items get k consecutive slots, in page order
  for (int64_t r = 0; r < nrows; ++r) {
    int32_t k = nitems_row[r];
    st.merge[r + 1] = st.merge[r] + (k >= 2 ? k : 0);
    if (k >= 2) st.split.push_back((int32_t)r);
  }
  st.item_slot.assign(st.item_row.size(), -1);
  int32_t prev_row = -1, j = 0;
  for (size_t k = 0; k < st.item_row.size(); ++k) {
    int32_t r = st.item_row[k];
    j = (r == prev_row) ? j + 1 : 0;
    prev_row = r;
    if (nitems_row[r] >= 2) st.item_slot[k] = st.merge[r] + j;
  }
  return FI_OK;
}

int validate(const fi_plan_in& in) {
  const int B = in.batch_size;
  if (B < 0) return set_error(FI_ERR_INVALID_ARG, "fi_plan: batch_size < 0");
  if (in.page_size < 1) return set_error(FI_ERR_INVALID_ARG, "fi_plan: page_size < 1");
  if (in.num_qo_heads < 1 || in.num_kv_heads < 1 || in.num_qo_heads % in.num_kv_heads)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan: num_qo_heads must be a multiple of num_kv_heads");
  if (in.head_dim != 64 && in.head_dim != 128)
    return set_error(FI_ERR_UNSUPPORTED, "fi_plan: head_dim must be 64 or 128");
  const int G = in.num_qo_heads / in.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return set_error(FI_ERR_UNSUPPORTED, "fi_plan: group size must be 1, 2, 4 or 8");
  if (in.workers_decode < 1 || in.workers_prefill < 1)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan: workers must be >= 1");
  if (in.min_seg_pages < 1) return set_error(FI_ERR_INVALID_ARG, "fi_plan: min_seg_pages < 1");
  if (in.br_override != 0 && in.br_override != 16 && in.br_override != 32 &&
      in.br_override != 64 && in.br_override != 128)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan: br_override must be 0, 16, 32, 64 or 128");
  if (in.no_split != 0 && in.no_split != 1) return set_error(FI_ERR_INVALID_ARG, "fi_plan: no_split");
  if (in.window_left < -1) return set_error(FI_ERR_INVALID_ARG, "fi_plan: window_left < -1");
  if (B > 0 && (!in.kv_indptr || !in.kv_last_page_len))
    return set_error(FI_ERR_INVALID_ARG, "fi_plan: null index array");
  if (B == 0 && !in.kv_indptr) return set_error(FI_ERR_INVALID_ARG, "fi_plan: null kv_indptr");
  if (in.kv_indptr[0] != 0) return set_error(FI_ERR_INVALID_ARG, "fi_plan: kv_indptr[0] != 0");
  if (in.qo_indptr && in.qo_indptr[0] != 0) return set_error(FI_ERR_INVALID_ARG, "fi_plan: qo_indptr[0] != 0");
  for (int i = 0; i < B; ++i) {
    int64_t np = (int64_t)in.kv_indptr[i + 1] - in.kv_indptr[i];
    if (np < 0) return set_error(FI_ERR_INVALID_ARG, "fi_plan: kv_indptr decreases at %d", i);
    int64_t qo = in.qo_indptr ? (int64_t)in.qo_indptr[i + 1] - in.qo_indptr[i] : 1;
    if (qo < 0) return set_error(FI_ERR_INVALID_ARG, "fi_plan: qo_indptr decreases at %d", i);
    int32_t last = in.kv_last_page_len[i];
    if (np > 0 && (last < 1 || last > in.page_size))
      return set_error(FI_ERR_INVALID_ARG, "fi_plan: kv_last_page_len[%d] = %d not in [1, %d]", i,
                       last, in.page_size);
    int64_t kv = np == 0 ? 0 : (np - 1) * in.page_size + last;
    if (kv > INT32_MAX) return set_error(FI_ERR_INVALID_ARG, "fi_plan: kv_len of request %d too large", i);
    if (in.causal && qo >= 2 && qo > kv)
      return set_error(FI_ERR_INVALID_ARG, "fi_plan: causal request %d has qo_len %lld > kv_len %lld",
                       i, (long long)qo, (long long)kv);
    if (in.window_left >= 0 && kv + qo >= kWindowMaxTokens)
      return set_error(FI_ERR_UNSUPPORTED, "fi_plan: windowed request %d has kv_len + qo_len >= 2^30", i);
  }
  return FI_OK;
}

// Float workspace regions (float units, each padded to 64 floats = 256 B):
// the control region (status word; fixed place and size),
// then decode partial o, decode partial lse, prefill partial o, prefill
// partial lse.
void ws_layout(int32_t Hq, int32_t Hk, int32_t D, int32_t Wd, int32_t Wp, int64_t off[4],
               int64_t* total) {
  int64_t cap_d = 2 * (int64_t)(Wd - 1), cap_p = 2 * (int64_t)(Wp - 1);
  int64_t sz[4] = {align64(cap_d * Hq * D), align64(cap_d * Hq),
                   align64(cap_p * Hk * kMaxTileRows * D), align64(cap_p * Hk * kMaxTileRows)};
  off[0] = kWsControlInts;
  off[1] = off[0] + sz[0];
  off[2] = off[1] + sz[1];
  off[3] = off[2] + sz[2];
  *total = off[3] + sz[3];
}

}  // namespace

int plan_bounds(int32_t B, int64_t total_qo, int32_t Hq, int32_t Hk, int32_t D, int32_t Wd,
                int32_t Wp, int64_t* plan_ints, int64_t* ws_bytes) {
  if (B < 0 || total_qo < 0 || Hq < 1 || Hk < 1 || Hq % Hk || D < 1 || Wd < 1 || Wp < 1)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan_bounds: bad arguments");
  const int64_t G = Hq / Hk;
  const int64_t rows_d = B;
  const int64_t rows_p = ceil_div(total_qo * G, 16) + B;
  auto stream_ints = [](int64_t rows, int64_t W) {
    int64_t items = rows + W - 1;
    return 4 * rows + (4 + kMetaInts) * items + (W + 1) + (rows + 1) + 5 * rows;
  };
  if (plan_ints) *plan_ints = kHeaderInts + stream_ints(rows_d, Wd) + stream_ints(rows_p, Wp);
  int64_t off[4], total;
  ws_layout(Hq, Hk, D, Wd, Wp, off, &total);
  if (ws_bytes) *ws_bytes = total * 4;
  return FI_OK;
}

int build_plan(const fi_plan_in* inp, int32_t* buf, int64_t capacity, fi_plan_info* info) {
  clear_error();
  if (!inp) return set_error(FI_ERR_INVALID_ARG, "fi_plan: null input");
  const fi_plan_in& in = *inp;
  int rc = validate(in);
  if (rc) return rc;
  const int B = in.batch_size, P = in.page_size;
  const int32_t Hq = in.num_qo_heads, Hk = in.num_kv_heads, D = in.head_dim;
  const int32_t G = Hq / Hk;

  // P2 / P3 / P4
  std::vector<int64_t> np(B), kv(B), qo(B);
  int64_t total_qo = 0, sum_prefill_qo = 0, n_prefill = 0;
  for (int i = 0; i < B; ++i) {
    np[i] = (int64_t)in.kv_indptr[i + 1] - in.kv_indptr[i];
    kv[i] = np[i] == 0 ? 0 : (np[i] - 1) * P + in.kv_last_page_len[i];
    qo[i] = in.qo_indptr ? (int64_t)in.qo_indptr[i + 1] - in.qo_indptr[i] : 1;
    total_qo += qo[i];
    if (qo[i] >= 2) {
      sum_prefill_qo += qo[i];
      n_prefill += 1;
    }
  }
  int32_t BR = 0;
  if (in.br_override) {
    BR = in.br_override;
  } else if (n_prefill) {
    int64_t mean = ceil_div((int64_t)G * sum_prefill_qo, n_prefill);
    BR = std::min<int32_t>(kMaxTileRows, std::max<int32_t>(16, next_pow2(mean)));
  }
  if (total_qo > INT32_MAX) return set_error(FI_ERR_INVALID_ARG, "fi_plan: too many queries");

  // P5
  StreamPlan st[2];
  st[0].W = in.workers_decode;
  st[0].tile = G;
  st[1].W = in.workers_prefill;
  st[1].tile = BR;
  // A row of query tokens [tok_lo, tok_hi] sees keys [first, end): end from
  // the causal bound of tok_hi (or kv_len), first from the window bound of
  // tok_lo (or 0); its pages are first / P .. ceil(end / P).
  const int64_t w = in.window_left;
  auto first_page = [&](int i, int64_t tok_lo) -> int64_t {
    return w < 0 ? 0 : std::max<int64_t>(0, kv[i] - qo[i] + tok_lo - w) / P;
  };
  for (int i = 0; i < B; ++i) {
    if (qo[i] == 1) {
      const int64_t fp = first_page(i, 0);
      st[0].rows.push_back({i, 0, G, (int32_t)std::max<int64_t>(0, np[i] - fp), (int32_t)fp});
    } else if (qo[i] >= 2) {
      const int64_t npk = qo[i] * G;
      for (int64_t rb = 0; rb < npk; rb += BR) {
        int64_t re = std::min<int64_t>(rb + BR, npk);
        int64_t tok_hi = (re - 1) / G;
        int64_t end = in.causal ? kv[i] - qo[i] + tok_hi + 1 : kv[i];
        const int64_t fp = first_page(i, rb / G);
        st[1].rows.push_back({i, (int32_t)rb, (int32_t)re,
                              (int32_t)std::max<int64_t>(0, ceil_div(end, P) - fp), (int32_t)fp});
      }
    }
  }
  // P6 - P8
  rc = partition(st[0], in.min_seg_pages, in.no_split != 0, ceil_div(kDecodeItemCostKeys, P));
  if (rc) return rc;
  rc = partition(st[1], in.min_seg_pages, in.no_split != 0, ceil_div(kTileCostKeys, P));
  if (rc) return rc;

  int64_t off[4], ws_total;
  ws_layout(Hq, Hk, D, in.workers_decode, in.workers_prefill, off, &ws_total);
  if (ws_total > INT32_MAX)
    return set_error(FI_ERR_INVALID_ARG, "fi_plan: float workspace too large for these workers");

  // P9: size, then emit
  int64_t need = kHeaderInts;
  for (auto& s : st)
    need += 4 * (int64_t)s.rows.size() + (4 + kMetaInts) * (int64_t)s.item_row.size() + (s.W + 1) +
            ((int64_t)s.rows.size() + 1) + 5 * (int64_t)s.split.size();
  if (!buf || capacity < need)
    return set_error(FI_ERR_WORKSPACE_TOO_SMALL, "fi_plan: plan buffer holds %lld ints, needs %lld",
                     (long long)capacity, (long long)need);
  if (need > INT32_MAX) return set_error(FI_ERR_INVALID_ARG, "fi_plan: plan too large");
  std::memset(buf, 0, sizeof(int32_t) * kHeaderInts);
  int64_t pos = kHeaderInts;
  for (int k = 0; k < 2; ++k) {
    StreamPlan& s = st[k];
    int32_t* d = buf + (k == 0 ? H_STREAM0 : H_STREAM1);
    const int64_t nr = (int64_t)s.rows.size(), ni = (int64_t)s.item_row.size();
    d[S_W] = s.W;
    d[S_SEG] = s.S;
    d[S_TILE] = s.tile;
    d[S_NROWS] = (int32_t)nr;
    d[S_NITEMS] = (int32_t)ni;
    d[S_NSLOTS] = s.merge.back();
    d[S_NSPLIT] = (int32_t)s.split.size();
    d[S_SLOTCAP] = 2 * (s.W - 1);
    d[S_WS_O] = (int32_t)off[k == 0 ? 0 : 2];
    d[S_WS_LSE] = (int32_t)off[k == 0 ? 1 : 3];
    d[S_KIND] = k;
    d[S_OFF_ROWS] = (int32_t)pos;
    for (const Row& r : s.rows) {
      buf[pos++] = r.req;
      buf[pos++] = r.rb;
      buf[pos++] = r.re;
      buf[pos++] = r.vis;
    }
    d[S_OFF_ITEMS] = (int32_t)pos;
    for (int64_t j = 0; j < ni; ++j) {  // request pages: shifted by the row's first visible page
      const int32_t fp = s.rows[s.item_row[j]].fp;
      buf[pos++] = s.item_row[j];
      buf[pos++] = fp + s.item_pb[j];
      buf[pos++] = fp + s.item_pe[j];
      buf[pos++] = s.item_slot[j];
    }
    d[S_OFF_WIP] = (int32_t)pos;
    for (int32_t v : s.wip) buf[pos++] = v;
    d[S_OFF_MERGE] = (int32_t)pos;
    for (int32_t v : s.merge) buf[pos++] = v;
    d[S_OFF_SPLIT] = (int32_t)pos;
    for (int32_t v : s.split) buf[pos++] = v;
    d[S_OFF_SREC] = (int32_t)pos;
    for (int32_t r : s.split) {
      const Row& row = s.rows[r];
      buf[pos++] = row.rb;
      buf[pos++] = row.re;
      buf[pos++] = in.qo_indptr ? in.qo_indptr[row.req] : row.req;
      buf[pos++] = s.merge[r];
    }
    d[S_OFF_META] = (int32_t)pos;
    for (int64_t j = 0; j < ni; ++j) {
      const Row& r = s.rows[s.item_row[j]];
      buf[pos++] = r.req;
      buf[pos++] = in.kv_indptr[r.req];
      buf[pos++] = (int32_t)kv[r.req];
      buf[pos++] = in.qo_indptr ? in.qo_indptr[r.req] : r.req;
      buf[pos++] = (int32_t)qo[r.req];
      buf[pos++] = r.rb;
      buf[pos++] = r.re;
      buf[pos++] = 0;
    }
  }
  buf[H_MAGIC] = kPlanMagic;
  buf[H_VERSION] = kPlanVersion;
  buf[H_SIZE] = (int32_t)pos;
  buf[H_BATCH] = B;
  buf[H_TOTAL_QO] = (int32_t)total_qo;
  buf[H_HQ] = Hq;
  buf[H_HK] = Hk;
  buf[H_D] = D;
  buf[H_PAGE] = P;
  buf[H_CAUSAL] = in.causal ? 1 : 0;
  buf[H_GROUP] = G;
  buf[H_WS_FLOATS] = (int32_t)ws_total;
  buf[H_WINDOW] = in.window_left;
  int32_t any_pages = 0;
  for (auto& s : st)
    for (const Row& r : s.rows) any_pages |= r.vis > 0;
  buf[H_ANY_PAGES] = any_pages;
  if (info) {
    info->plan_ints = pos;
    info->float_ws_bytes = ws_total * 4;
    info->decode_rows = (int32_t)st[0].rows.size();
    info->decode_items = (int32_t)st[0].item_row.size();
    info->decode_slots = st[0].merge.back();
    info->decode_segment_pages = st[0].S;
    info->prefill_rows = (int32_t)st[1].rows.size();
    info->prefill_items = (int32_t)st[1].item_row.size();
    info->prefill_slots = st[1].merge.back();
    info->prefill_segment_pages = st[1].S;
    info->prefill_tile_rows = BR;
  }
  return FI_OK;
}

}  // namespace fi
