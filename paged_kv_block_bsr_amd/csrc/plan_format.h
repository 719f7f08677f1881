// plan_format.h -- layout of the int32 plan buffer that fi_plan writes and the
// kernels read from device memory.
//
// The buffer starts with a fixed header, then per stream (0 = decode rows,
// 1 = prefill tiles) seven arrays:
//   rows   [n_rows][4]  {request, packed_row_begin, packed_row_end, visible_pages}
//                        (counted from the row's first visible page)
//   items  [n_items][4] {row, page_begin, page_end, slot}  (slot -1: write the
//                        output directly; else the partial-result slot)
//   wip    [W+1]        items of worker w are items[wip[w] .. wip[w+1])
//   merge  [n_rows+1]   slots of row r are merge[r] .. merge[r+1]
//   split  [n_split]    rows with two or more items, in row order
//   srec   [n_split][4] {packed_row_begin, packed_row_end, qo_base,
//                        first slot} of each split row (its slots end where
//                        the next record's begin, the last at n_slots), so
//                        the merge reads one record instead of a chain
//   meta   [n_items][8] {request, kv_indptr[request], kv_len, qo_base, qo_len,
//                        packed_row_begin, packed_row_end, 0} of each item's
//                        request and row (qo_base = qo_indptr[request], or the
//                        request itself for a decode-only batch), so a kernel
//                        reads one record per item instead of a dependent chain
// A row's first visible page is 0, or, with a sliding window of w keys
// (header word H_WINDOW >= 0), the page of key max(0, kv_len - qo_len +
// tok_lo - w), tok_lo being the row's first query token: no query of the row
// sees a key before it.
// A packed row r of a request stands for (token r / G, head-in-group r % G);
// a decode row packs the G query heads of one KV head.  Page indices in
// items are local to the request (the kernel adds kv_indptr[request]); a
// row's items cover its pages [first, first + visible_pages).
//
// The float workspace starts with a control region whose place and size do
// not depend on the plan: word 0 is the status word (bit flags the kernels OR
// in, read and cleared by the host), the rest of its 64 words reserved and
// zero.  After it, per stream, partial outputs [slot_cap][Hk][tile][D]
// and partial lse [slot_cap][Hk][tile] (fp32, natural log) at the float
// offsets recorded in the stream descriptor; tile = G for decode, 128 for
// prefill.
#pragma once
#include <stdint.h>

namespace fi {

constexpr int32_t kPlanMagic = 0x31504946;  // "FIP1"
constexpr int32_t kPlanVersion = 6;
constexpr int kHeaderInts = 64;
constexpr int kMetaInts = 8;  // ints per item_meta record
// item_meta fields
enum : int { M_REQ = 0, M_KVB = 1, M_KVLEN = 2, M_QOBASE = 3, M_QOLEN = 4, M_RB = 5, M_RE = 6 };
constexpr int kMaxTileRows = 128;
// workspace control region (int32 words): the status word, then reserved words
constexpr int64_t kWsControlInts = 64;
// status word bits
constexpr int32_t kStatusBadPage = 1;  // a page id at or past pool_pages was read (and replaced by page 0)
// A request of a windowed plan needs kv_len + qo_len below this, so that the
// kernels' key bounds stay inside int32.
constexpr int64_t kWindowMaxTokens = (int64_t)1 << 30;

// header words
enum : int {
  H_MAGIC = 0,
  H_VERSION = 1,
  H_SIZE = 2,
  H_BATCH = 3,
  H_TOTAL_QO = 4,
  H_HQ = 5,
  H_HK = 6,
  H_D = 7,
  H_PAGE = 8,
  H_CAUSAL = 9,
  H_GROUP = 10,
  H_WS_FLOATS = 11,
  H_STREAM0 = 12,
  H_STREAM1 = 32,
  H_WINDOW = 52,     // sliding window: keys a query sees before its own; -1 = none
  H_ANY_PAGES = 53,  // 1 if some row has visible KV pages (the run calls then read kv_indices and the pool)
};

// stream descriptor words (relative to H_STREAM0 / H_STREAM1)
enum : int {
  S_W = 0,
  S_SEG = 1,
  S_TILE = 2,
  S_NROWS = 3,
  S_NITEMS = 4,
  S_NSLOTS = 5,
  S_NSPLIT = 6,
  S_SLOTCAP = 7,
  S_OFF_ROWS = 8,
  S_OFF_ITEMS = 9,
  S_OFF_WIP = 10,
  S_OFF_MERGE = 11,
  S_OFF_SPLIT = 12,
  S_WS_O = 13,
  S_WS_LSE = 14,
  S_KIND = 15,
  S_OFF_META = 16,
  S_OFF_SREC = 17,
  kStreamDescInts = 20,
};

}  // namespace fi
