"""Plan oracle: the CPU-side work partition, written step by step in pure Python.

TEST INFRASTRUCTURE ONLY.

The pages describe the plan only in words: each generation step, a CPU-side
plan splits long KV sequences into equal chunks across the GPU's processors and
records where partial results go; persistent kernels with fixed grids then run
it and merge the partials by log-sum-exp composition (FlashInfer paper page,
"Load balancing that survives CUDA graphs"); the scheduler inspects the lengths
ahead of time and balances deterministically with a cost model (talk page,
"Runtime Scheduler for Dynamic Problem Shapes"); the query tile size is picked
from the batch's average query length (paper page, JIT paragraph).  Where they
stop, this module takes the plainest reading (cost = KV pages plus a fixed
charge per work item; workers filled in row order up to one segment size
each) and spells out every step:

P1 validate; P2 per-request pages, kv_len, qo_len; P3 classify requests
(qo_len 0: nothing, 1: a decode row, >= 2: prefill tiles); P4 prefill tile
size BR; P5 rows in request order, each with its first visible page fp
(0, or with a sliding window of w keys the page of the first key the row's
earliest query sees, max(0, kv_len - qo_len + tok_lo - w)) and its visible
pages counted from fp; P6 per stream, an item (a row's pages on one worker)
costs h plus its pages, with h = ceil(32 / P) for a decode row and
h = ceil(512 / P) for a prefill tile (a fixed charge for the work an item does
whatever its length: loading its queries, writing its output rows or partial
state, starting the item); C = the sum
over rows of h + vis_r; P7 fill workers in row order: a worker that has
already used S - h or more of its segment S takes nothing more, a row that
does not fit is cut where the worker is full and its rest starts a new item
on the next worker, the last worker takes what is left, and a row without
visible pages is one empty item on the current worker; S is the smallest
value >= max(h + min_seg_pages, ceil(C / W)) at which the last worker's cost
stays within S; item pages are shifted by fp (pages of its request); P8 rows
with k >= 2 items get k consecutive partial slots; P9 emit int32 arrays.

Parity against the pages: unpinned (they print no plan); the tests pin this
module by invariants and by an independent brute-force partition.
"""
from __future__ import annotations

FI_OK = 0
FI_ERR_INVALID_ARG = -1
FI_ERR_UNSUPPORTED = -2

MAGIC = 0x31504946
VERSION = 6
HEADER_INTS = 64
STREAM_DESC_INTS = 20
STREAM0_AT = 12
STREAM1_AT = 32
WINDOW_AT = 52
ANY_PAGES_AT = 53  # 1 if some row has visible pages
MAX_TILE_ROWS = 128
# workspace control region (ints): the status word, then reserved words; its
# place and size do not depend on the plan
WS_CONTROL_INTS = 64
INT32_MAX = 2 ** 31 - 1
WINDOW_MAX_TOKENS = 2 ** 30  # a windowed request needs kv_len + qo_len below this
TILE_COST_KEYS = 512  # fixed cost of a prefill work item, in keys (rounded up to pages)
DECODE_ITEM_COST_KEYS = 32  # fixed cost of a decode work item, in keys (rounded up to pages)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _next_pow2(x: int) -> int:
    p = 1
    while p < x:
        p *= 2
    return p


def _align64(n: int) -> int:
    """Round a float count up to a multiple of 64 floats (256 bytes)."""
    return _ceil_div(n, 64) * 64


def validate(B, qo_indptr, kv_indptr, kv_last_page_len, P, Hq, Hk, D, causal, W_d, W_p,
             min_seg_pages, br_override, no_split, window_left=-1):
    """P1.  Returns (code, message)."""
    if B < 0:
        return FI_ERR_INVALID_ARG, "negative batch size"
    if P < 1:
        return FI_ERR_INVALID_ARG, "page_size < 1"
    if Hq < 1 or Hk < 1 or Hq % Hk != 0:
        return FI_ERR_INVALID_ARG, "head counts"
    if D not in (64, 128):
        return FI_ERR_UNSUPPORTED, "head_dim"
    if Hq // Hk not in (1, 2, 4, 8):
        return FI_ERR_UNSUPPORTED, "group size"
    if W_d < 1 or W_p < 1:
        return FI_ERR_INVALID_ARG, "workers < 1"
    if min_seg_pages < 1:
        return FI_ERR_INVALID_ARG, "min_seg_pages < 1"
    if br_override not in (0, 16, 32, 64, 128):
        return FI_ERR_INVALID_ARG, "br_override"
    if no_split not in (0, 1):
        return FI_ERR_INVALID_ARG, "no_split"
    if not -1 <= window_left <= INT32_MAX:
        return FI_ERR_INVALID_ARG, "window_left"
    if len(kv_indptr) != B + 1 or len(kv_last_page_len) < B:
        return FI_ERR_INVALID_ARG, "array lengths"
    if qo_indptr is not None and len(qo_indptr) != B + 1:
        return FI_ERR_INVALID_ARG, "array lengths"
    if kv_indptr[0] != 0:
        return FI_ERR_INVALID_ARG, "kv_indptr[0]"
    if qo_indptr is not None and qo_indptr[0] != 0:
        return FI_ERR_INVALID_ARG, "qo_indptr[0]"
    for i in range(B):
        npg = int(kv_indptr[i + 1]) - int(kv_indptr[i])
        if npg < 0:
            return FI_ERR_INVALID_ARG, "kv_indptr decreases"
        qo = 1 if qo_indptr is None else int(qo_indptr[i + 1]) - int(qo_indptr[i])
        if qo < 0:
            return FI_ERR_INVALID_ARG, "qo_indptr decreases"
        if npg > 0 and not (1 <= int(kv_last_page_len[i]) <= P):
            return FI_ERR_INVALID_ARG, "last_page_len"
        kv = 0 if npg == 0 else (npg - 1) * P + int(kv_last_page_len[i])
        if kv > INT32_MAX:
            return FI_ERR_INVALID_ARG, "kv_len too large"
        if causal and qo >= 2 and qo > kv:
            return FI_ERR_INVALID_ARG, "causal with qo_len > kv_len"
        if window_left >= 0 and kv + qo >= WINDOW_MAX_TOKENS:
            return FI_ERR_UNSUPPORTED, "window with kv_len + qo_len >= 2^30"
    return FI_OK, ""


def _fill(rows_vis, W, S, h):
    """P7 for one segment size S: returns (items as (w, r, page_begin,
    page_end), the last worker's cost)."""
    items = []
    w, used = 0, 0
    for r, vis in enumerate(rows_vis):
        if w < W - 1 and S - used <= h:
            w, used = w + 1, 0
        if vis == 0:
            items.append((w, r, 0, 0))
            used += h
            continue
        done = 0
        while done < vis:
            room = vis - done if w == W - 1 else S - used - h
            n = min(vis - done, room)
            items.append((w, r, done, done + n))
            used += h + n
            done += n
            if done < vis:
                w, used = w + 1, 0
    return items, used


def _partition(rows_vis, W, min_seg_pages, no_split, h=0):
    """P6-P8 for one stream.  rows_vis[r] = visible pages of row r, h = the
    fixed cost of an item.  Returns (S, items sorted by (worker, row), wip,
    merge_indptr, split_rows)."""
    C = sum(h + v for v in rows_vis)
    S = max(h + min_seg_pages, _ceil_div(C, W))
    if no_split:
        items = [(r % W, r, 0, vis) for r, vis in enumerate(rows_vis)]
    else:
        while True:  # smallest S that fits: try S, S + 1, ...
            items, last = _fill(rows_vis, W, S, h)
            if last <= S:
                break
            S += 1
    items.sort(key=lambda it: (it[0], it[1]))
    # P8: rows split over k >= 2 items get k consecutive slots (row order,
    # then page_begin order inside the row).
    per_row = [[] for _ in rows_vis]
    for idx, (w, r, pb, pe) in enumerate(items):
        per_row[r].append((pb, idx))
    slot_of_item = [-1] * len(items)
    merge_indptr = [0]
    split_rows = []
    for r, lst in enumerate(per_row):
        k = len(lst)
        base = merge_indptr[-1]
        if k >= 2:
            split_rows.append(r)
            for j, (pb, idx) in enumerate(sorted(lst)):
                slot_of_item[idx] = base + j
            merge_indptr.append(base + k)
        else:
            merge_indptr.append(base)
    wip = [0] * (W + 1)
    for (w, r, pb, pe) in items:
        wip[w + 1] += 1
    for w in range(W):
        wip[w + 1] += wip[w]
    out_items = [(r, pb, pe, slot_of_item[idx]) for idx, (w, r, pb, pe) in enumerate(items)]
    return S, out_items, wip, merge_indptr, split_rows


def plan(qo_indptr, kv_indptr, kv_last_page_len, *, page_size, num_qo_heads, num_kv_heads,
         head_dim, causal, workers_decode, workers_prefill, min_seg_pages=8, br_override=0,
         no_split=0, window_left=-1):
    """Build the plan.  Returns (code, result) where result is a dict with the
    header scalars, each stream's arrays and the flat int32 buffer."""
    B = len(kv_indptr) - 1
    P, Hq, Hk, D = page_size, num_qo_heads, num_kv_heads, head_dim
    qo_indptr = None if qo_indptr is None else [int(x) for x in qo_indptr]
    kv_indptr = [int(x) for x in kv_indptr]
    last = [int(x) for x in kv_last_page_len]
    code, msg = validate(B, qo_indptr, kv_indptr, last, P, Hq, Hk, D, int(bool(causal)),
                         workers_decode, workers_prefill, min_seg_pages, br_override, no_split,
                         window_left)
    if code != FI_OK:
        return code, msg
    G = Hq // Hk
    # P2
    npages = [kv_indptr[i + 1] - kv_indptr[i] for i in range(B)]
    kv_len = [0 if npages[i] == 0 else (npages[i] - 1) * P + last[i] for i in range(B)]
    qo_len = [1] * B if qo_indptr is None else [qo_indptr[i + 1] - qo_indptr[i] for i in range(B)]
    # P3
    decode_reqs = [i for i in range(B) if qo_len[i] == 1]
    prefill_reqs = [i for i in range(B) if qo_len[i] >= 2]
    # P4
    if br_override:
        BR = br_override
    elif prefill_reqs:
        mean = _ceil_div(G * sum(qo_len[i] for i in prefill_reqs), len(prefill_reqs))
        BR = min(MAX_TILE_ROWS, max(16, _next_pow2(mean)))
    else:
        BR = 0
    # P5.  A row of query tokens [tok_lo, tok_hi] sees keys [first, end):
    # end from the causal bound of tok_hi (or kv_len), first from the window
    # bound of tok_lo (or 0).  Its pages are fp = first // P .. ceil(end / P).
    def first_page(i, tok_lo):
        if window_left < 0:
            return 0
        return max(0, kv_len[i] - qo_len[i] + tok_lo - window_left) // P

    rows_d, fp_d = [], []
    for i in decode_reqs:
        fp = first_page(i, 0)
        rows_d.append((i, 0, G, max(0, npages[i] - fp)))
        fp_d.append(fp)
    rows_p, fp_p = [], []
    for i in prefill_reqs:
        n_packed = qo_len[i] * G
        for k in range(_ceil_div(n_packed, BR)):
            rb, re = k * BR, min((k + 1) * BR, n_packed)
            tok_lo, tok_hi = rb // G, (re - 1) // G
            end = kv_len[i] - qo_len[i] + tok_hi + 1 if causal else kv_len[i]
            fp = first_page(i, tok_lo)
            rows_p.append((i, rb, re, max(0, _ceil_div(end, P) - fp)))
            fp_p.append(fp)
    # float workspace regions (float units, each a multiple of 64 floats)
    cap_d = 2 * (workers_decode - 1)
    cap_p = 2 * (workers_prefill - 1)
    sizes = [_align64(cap_d * Hq * D), _align64(cap_d * Hq),
             _align64(cap_p * Hk * MAX_TILE_ROWS * D), _align64(cap_p * Hk * MAX_TILE_ROWS)]
    ws_off = [WS_CONTROL_INTS + sum(sizes[:k]) for k in range(4)]
    ws_total = WS_CONTROL_INTS + sum(sizes)
    if ws_total > INT32_MAX:
        return FI_ERR_INVALID_ARG, "workspace too large for the workers given"

    streams = []
    for kind, rows, fps, W, tile in ((0, rows_d, fp_d, workers_decode, G),
                                     (1, rows_p, fp_p, workers_prefill, BR)):
        vis = [r[3] for r in rows]
        h = _ceil_div(DECODE_ITEM_COST_KEYS if kind == 0 else TILE_COST_KEYS, P)
        S, items, wip, merge_indptr, split_rows = _partition(vis, W, min_seg_pages, no_split, h)
        if S > INT32_MAX:
            return FI_ERR_INVALID_ARG, "segment too large"
        # item pages are request pages: shift by the row's first visible page
        items = [(r, fps[r] + pb, fps[r] + pe, slot) for (r, pb, pe, slot) in items]
        streams.append(dict(kind=kind, W=W, S=S, h=h, BR=tile, rows=rows, first_page=fps, items=items, wip=wip,
                            merge_indptr=merge_indptr, split_rows=split_rows,
                            n_slots=merge_indptr[-1],
                            slot_cap=cap_d if kind == 0 else cap_p,
                            ws_off_o=ws_off[0] if kind == 0 else ws_off[2],
                            ws_off_lse=ws_off[1] if kind == 0 else ws_off[3]))
    # P9: flat buffer
    buf = [0] * HEADER_INTS
    for st in streams:
        st["off_rows"] = len(buf)
        for r in st["rows"]:
            buf.extend(r)
        st["off_items"] = len(buf)
        for it in st["items"]:
            buf.extend(it)
        st["off_wip"] = len(buf)
        buf.extend(st["wip"])
        st["off_merge_indptr"] = len(buf)
        buf.extend(st["merge_indptr"])
        st["off_split"] = len(buf)
        buf.extend(st["split_rows"])
        # per split row: its packed rows, query base and first slot
        st["off_split_rec"] = len(buf)
        for r in st["split_rows"]:
            req, rb, re, _ = st["rows"][r]
            buf.extend([rb, re, req if qo_indptr is None else qo_indptr[req], st["merge_indptr"][r]])
        # per-item copy of what a kernel needs about the item's request and
        # row, so that one load per item replaces a chain of dependent ones
        st["item_meta"] = []
        for (r, pb, pe, slot) in st["items"]:
            req, rb, re, _ = st["rows"][r]
            qb = req if qo_indptr is None else qo_indptr[req]
            st["item_meta"].append((req, kv_indptr[req], kv_len[req], qb, qo_len[req], rb, re, 0))
        st["off_item_meta"] = len(buf)
        for m in st["item_meta"]:
            buf.extend(m)
    head = [MAGIC, VERSION, len(buf), B, sum(qo_len), Hq, Hk, D, P, int(bool(causal)), G,
            ws_total]
    buf[:len(head)] = head
    buf[WINDOW_AT] = window_left
    buf[ANY_PAGES_AT] = int(any(r[3] > 0 for st in streams for r in st["rows"]))
    for at, st in ((STREAM0_AT, streams[0]), (STREAM1_AT, streams[1])):
        desc = [st["W"], st["S"], st["BR"], len(st["rows"]), len(st["items"]), st["n_slots"],
                len(st["split_rows"]), st["slot_cap"], st["off_rows"], st["off_items"],
                st["off_wip"], st["off_merge_indptr"], st["off_split"], st["ws_off_o"],
                st["ws_off_lse"], st["kind"], st["off_item_meta"], st["off_split_rec"], 0, 0]
        buf[at:at + STREAM_DESC_INTS] = desc
    result = dict(B=B, total_qo=sum(qo_len), G=G, ws_floats=ws_total, window_left=window_left,
                  decode=streams[0],
                  prefill=streams[1], buf=buf, kv_len=kv_len, qo_len=qo_len)
    return FI_OK, result
