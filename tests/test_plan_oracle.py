"""Pins of the plan oracle (oracle/plan_ref.py).

The pages print no plan, so the oracle is pinned by what its rules imply:
- a brute-force partition that hands the pages out one at a time, each
  work item paying the stream's fixed cost, and cuts a row wherever the
  owning worker changes; the segment size is the smallest this walk fits;
- invariants: every row's visible pages are covered exactly once and in order,
  no worker's cost (fixed cost per item plus pages) exceeds S, items <= rows
  + W - 1, slots <= 2 (W - 1), slot numbering, worker item ranges;
- a worked example of the prefill fixed cost;
- the tile-size rule on the worked values (mean query length 960 -> 128,
  256 -> 128, 12 -> 16);
- validation codes.
"""

import numpy as np
import pytest

from oracle import plan_ref as pr


def _random_case(rng, B, max_qo, max_kv, P, causal):
    qo = rng.integers(0, max_qo + 1, size=B)
    kv = np.array([rng.integers(q if (causal and q >= 2) else 0, max(q, max_kv) + 1) for q in qo])
    npg = -(-kv // P)
    last = np.where(npg > 0, kv - (npg - 1) * P, 0).astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    return qo_indptr, kv_indptr, last, qo, kv


def brute_force_items(vis, W, S, h=0):
    """Hand the pages out one at a time: a row starts with the fixed cost h
    on the current worker (the next one if not even one page would fit after
    it), each page goes where the running cost stays within S, and a page
    that does not fit opens a new item, with its own h, on the next worker;
    the last worker takes all that is left.  Returns (w, r, pb, pe) runs and
    the last worker's cost."""
    out = []
    w, used = 0, 0
    for r, v in enumerate(vis):
        if w < W - 1 and used + h >= S:
            w, used = w + 1, 0
        run = [w, r, 0, 0]
        used += h
        for page in range(v):
            if w < W - 1 and used + 1 > S:
                out.append(tuple(run))
                w, used = w + 1, h
                run = [w, r, page, page]
            run[3] += 1
            used += 1
        out.append(tuple(run))
    return sorted(out, key=lambda t: (t[0], t[1])), used


def _check_stream(st, no_split):
    W, S = st["W"], st["S"]
    rows, items, wip = st["rows"], st["items"], st["wip"]
    vis = [r[3] for r in rows]
    assert wip[0] == 0 and wip[-1] == len(items)
    assert all(wip[w] <= wip[w + 1] for w in range(W))
    owner = np.zeros(len(items), int)
    for w in range(W):
        owner[wip[w]:wip[w + 1]] = w
        rs = [items[k][0] for k in range(wip[w], wip[w + 1])]
        assert rs == sorted(rs)
    fps = st["first_page"]
    per_row = {r: [] for r in range(len(rows))}
    for k, (r, pb, pe, slot) in enumerate(items):
        # item pages are request pages; relative to the row's first page here
        per_row[r].append((pb - fps[r], pe - fps[r], slot, owner[k]))
    mi = st["merge_indptr"]
    assert len(mi) == len(rows) + 1 and mi[0] == 0
    for r, lst in per_row.items():
        lst.sort()
        assert len(lst) >= 1
        # coverage: contiguous, exactly once, in order
        pos = 0
        for pb, pe, slot, w in lst:
            assert pb == pos and pe >= pb
            pos = pe
        assert pos == vis[r]
        if len(lst) == 1:
            assert lst[0][2] == -1 and mi[r + 1] == mi[r]
        else:
            assert [x[2] for x in lst] == list(range(mi[r], mi[r] + len(lst)))
            assert mi[r + 1] - mi[r] == len(lst)
    assert st["split_rows"] == [r for r, lst in per_row.items() if len(lst) >= 2]
    if no_split:
        assert len(items) == len(rows) and st["merge_indptr"][-1] == 0
        for k, (r, pb, pe, slot) in enumerate(items):
            assert owner[k] == r % W
    else:
        h = st["tile_cost"]
        load = np.zeros(W, int)  # an item costs h plus its pages
        for k, (r, pb, pe, slot) in enumerate(items):
            load[owner[k]] += h + pe - pb
        assert load.max(initial=0) <= S
        assert len(items) <= len(rows) + W - 1
        assert st["merge_indptr"][-1] <= 2 * (W - 1)
        lo = max(h + st["min_seg"], -(-(sum(vis) + h * len(vis)) // W))
        assert lo <= S <= lo + 2 * h
        # S is the smallest segment at which the walk fits the W workers
        assert S == lo or brute_force_items(vis, W, S - 1, h)[1] > S - 1
        bf, last = brute_force_items(vis, W, S, h)
        assert last <= S
        got = sorted([(owner[k], r, pb - fps[r], pe - fps[r]) for k, (r, pb, pe, slot) in enumerate(items)],
                     key=lambda t: (t[0], t[1]))
        assert got == bf


@pytest.mark.parametrize("seed", range(40))
def test_plan_oracle_invariants_and_brute_force(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.choice([1, 3, 16]))
    causal = bool(rng.integers(0, 2))
    B = int(rng.integers(0, 12))
    qo_indptr, kv_indptr, last, qo, kv = _random_case(rng, B, 40, 300, P, causal)
    Hk = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    Wd, Wp = int(rng.integers(1, 20)), int(rng.integers(1, 20))
    ms = int(rng.integers(1, 9))
    no_split = int(rng.integers(0, 2))
    decode_only = bool(rng.integers(0, 3) == 0)
    code, res = pr.plan(None if decode_only else qo_indptr, kv_indptr, last, page_size=P,
                        num_qo_heads=Hk * G, num_kv_heads=Hk, head_dim=128, causal=causal,
                        workers_decode=Wd, workers_prefill=Wp, min_seg_pages=ms,
                        no_split=no_split)
    assert code == 0, res
    for st, h in ((res["decode"], -(-32 // P)), (res["prefill"], -(-512 // P))):
        st["min_seg"] = ms
        st["tile_cost"] = h
        _check_stream(st, no_split)
    qo_eff = np.ones(B, int) if decode_only else qo
    assert len(res["decode"]["rows"]) == int((qo_eff == 1).sum())
    BR = res["prefill"]["BR"]
    n_tiles = sum(-(-(int(q) * G) // BR) for q in qo_eff if q >= 2)
    assert len(res["prefill"]["rows"]) == n_tiles
    # prefill rows: packed-row ranges tile [0, qo*G); causal visibility
    for (i, rb, re, vp) in res["prefill"]["rows"]:
        assert 0 <= rb < re <= qo_eff[i] * G and re - rb <= BR
        vis = kv[i] - qo_eff[i] + (re - 1) // G + 1 if causal else kv[i]
        assert vp == -(-vis // P)
    for (i, rb, re, vp) in res["decode"]["rows"]:
        assert (rb, re) == (0, G) and vp == kv_indptr[i + 1] - kv_indptr[i]


def test_tile_size_rule_worked_values():
    def br(qo_lens, G=4):
        B = len(qo_lens)
        kv = [max(q, 1) for q in qo_lens]
        qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)])
        kv_indptr = np.arange(B + 1)  # one page each with P = 4096
        code, res = pr.plan(qo_indptr, kv_indptr, kv, page_size=4096, num_qo_heads=8 * G,
                            num_kv_heads=8, head_dim=128, causal=True, workers_decode=4,
                            workers_prefill=4)
        assert code == 0
        return res["prefill"]["BR"]
    assert br([240] * 4) == 128          # mean packed rows 960 -> capped at 128
    assert br([64]) == 128               # 256 -> 128
    assert br([3]) == 16                 # 12 -> 16
    assert br([5, 6]) == 32              # ceil(4 * 11 / 2) = 22 -> 32
    assert br([1, 1]) == 0               # no prefill request


def test_long_request_is_split_into_equal_segments():
    P = 16
    kv = np.array([131072] + [1000] * 31)
    npg = -(-kv // P)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)])
    last = kv - (npg - 1) * P
    code, res = pr.plan(None, kv_indptr, last, page_size=P, num_qo_heads=32, num_kv_heads=8,
                        head_dim=128, causal=True, workers_decode=128, workers_prefill=1)
    st = res["decode"]
    S, h = st["S"], 2  # a decode item's fixed cost: 32 keys = 2 pages
    lo = -(-(int(npg.sum()) + h * len(npg)) // 128)
    assert lo <= S <= lo + 2 * h
    # the long request starts on an empty worker: every piece but the last
    # fills a whole segment with pages after its fixed cost
    long_items = [it for it in st["items"] if it[0] == 0]
    assert len(long_items) == -(-8192 // (S - h))
    assert all(pe - pb == S - h for (_, pb, pe, _) in long_items[:-1])


def test_prefill_tile_fixed_cost_worked_example():
    """Five one-tile prefill requests of 64, 8, 8, 8 and 8 pages (page 16, so
    an item's fixed cost is 512 / 16 = 32) on two workers.  Costs 96, 40, 40,
    40, 40 sum to 256, so S >= 128.  Below S = 136 worker 0 can hold the long
    tile and at most part of the second, whose rest pays 32 again on worker
    1 (33 + 120 > 135); at 136 worker 0 holds tiles 0 and 1 whole (136) and
    worker 1 the other three (120): nothing is cut.  The same requests as
    single queries (decode items, a fixed cost of 2) cut the long row."""
    P = 16
    npg = np.array([64, 8, 8, 8, 8])
    kv_indptr = np.concatenate([[0], np.cumsum(npg)])
    last = np.full(5, P)
    qo_indptr = np.arange(6) * 16
    kw = dict(page_size=P, num_qo_heads=1, num_kv_heads=1, head_dim=64, causal=False,
              workers_decode=1, workers_prefill=2, min_seg_pages=1, br_override=16)
    code, res = pr.plan(qo_indptr, kv_indptr, last, **kw)
    assert code == 0, res
    st = res["prefill"]
    assert st["S"] == 136
    assert st["wip"] == [0, 2, 5]
    assert st["items"] == [(0, 0, 64, -1), (1, 0, 8, -1), (2, 0, 8, -1), (3, 0, 8, -1), (4, 0, 8, -1)]
    assert st["split_rows"] == [] and st["n_slots"] == 0
    # decode items pay 32 / 16 = 2: single-query requests of the same pages
    # cost 66, 10, 10, 10, 10 (sum 106, S >= 53).  At 53 worker 0 takes 51
    # pages of the long row, and worker 1 its other 13 plus 2, then 40: 55.
    # At 54 worker 0 takes 52 and worker 1 2 + 12 + 40 = 54: the long row is
    # cut after page 52.
    code, res = pr.plan(None, kv_indptr, last, **dict(kw, workers_decode=2))
    st = res["decode"]
    assert st["S"] == 54 and st["split_rows"] == [0]
    assert st["items"][:2] == [(0, 0, 52, 0), (0, 52, 64, 1)]


@pytest.mark.parametrize("bad,code", [
    (dict(page_size=0), pr.FI_ERR_INVALID_ARG),
    (dict(num_qo_heads=6, num_kv_heads=4), pr.FI_ERR_INVALID_ARG),
    (dict(head_dim=96), pr.FI_ERR_UNSUPPORTED),
    (dict(num_qo_heads=48, num_kv_heads=3), pr.FI_ERR_UNSUPPORTED),
    (dict(workers_decode=0), pr.FI_ERR_INVALID_ARG),
    (dict(min_seg_pages=0), pr.FI_ERR_INVALID_ARG),
    (dict(br_override=24), pr.FI_ERR_INVALID_ARG),
    (dict(kv_last_page_len=[0, 3]), pr.FI_ERR_INVALID_ARG),
    (dict(kv_last_page_len=[5, 3]), pr.FI_ERR_INVALID_ARG),
    (dict(kv_indptr=[1, 2, 3]), pr.FI_ERR_INVALID_ARG),
    (dict(kv_indptr=[0, 2, 1]), pr.FI_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 9, 10]), pr.FI_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 2, 1]), pr.FI_ERR_INVALID_ARG),
    (dict(window_left=-2), pr.FI_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 2, 3], kv_indptr=[0, 2 ** 28, 2 ** 28 + 1],
          kv_last_page_len=[4, 3], window_left=5), pr.FI_ERR_UNSUPPORTED),
])
def test_plan_oracle_validation(bad, code):
    kw = dict(qo_indptr=[0, 2, 3], kv_indptr=[0, 2, 3], kv_last_page_len=[4, 3], page_size=4,
              num_qo_heads=8, num_kv_heads=2, head_dim=64, causal=True, workers_decode=2,
              workers_prefill=2)
    kw.update(bad)
    got, msg = pr.plan(kw.pop("qo_indptr"), kw.pop("kv_indptr"), kw.pop("kv_last_page_len"), **kw)
    assert got == code, msg


def test_flat_buffer_layout_matches_arrays():
    qo_indptr = [0, 5, 6, 6, 30]
    kv_indptr = [0, 2, 5, 5, 12]
    last = [3, 4, 0, 2]
    code, res = pr.plan(qo_indptr, kv_indptr, last, page_size=4, num_qo_heads=8, num_kv_heads=2,
                        head_dim=64, causal=True, workers_decode=3, workers_prefill=5,
                        min_seg_pages=1)
    assert code == 0
    buf = res["buf"]
    assert buf[0] == pr.MAGIC and buf[2] == len(buf) and buf[4] == 30
    for at, st in ((pr.STREAM0_AT, res["decode"]), (pr.STREAM1_AT, res["prefill"])):
        W, nr, ni = buf[at], buf[at + 3], buf[at + 4]
        assert W == st["W"] and nr == len(st["rows"]) and ni == len(st["items"])
        o = buf[at + 8]
        assert [tuple(buf[o + 4 * k:o + 4 * k + 4]) for k in range(nr)] == [tuple(r) for r in st["rows"]]
        o = buf[at + 9]
        assert [tuple(buf[o + 4 * k:o + 4 * k + 4]) for k in range(ni)] == [tuple(r) for r in st["items"]]
        o = buf[at + 10]
        assert buf[o:o + W + 1] == st["wip"]


@pytest.mark.parametrize("seed", range(12))
def test_item_meta_describes_each_items_request_and_row(seed):
    """item_meta restates, per item, what the row and the inputs say about its
    request; checked here from the raw index arrays, item by item."""
    rng = np.random.default_rng(500 + seed)
    P = int(rng.choice([1, 16]))
    B = int(rng.integers(1, 12))
    qo = rng.integers(0, 40, size=B)
    kv = np.array([rng.integers(max(int(q), 1) if q >= 2 else 0, 300) for q in qo])
    npg = -(-kv // P)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    last = np.where(npg > 0, kv - (npg - 1) * P, 1).astype(np.int32)
    for qo_indptr in (None, np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)):
        code, res = pr.plan(qo_indptr, kv_indptr, last, page_size=P, num_qo_heads=8, num_kv_heads=2,
                            head_dim=64, causal=True, workers_decode=5, workers_prefill=3,
                            min_seg_pages=1)
        assert code == 0, res
        for name in ("decode", "prefill"):
            st = res[name]
            assert len(st["item_meta"]) == len(st["items"])
            for (r, pb, pe, slot), m in zip(st["items"], st["item_meta"]):
                req, rb, re, _ = st["rows"][r]
                n_pages = kv_indptr[req + 1] - kv_indptr[req]
                want_kv = 0 if n_pages == 0 else (n_pages - 1) * P + last[req]
                want_qb = req if qo_indptr is None else qo_indptr[req]
                want_ql = 1 if qo_indptr is None else qo_indptr[req + 1] - qo_indptr[req]
                assert m == (req, kv_indptr[req], want_kv, want_qb, want_ql, rb, re, 0)
            off = st["off_item_meta"]
            assert res["buf"][off:off + 8 * len(st["item_meta"])] == [x for m in st["item_meta"] for x in m]


@pytest.mark.parametrize("seed", range(12))
def test_split_records_describe_each_split_row(seed):
    """Record k restates the k-th split row for the merge: its packed rows,
    its query base (from the raw qo_indptr) and its first slot; its slots end
    where the next record's begin, the last at the stream's slot count."""
    rng = np.random.default_rng(700 + seed)
    P = int(rng.choice([1, 3, 16]))
    B = int(rng.integers(1, 12))
    qo_indptr, kv_indptr, last, qo, kv = _random_case(rng, B, 40, 400, P, True)
    Wd, Wp = int(rng.integers(1, 24)), int(rng.integers(1, 24))
    for qi in (None, qo_indptr):
        code, res = pr.plan(qi, kv_indptr, last, page_size=P, num_qo_heads=8, num_kv_heads=2,
                            head_dim=64, causal=True, workers_decode=Wd, workers_prefill=Wp,
                            min_seg_pages=1)
        assert code == 0, res
        buf = res["buf"]
        for at, st in ((pr.STREAM0_AT, res["decode"]), (pr.STREAM1_AT, res["prefill"])):
            off, n = buf[at + 17], len(st["split_rows"])
            recs = [tuple(buf[off + 4 * k:off + 4 * k + 4]) for k in range(n)]
            mi = st["merge_indptr"]
            ends = [rec[3] for rec in recs[1:]] + [st["n_slots"]]
            for k, r in enumerate(st["split_rows"]):
                req, rb, re, _ = st["rows"][r]
                qb = req if qi is None else int(qi[req])
                assert recs[k] == (rb, re, qb, mi[r])
                assert ends[k] == mi[r + 1] and mi[r + 1] - mi[r] >= 2


def _visible_pages(kv, qo, toks, P, causal, window):
    """Pages holding a key that some query token of ``toks`` sees, straight
    from the definition: token t (position p = kv - qo + t) sees key j iff
    j < kv, j <= p when causal, and j >= p - window when window >= 0."""
    pages = set()
    for t in toks:
        p = kv - qo + t
        for j in range(kv):
            if causal and j > p:
                continue
            if window >= 0 and j < p - window:
                continue
            pages.add(j // P)
    return pages


@pytest.mark.parametrize("seed", range(24))
def test_window_rows_cover_exactly_the_pages_their_queries_see(seed):
    """With a sliding window every row's items cover exactly the pages that
    hold a key one of its queries sees (a brute-force visibility map), and
    the partition invariants still hold."""
    rng = np.random.default_rng(3000 + seed)
    P = int(rng.choice([1, 3, 16]))
    causal = bool(rng.integers(0, 2))
    B = int(rng.integers(1, 8))
    qo_indptr, kv_indptr, last, qo, kv = _random_case(rng, B, 24, 160, P, causal)
    window = int(rng.choice([0, 1, 5, 17, 40, 100, 1000]))
    G = int(rng.choice([1, 2, 4]))
    ms = int(rng.integers(1, 4))
    no_split = int(rng.integers(0, 2))
    code, res = pr.plan(qo_indptr, kv_indptr, last, page_size=P, num_qo_heads=2 * G,
                        num_kv_heads=2, head_dim=64, causal=causal, workers_decode=int(rng.integers(1, 9)),
                        workers_prefill=int(rng.integers(1, 9)), min_seg_pages=ms,
                        no_split=no_split, window_left=window)
    assert code == 0, res
    assert res["buf"][pr.WINDOW_AT] == window
    for st, h in ((res["decode"], -(-32 // P)), (res["prefill"], -(-512 // P))):
        st["min_seg"] = ms
        st["tile_cost"] = h
        _check_stream(st, no_split)
        covered = {r: set() for r in range(len(st["rows"]))}
        for (r, pb, pe, slot) in st["items"]:
            covered[r] |= set(range(pb, pe))
        for r, (i, rb, re, vp) in enumerate(st["rows"]):
            toks = range(rb // G, (re - 1) // G + 1)
            want = _visible_pages(int(kv[i]), int(qo[i]), toks, P, causal, window)
            assert covered[r] == want, (r, i, rb, re)
            assert vp == len(want)


def test_window_as_long_as_every_request_changes_no_array():
    rng = np.random.default_rng(3100)
    qo_indptr, kv_indptr, last, qo, kv = _random_case(rng, 10, 30, 300, 16, True)
    kw = dict(page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128, causal=True,
              workers_decode=7, workers_prefill=5, min_seg_pages=2)
    _, none = pr.plan(qo_indptr, kv_indptr, last, **kw)
    _, wide = pr.plan(qo_indptr, kv_indptr, last, window_left=int(kv.max()), **kw)
    assert none["buf"][pr.WINDOW_AT] == -1 and wide["buf"][pr.WINDOW_AT] == int(kv.max())
    a, b = list(none["buf"]), list(wide["buf"])
    a[pr.WINDOW_AT] = b[pr.WINDOW_AT] = 0
    assert a == b


def test_window_zero_decode_rows_keep_only_the_last_page():
    # a window of 0 keys: a decode query sees its own key alone, the last one
    kv = np.array([1, 16, 17, 100, 0])
    npg = -(-kv // 16)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)])
    last = np.where(npg > 0, kv - (npg - 1) * 16, 0)
    code, res = pr.plan(None, kv_indptr, last, page_size=16, num_qo_heads=4, num_kv_heads=1,
                        head_dim=64, causal=True, workers_decode=3, workers_prefill=1,
                        window_left=0)
    assert code == 0
    st = res["decode"]
    assert [r[3] for r in st["rows"]] == [1, 1, 1, 1, 0]
    for (r, pb, pe, slot) in st["items"]:
        n = int(npg[r])
        assert (pb, pe) == ((n - 1, n) if n else (0, 0))


@pytest.mark.parametrize("seed", range(20))
def test_any_pages_word_marks_plans_whose_rows_see_pages(seed):
    """Header word 53 is 1 exactly when some request with queries has KV
    tokens: such a row sees at least one page (a causal prefill row has
    qo_len <= kv_len, so it sees its own key)."""
    rng = np.random.default_rng(4400 + seed)
    B = int(rng.integers(0, 6))
    qo = rng.integers(0, 4, B) * rng.integers(0, 2, B)
    kv = np.where((rng.random(B) < 0.5) & (qo < 2), 0, qo + rng.integers(0, 40, B))
    npg = -(-kv // 16)
    last = np.where(npg > 0, kv - (npg - 1) * 16, 0)
    code, res = pr.plan(np.concatenate([[0], np.cumsum(qo)]), np.concatenate([[0], np.cumsum(npg)]), last,
                        page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=64, causal=True,
                        workers_decode=3, workers_prefill=2, window_left=int(rng.integers(-1, 20)))
    assert code == pr.FI_OK
    assert res["buf"][pr.ANY_PAGES_AT] == int(bool(np.any((qo >= 1) & (kv > 0))))
