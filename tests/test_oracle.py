"""Pins of the fp64 oracle against things other than itself.

- the pages' own worked page-table example (tests/golden/page_table_example.json);
- dense brute force from contiguous per-request tensors (numpy + scipy's
  logsumexp / softmax, np.repeat for the head groups, np.tril for the causal
  mask) on tiny problems whose pool is filled page-block by page-block;
- torch's scaled_dot_product_attention in fp64 on the CPU (library routine),
  including the textbook causal case qo_len == kv_len;
- closed forms (single key, identical keys, q = 0, constant V, two keys under
  the soft-cap, the log-sum-exp bounds);
- invariants: physical page permutation, split + merge == unsplit,
  cascade == flat, request order, NaN in slots that must not be read.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attn as ref

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- helpers

def _pages(L, P):
    return -(-L // P)


def dense_problem(seed, qo_lens, kv_lens, P, Hq, Hk, D, extra_pages=3, scale_q=1.0):
    """Contiguous per-request Q/K/V, then a NaN-filled pool written page block
    by page block through a random page assignment."""
    rng = np.random.default_rng(seed)
    Qs = [rng.standard_normal((qo, Hq, D)) * scale_q for qo in qo_lens]
    Ks = [rng.standard_normal((L, Hk, D)) for L in kv_lens]
    Vs = [rng.standard_normal((L, Hk, D)) for L in kv_lens]
    npg = [_pages(L, P) for L in kv_lens]
    pool_pages = sum(npg) + extra_pages
    perm = rng.permutation(pool_pages)
    pool = np.full((pool_pages, 2, P, Hk, D), np.nan)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    kv_indices = perm[:sum(npg)].astype(np.int32)
    last = np.zeros(len(kv_lens), np.int32)
    for i, L in enumerate(kv_lens):
        ids = kv_indices[kv_indptr[i]:kv_indptr[i + 1]]
        for p, page in enumerate(ids):
            blk = slice(p * P, min((p + 1) * P, L))
            n = blk.stop - blk.start
            pool[page, 0, :n] = Ks[i][blk]
            pool[page, 1, :n] = Vs[i][blk]
        last[i] = L - (len(ids) - 1) * P if len(ids) else 0
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    q = np.concatenate(Qs) if sum(qo_lens) else np.zeros((0, Hq, D))
    return dict(Qs=Qs, Ks=Ks, Vs=Vs, q=q, pool=pool, qo_indptr=qo_indptr,
                kv_indptr=kv_indptr, kv_indices=kv_indices, last=last)


def dense_ref(Q, K, V, scale, cap, causal):
    """Brute-force attention of one request on contiguous tensors."""
    qo, Hq, D = Q.shape
    kv, Hk, _ = K.shape
    G = Hq // Hk
    Kr = np.repeat(K, G, axis=1)
    Vr = np.repeat(V, G, axis=1)
    s = np.einsum("thd,jhd->htj", Q, Kr) * scale
    if cap > 0:
        s = cap * np.tanh(s / cap)
    mask = np.ones((qo, kv), bool)
    if causal:
        mask = np.tril(mask, k=kv - qo)
    s = np.where(mask[None], s, -np.inf)
    o = np.zeros((qo, Hq, D))
    lse = np.full((qo, Hq), -np.inf)
    live = mask.any(axis=1)
    if kv and live.any():
        sl = s[:, live, :]
        lse[live] = scipy.special.logsumexp(sl, axis=-1).T
        p = scipy.special.softmax(sl, axis=-1)
        o[live] = np.einsum("htj,jhd->thd", p, Vr)
    return o, lse


def run_oracle(pb, P, Hq, Hk, D, causal, scale, cap):
    return ref.attention(pb["q"], pb["pool"], pb["qo_indptr"], pb["kv_indptr"], pb["kv_indices"],
                         pb["last"], page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=D,
                         causal=causal, sm_scale=scale, soft_cap=cap)


# ---------------------------------------------------------------- the pages' example

def test_page_table_example_from_the_pages():
    g = json.load(open(os.path.join(HERE, "golden", "page_table_example.json")))
    P = g["page_size"]
    tables = [r["page_table"] for r in g["requests"]]
    kv_indptr = np.concatenate([[0], np.cumsum([len(t) for t in tables])]).astype(np.int32)
    kv_indices = np.concatenate(tables).astype(np.int32)
    last = np.array(g["expected_last_page_len"], np.int32)
    for i, r in enumerate(g["requests"]):
        for lo, hi, page in r["ranges"]:
            for tok in range(lo, hi + 1):
                pg, slot = ref.token_location(kv_indptr, kv_indices, P, i, tok)
                assert pg == page, (i, tok)
                assert slot == tok - lo, (i, tok)
    # kv_len read back through attention: with K = 0 every visible key has the
    # same weight, so o = mean of the V rows = mean of the logical positions.
    Hq = Hk = 1
    D = 2
    pool = np.full((16, 2, P, Hk, D), np.nan)
    for i, r in enumerate(g["requests"]):
        for lo, hi, page in r["ranges"]:
            pool[page, 0, : hi - lo + 1] = 0.0
            pool[page, 1, : hi - lo + 1, 0, :] = np.arange(lo, hi + 1, dtype=np.float64)[:, None]
    q = np.ones((2, Hq, D))
    o, lse = ref.attention(q, pool, None, kv_indptr, kv_indices, last, page_size=P,
                           num_qo_heads=Hq, num_kv_heads=Hk, head_dim=D, causal=True,
                           sm_scale=1.0)
    for i, n in enumerate(g["expected_kv_len"]):
        assert o[i, 0, 0] == pytest.approx((n - 1) / 2.0, abs=1e-12)
        assert lse[i, 0] == pytest.approx(math.log(n), abs=1e-12)


# ---------------------------------------------------------------- brute force

CASES = [
    # (seed, qo_lens, kv_lens, P, Hq, Hk, D, causal, cap)
    (1, [1, 1, 1], [1, 17, 40], 16, 4, 1, 16, True, 0.0),
    (2, [1, 1, 1, 1], [0, 3, 5, 33], 3, 8, 2, 16, True, 0.0),
    (3, [2, 5, 1], [2, 9, 20], 1, 4, 4, 16, True, 0.0),
    (4, [3, 7, 4], [10, 7, 4], 4, 8, 1, 32, True, 30.0),
    (5, [3, 0, 6], [5, 4, 6], 2, 2, 2, 16, False, 0.0),
    (6, [4, 4], [0, 6], 5, 8, 8, 16, False, 5.0),
    (7, [17, 1], [40, 40], 16, 8, 2, 64, True, 0.0),
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_dense_brute_force(case):
    seed, qo, kv, P, Hq, Hk, D, causal, cap = case
    pb = dense_problem(seed, qo, kv, P, Hq, Hk, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_oracle(pb, P, Hq, Hk, D, causal, scale, cap)
    for i in range(len(qo)):
        a, b = pb["qo_indptr"][i], pb["qo_indptr"][i + 1]
        od, ld = dense_ref(pb["Qs"][i], pb["Ks"][i], pb["Vs"][i], scale, cap, causal)
        np.testing.assert_allclose(o[a:b], od, rtol=0, atol=1e-12)
        fin = np.isfinite(ld)
        assert np.array_equal(np.isfinite(lse[a:b]), fin)
        np.testing.assert_allclose(lse[a:b][fin], ld[fin], rtol=0, atol=1e-12)
        assert np.all(o[a:b][~fin] == 0.0)


@pytest.mark.parametrize("qo,kv,causal,Hq,Hk", [
    (5, 5, True, 4, 2), (1, 9, False, 4, 4), (6, 6, False, 8, 2), (3, 11, True, 2, 1),
])
def test_oracle_matches_torch_sdpa_fp64(qo, kv, causal, Hq, Hk):
    D, P = 16, 4
    pb = dense_problem(11 + qo + kv, [qo], [kv], P, Hq, Hk, D)
    scale = 0.3
    o, lse = run_oracle(pb, P, Hq, Hk, D, causal, scale, 0.0)
    Q = torch.from_numpy(pb["Qs"][0]).permute(1, 0, 2)[None]          # [1,Hq,qo,D]
    K = torch.from_numpy(pb["Ks"][0]).permute(1, 0, 2)[None]
    V = torch.from_numpy(pb["Vs"][0]).permute(1, 0, 2)[None]
    K = K.repeat_interleave(Hq // Hk, dim=1)
    V = V.repeat_interleave(Hq // Hk, dim=1)
    F = torch.nn.functional
    if causal and qo == kv:
        out = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    elif causal:
        m = torch.ones(qo, kv, dtype=torch.bool).tril(diagonal=kv - qo)
        out = F.scaled_dot_product_attention(Q, K, V, attn_mask=m, scale=scale)
    else:
        out = F.scaled_dot_product_attention(Q, K, V, scale=scale)
    np.testing.assert_allclose(o, out[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    s = torch.einsum("bhtd,bhjd->bhtj", Q, K) * scale
    if causal:
        s = s.masked_fill(~torch.ones(qo, kv, dtype=torch.bool).tril(diagonal=kv - qo), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1)[0].T.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def _single(q, K, V, P=4, cap=0.0, scale=1.0):
    """Run one request (one query token, one head) through the oracle."""
    L, D = K.shape
    pb = dense_problem(0, [1], [L], P, 1, 1, D)
    pb["Qs"] = [q[None, None]]
    pb["q"] = q[None, None].copy()
    for p, page in enumerate(pb["kv_indices"]):
        n = min(P, L - p * P)
        pb["pool"][page, 0, :n, 0] = K[p * P:p * P + n]
        pb["pool"][page, 1, :n, 0] = V[p * P:p * P + n]
    o, lse = run_oracle(pb, P, 1, 1, D, True, scale, cap)
    return o[0, 0], lse[0, 0]


def test_closed_form_single_key():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    o, lse = _single(q, k, v, scale=0.7)
    np.testing.assert_allclose(o, v[0], atol=1e-15)
    assert lse == pytest.approx(0.7 * float(q @ k[0]), abs=1e-13)


def test_closed_form_identical_keys_and_zero_query():
    rng = np.random.default_rng(4)
    n = 23
    k = np.tile(rng.standard_normal(8), (n, 1))
    V = rng.standard_normal((n, 8))
    q = rng.standard_normal(8)
    o, lse = _single(q, k, V, P=5, scale=0.5)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-13)
    assert lse == pytest.approx(0.5 * float(q @ k[0]) + math.log(n), abs=1e-12)
    o, lse = _single(np.zeros(8), rng.standard_normal((n, 8)), V, P=5, cap=30.0)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-13)
    assert lse == pytest.approx(math.log(n), abs=1e-13)


def test_closed_form_constant_values_and_bounds():
    rng = np.random.default_rng(5)
    n = 37
    K = rng.standard_normal((n, 8))
    q = rng.standard_normal(8)
    V = np.tile(rng.standard_normal(8), (n, 1))
    o, lse = _single(q, K, V, P=3, scale=0.9)
    np.testing.assert_allclose(o, V[0], atol=1e-13)
    s = 0.9 * (K @ q)
    assert s.max() - 1e-12 <= lse <= s.max() + math.log(n) + 1e-12


def test_closed_form_two_keys_soft_cap():
    """With two keys the softmax is the logistic function of the capped
    logit difference: o = expit(a - b) v0 + expit(b - a) v1."""
    rng = np.random.default_rng(6)
    cap = 2.0
    q = rng.standard_normal(16) * 3
    K = rng.standard_normal((2, 16))
    V = rng.standard_normal((2, 16))
    o, lse = _single(q, K, V, P=1, cap=cap, scale=0.25)
    a, b = (cap * np.tanh(0.25 * (K @ q) / cap))
    np.testing.assert_allclose(o, scipy.special.expit(a - b) * V[0] + scipy.special.expit(b - a) * V[1],
                               atol=1e-13)
    assert lse == pytest.approx(np.logaddexp(a, b), abs=1e-13)


# ---------------------------------------------------------------- invariants

def test_physical_page_permutation_is_bit_exact():
    P, Hq, Hk, D = 4, 4, 2, 16
    pb = dense_problem(21, [1, 3, 2], [9, 13, 6], P, Hq, Hk, D, extra_pages=5)
    o, lse = run_oracle(pb, P, Hq, Hk, D, True, 0.25, 0.0)
    rng = np.random.default_rng(99)
    sigma = rng.permutation(pb["pool"].shape[0])          # new id of old page p is sigma[p]
    pool2 = np.empty_like(pb["pool"])
    pool2[sigma] = pb["pool"]
    pb2 = dict(pb, pool=pool2, kv_indices=sigma[pb["kv_indices"]].astype(np.int32))
    o2, lse2 = run_oracle(pb2, P, Hq, Hk, D, True, 0.25, 0.0)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_request_order_does_not_matter():
    P, Hq, Hk, D = 3, 2, 1, 16
    pb = dense_problem(22, [2, 1, 3], [5, 7, 3], P, Hq, Hk, D)
    o, lse = run_oracle(pb, P, Hq, Hk, D, True, 0.3, 0.0)
    order = [2, 0, 1]
    qo_lens = np.diff(pb["qo_indptr"])
    npg = np.diff(pb["kv_indptr"])
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens[order])]).astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(npg[order])]).astype(np.int32)
    kv_indices = np.concatenate([pb["kv_indices"][pb["kv_indptr"][i]:pb["kv_indptr"][i + 1]]
                                 for i in order]).astype(np.int32)
    q = np.concatenate([pb["q"][pb["qo_indptr"][i]:pb["qo_indptr"][i + 1]] for i in order])
    pb2 = dict(pb, q=q, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
               last=pb["last"][order].copy())
    o2, lse2 = run_oracle(pb2, P, Hq, Hk, D, True, 0.3, 0.0)
    for new, old in enumerate(order):
        a, b = pb["qo_indptr"][old], pb["qo_indptr"][old + 1]
        c, d = qo_indptr[new], qo_indptr[new + 1]
        assert np.array_equal(o[a:b], o2[c:d]) and np.array_equal(lse[a:b], lse2[c:d])


def _sub_request(pb, i, page_lo, page_hi, P):
    """Request i restricted to its pages [page_lo, page_hi), as a decode batch."""
    ids = pb["kv_indices"][pb["kv_indptr"][i] + page_lo: pb["kv_indptr"][i] + page_hi]
    full = pb["kv_indptr"][i + 1] - pb["kv_indptr"][i]
    last = pb["last"][i] if page_hi == full else P
    return ids.astype(np.int32), np.array([0, len(ids)], np.int32), np.array([last], np.int32)


@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_split_then_merge_equals_unsplit(cap):
    P, Hq, Hk, D = 4, 8, 2, 32
    L = 61
    pb = dense_problem(23, [1], [L], P, Hq, Hk, D)
    full_o, full_lse = run_oracle(pb, P, Hq, Hk, D, True, 0.2, cap)
    npg = _pages(L, P)
    cuts = [0, 3, 4, 11, npg]
    parts_o, parts_l = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        ids, indptr, last = _sub_request(pb, 0, lo, hi, P)
        sub = dict(pb, kv_indices=ids, kv_indptr=indptr, last=last)
        o, l = run_oracle(sub, P, Hq, Hk, D, False, 0.2, cap)
        parts_o.append(o)
        parts_l.append(l)
    mo, ml = ref.merge_states(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, full_lse, rtol=0, atol=1e-12)


def test_merge_identity_commutativity_associativity():
    rng = np.random.default_rng(8)
    n, D = 5, 7
    o = rng.standard_normal((3, n, D))
    l = rng.standard_normal((3, n)) * 4
    empty_o = np.zeros((n, D))
    empty_l = np.full(n, -np.inf)
    mo, ml = ref.merge_states(np.stack([o[0], empty_o]), np.stack([l[0], empty_l]))
    np.testing.assert_allclose(mo, o[0], atol=1e-15)
    np.testing.assert_allclose(ml, l[0], atol=1e-15)
    eo, el = ref.merge_states(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(eo == 0) and np.all(el == -np.inf)
    a = ref.merge_states(o[[0, 1]], l[[0, 1]])
    b = ref.merge_states(o[[1, 0]], l[[1, 0]])
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    ab_c = ref.merge_states(np.stack([a[0], o[2]]), np.stack([a[1], l[2]]))
    bc = ref.merge_states(o[[1, 2]], l[[1, 2]])
    a_bc = ref.merge_states(np.stack([o[0], bc[0]]), np.stack([l[0], bc[1]]))
    abc = ref.merge_states(o, l)
    for x in (ab_c, a_bc):
        np.testing.assert_allclose(x[0], abc[0], atol=1e-13)
        np.testing.assert_allclose(x[1], abc[1], atol=1e-13)
    # the merged lse is the log of the summed normalisers
    np.testing.assert_allclose(abc[1], np.log(np.exp(l).sum(axis=0)), atol=1e-12)


def test_cascade_equals_flat_small():
    """Shared prefix attended once per group, merged with each suffix, equals
    the flat view whose every request lists the prefix pages itself."""
    import workloads
    cb = workloads.shared_prefix_cascade(num_requests=5, prefix_len=32, suffix_lo=1,
                                         suffix_hi=9, seed=77, num_qo_heads=8, num_kv_heads=2,
                                         head_dim=16, page_size=4, dtype=torch.float32,
                                         soft_cap=3.0)
    fo, fl = ref.attention_of(cb.flat)
    co, cl = ref.cascade_of(cb.level0, cb.level1, np.arange(5))
    np.testing.assert_allclose(co, fo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(cl, fl, rtol=0, atol=1e-12)


def test_nan_in_unread_slots_is_ignored():
    import workloads
    b = workloads.make_batch(31, [3, 1, 5], [7, 1, 19], page_size=4, num_qo_heads=4,
                             num_kv_heads=2, head_dim=16, dtype=torch.float32,
                             nan_poison=True)
    o, lse = ref.attention_of(b)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_rows_api_matches_full_api():
    import workloads
    b = workloads.make_batch(32, [3, 2, 5], [7, 2, 19], page_size=4, num_qo_heads=4,
                             num_kv_heads=1, head_dim=16, dtype=torch.float32)
    o, lse = ref.attention_of(b)
    rows = np.array([[0, 2, 3], [2, 0, 1], [1, 1, 0], [2, 4, 2]], np.int32)
    ro, rl = ref.attention_rows_of(b, rows)
    for k, (i, t, h) in enumerate(rows):
        g = b.qo_indptr[i] + t
        assert np.array_equal(ro[k], o[g, h]) and rl[k] == lse[g, h]


@pytest.mark.parametrize("mutate", ["indptr_decreasing", "last_zero", "last_too_big",
                                    "causal_qo_gt_kv", "page_out_of_pool"])
def test_oracle_rejects_invalid_index_arrays(mutate):
    P, Hq, Hk, D = 4, 2, 1, 8
    pb = dense_problem(41, [2, 1], [6, 3], P, Hq, Hk, D)
    causal = True
    if mutate == "indptr_decreasing":
        pb["kv_indptr"] = np.array([0, 2, 1], np.int32)
    elif mutate == "last_zero":
        pb["last"] = np.array([0, 3], np.int32)
    elif mutate == "last_too_big":
        pb["last"] = np.array([2, P + 1], np.int32)
    elif mutate == "causal_qo_gt_kv":
        pb["qo_indptr"] = np.array([0, 7, 8], np.int32)
        pb["q"] = np.zeros((8, Hq, D))
    elif mutate == "page_out_of_pool":
        pb["kv_indices"] = pb["kv_indices"].copy()
        pb["kv_indices"][0] = pb["pool"].shape[0]
    with pytest.raises(ref.OracleError):
        run_oracle(pb, P, Hq, Hk, D, causal, 1.0, 0.0)


# --------------------------------------------------------------------------
# Sliding window (paper page: sliding windows among the attention variants,
# a variant being a mask).  Pins: a window as long as the request changes
# nothing; window 0 leaves the query's own key (closed form); and every query
# row equals the unwindowed oracle on a truncated copy of its visible keys.
# --------------------------------------------------------------------------

def _window_batch(seed, qo, kv, P, causal, cap=0.0):
    import workloads as wl
    return wl.make_batch(seed, qo, kv, page_size=P, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                         dtype=torch.float32, causal=causal, soft_cap=cap)


def _keys_of(b, i):
    """Request i's K and V rows [kv_len, Hk, D], gathered token by token."""
    pool = b.kv_pool.numpy()
    n = int(b.kv_indptr[i + 1] - b.kv_indptr[i])
    L = 0 if n == 0 else (n - 1) * b.page_size + int(b.kv_last_page_len[i])
    pages = b.kv_indices[b.kv_indptr[i]:b.kv_indptr[i + 1]]
    j = np.arange(L)
    return pool[pages[j // b.page_size], 0, j % b.page_size], pool[pages[j // b.page_size], 1, j % b.page_size]


@pytest.mark.parametrize("causal", [True, False])
def test_window_as_long_as_the_request_changes_nothing(causal):
    b = _window_batch(501, [1, 3, 7], [40, 19, 7], 4, causal)
    o0, l0 = ref.attention_of(b)
    o1, l1 = ref.attention_of(b, window_left=40)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_zero_keeps_the_querys_own_key():
    b = _window_batch(502, [1, 5], [23, 9], 4, True, cap=7.0)
    o, lse = ref.attention_of(b, window_left=0)
    qo = b.qo_indptr
    for i in range(2):
        K, V = _keys_of(b, i)
        L, n = K.shape[0], qo[i + 1] - qo[i]
        for t in range(n):
            p = L - n + t
            for h in range(4):
                g = h // 2
                s = b.sm_scale * float(np.dot(b.q[qo[i] + t, h].double().numpy(), K[p, g]))
                s = 7.0 * math.tanh(s / 7.0)
                assert np.allclose(o[qo[i] + t, h], V[p, g], rtol=0, atol=1e-12)
                assert abs(lse[qo[i] + t, h] - s) < 1e-12


@pytest.mark.parametrize("causal,cap", [(True, 0.0), (False, 0.0), (True, 9.0)])
def test_window_equals_attention_over_the_visible_keys_alone(causal, cap):
    import workloads as wl
    b = _window_batch(503, [1, 6, 4, 2], [37, 30, 4, 18], 4, causal, cap)
    for w in (1, 3, 8, 17):
        o, lse = ref.attention_of(b, window_left=w)
        qo = b.qo_indptr
        for i in range(4):
            K, V = _keys_of(b, i)
            L, n = K.shape[0], qo[i + 1] - qo[i]
            for t in range(n):
                p = L - n + t
                hi = p + 1 if causal else L
                keep = np.arange(max(0, p - w), hi)
                # one query over exactly the kept keys, one token per page, no mask
                m = len(keep)
                pool = np.zeros((m, 2, 1, 2, 8), np.float32)
                pool[:, 0, 0] = K[keep]
                pool[:, 1, 0] = V[keep]
                sub = wl.PagedBatch(page_size=1, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                                    dtype=torch.float32, causal=False, sm_scale=b.sm_scale,
                                    soft_cap=cap, qo_lens=np.array([1]), kv_lens=np.array([m]),
                                    qo_indptr=np.array([0, 1], np.int32),
                                    kv_indptr=np.array([0, m], np.int32),
                                    kv_indices=np.arange(m, dtype=np.int32),
                                    kv_last_page_len=np.array([1], np.int32),
                                    q=b.q[qo[i] + t:qo[i] + t + 1].clone(),
                                    kv_pool=torch.from_numpy(pool))
                o_s, l_s = ref.attention_of(sub)
                assert np.allclose(o[qo[i] + t], o_s[0], rtol=0, atol=1e-12), (w, i, t)
                assert np.allclose(lse[qo[i] + t], l_s[0], rtol=0, atol=1e-12), (w, i, t)


# ---- rotary embedding (rotate-half reading: the pair (x[d], x[d + D/2])
# turns by pos / scale * theta^(-2d/D); key j at position j, query t at
# kv_len - qo_len + t)

def _rope_pair_case(q, k0, k1, theta, scale):
    """One decode request with two keys (positions 0 and 1), D = 4; the query
    sits at position 1.  V = identity rows so o reads back the weights."""
    P = 2
    pool = np.zeros((1, 2, P, 1, 4))
    pool[0, 0, 0, 0] = k0
    pool[0, 0, 1, 0] = k1
    pool[0, 1, 0, 0] = [1, 0, 0, 0]
    pool[0, 1, 1, 0] = [0, 1, 0, 0]
    qa = np.asarray(q, np.float64).reshape(1, 1, 4)
    return ref.attention(qa, pool, None, np.array([0, 1], np.int32), np.array([0], np.int32),
                         np.array([2], np.int32), page_size=P, num_qo_heads=1, num_kv_heads=1,
                         head_dim=4, causal=True, sm_scale=1.0, rope_theta=theta, rope_scale=scale)


@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_rope_closed_form_first_pair(scale):
    # pair d = 0 turns by pos / scale rad: q = e0 at position 1 becomes
    # (cos a, 0, sin a, 0); k0 = e0 at position 0 stays; k1 = e2 at
    # position 1 becomes (-sin a, 0, cos a, 0).  Logits cos a and 0.
    a = 1.0 / scale
    o, lse = _rope_pair_case([1, 0, 0, 0], [1, 0, 0, 0], [0, 0, 1, 0], 100.0, scale)
    s0, s1 = math.cos(a), 0.0
    assert lse[0, 0] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), abs=1e-14)
    w0 = math.exp(s0) / (math.exp(s0) + math.exp(s1))
    assert o[0, 0, 0] == pytest.approx(w0, abs=1e-14) and o[0, 0, 1] == pytest.approx(1 - w0, abs=1e-14)


@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_rope_closed_form_second_pair(scale):
    # pair d = 1 of D = 4 turns by pos / scale * theta^(-1/2) = 0.1 / scale
    # at theta 100: logits cos(0.1 / scale) (k0 = e1 at position 0) and 0
    # (k1 = e3 at position 1).
    a = 0.1 / scale
    o, lse = _rope_pair_case([0, 1, 0, 0], [0, 1, 0, 0], [0, 0, 0, 1], 100.0, scale)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(math.cos(a)) + 1.0), abs=1e-14)


def test_rope_at_position_zero_is_the_identity():
    # one key, one query: both at position 0, so the logit (= lse) is the
    # plain scaled dot product and o is the key's value
    b = _window_batch(601, [1, 1], [1, 1], 4, True)
    o0, l0 = ref.attention_of(b)
    o1, l1 = ref.attention_of(b, rope_theta=10000.0)
    assert np.allclose(l0, l1, atol=1e-14, rtol=0) and np.allclose(o0, o1, atol=1e-14, rtol=0)


def _rotate_complex(x, pos, theta, scale):
    """Independent form of the rotation: pair (x[d], x[d + D/2]) as the
    complex number x[d] + i x[d + D/2], multiplied by exp(i angle)."""
    D = x.shape[-1]
    h = D // 2
    ang = np.asarray(pos, np.float64)[..., None] / scale * theta ** (-2.0 * np.arange(h) / D)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("causal,theta,scale", [(True, 10000.0, 1.0), (False, 500.0, 4.0),
                                                 (True, 1e6, 0.5)])
def test_rope_equals_plain_attention_on_rotated_inputs(causal, theta, scale):
    """Rotating q and every cached key up front (complex form, numpy) and
    running plain attention gives the fused result: this pins the positions
    (key j at j, query t at kv_len - qo_len + t) and the frequencies."""
    b = _window_batch(602, [1, 6, 3], [37, 13, 3], 4, causal)
    q = b.q.numpy().astype(np.float64)
    pool = b.kv_pool.numpy().astype(np.float64).copy()
    qr = q.copy()
    for i in range(3):
        kv = int(b.kv_lens[i])
        q0, q1 = int(b.qo_indptr[i]), int(b.qo_indptr[i + 1])
        qr[q0:q1] = _rotate_complex(q[q0:q1], (kv - (q1 - q0) + np.arange(q1 - q0))[:, None], theta, scale)
        pages = b.kv_indices[b.kv_indptr[i]:b.kv_indptr[i + 1]]
        for j in range(kv):
            pg, sl = pages[j // 4], j % 4
            pool[pg, 0, sl] = _rotate_complex(pool[pg, 0, sl], np.full(pool.shape[3], j), theta, scale)
    o0, l0 = ref.attention(qr, pool, b.qo_indptr, b.kv_indptr, b.kv_indices, b.kv_last_page_len,
                           page_size=4, num_qo_heads=4, num_kv_heads=2, head_dim=8, causal=causal,
                           sm_scale=b.sm_scale)
    o1, l1 = ref.attention_of(b, rope_theta=theta, rope_scale=scale)
    assert np.allclose(o0, o1, atol=1e-12, rtol=0) and np.allclose(l0, l1, atol=1e-12, rtol=0)


def test_rope_logits_depend_only_on_relative_positions():
    """A request whose keys sit c positions later (c extra keys in front,
    hidden by a window) gives the same output: rotary logits depend only
    on position differences."""
    import workloads as wl
    c, L, w = 9, 20, 11
    a = wl.make_batch(603, None, [L], page_size=1, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                      dtype=torch.float32, decode=True)
    bb = wl.make_batch(604, None, [L + c], page_size=1, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                       dtype=torch.float32, decode=True)
    pa, pb = a.kv_pool.numpy(), bb.kv_pool.numpy().copy()
    for j in range(L):   # B's key c + j = A's key j (pages of one token each)
        pb[bb.kv_indices[c + j]] = pa[a.kv_indices[j]]
    bb.kv_pool = torch.from_numpy(pb)
    bb.q = a.q.clone()
    oa, la = ref.attention_of(a, window_left=w, rope_theta=10000.0)
    ob, lb = ref.attention_of(bb, window_left=w, rope_theta=10000.0)
    assert np.allclose(oa, ob, atol=1e-12, rtol=0) and np.allclose(la, lb, atol=1e-12, rtol=0)
    # without the rotation the shift changes nothing either, with it off the
    # window alone decides; with a different key set the outputs differ
    on, ln = ref.attention_of(a, window_left=w)
    assert not np.allclose(on, oa, atol=1e-6)


# ---- tree mask (speculative decoding: the draft tokens are the request's
# last qo_len keys; draft token t sees the keys before the draft, itself and
# the draft tokens whose bit (t, u) is set, never a later one)
# --------------------------------------------------------------------------

def _tree_batch(seed, qo, kv, P, cap=0.0, D=8):
    import workloads as wl
    b = wl.make_batch(seed, qo, kv, page_size=P, num_qo_heads=4, num_kv_heads=2, head_dim=D,
                      dtype=torch.float32, causal=True, soft_cap=cap)
    rng = np.random.default_rng(seed + 1)
    parents = [wl.random_tree_parents(rng, int(n), max_children=2) for n in qo]
    b.tree_mask, b.mask_indptr = wl.tree_mask_bits(parents, qo)
    return b, parents


def _lower_block(qo, fill):
    """Bits of per-request qo x qo blocks from a function fill(i, t, u)."""
    bits = []
    for i, n in enumerate(qo):
        for t in range(n):
            for u in range(n):
                bits.append(bool(fill(i, t, u)))
    ind = np.zeros(len(qo) + 1, np.int32)
    ind[1:] = np.cumsum([n * n for n in qo])
    return np.packbits(np.array(bits, bool), bitorder="little"), ind


def test_tree_mask_of_the_whole_lower_triangle_is_causal():
    b, _ = _tree_batch(601, [5, 1, 9, 3], [20, 7, 9, 30], 4, cap=6.0)
    qo = [5, 1, 9, 3]
    bits, ind = _lower_block(qo, lambda i, t, u: u <= t)
    o0, l0 = ref.attention_of(b, tree_mask=None, mask_indptr=None)
    o1, l1 = ref.attention_of(b, tree_mask=bits, mask_indptr=ind)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_tree_mask_ignores_bits_above_the_diagonal():
    b, _ = _tree_batch(602, [6, 4], [30, 4], 3)
    qo = [6, 4]
    rng = np.random.default_rng(7)
    r = rng.random((2, 6, 6)) < 0.5
    full, ind = _lower_block(qo, lambda i, t, u: r[i, t, u])
    low, _ = _lower_block(qo, lambda i, t, u: r[i, t, u] and u <= t)
    o0, l0 = ref.attention_of(b, tree_mask=full, mask_indptr=ind)
    o1, l1 = ref.attention_of(b, tree_mask=low, mask_indptr=ind)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_tree_mask_single_query_requests_ignore_their_bit():
    import workloads as wl
    b = wl.make_batch(603, [1, 1, 1], [9, 1, 40], page_size=4, num_qo_heads=4, num_kv_heads=2,
                      head_dim=8, dtype=torch.float32, causal=True)
    o0, l0 = ref.attention_of(b)
    zero = np.zeros(1, np.uint8)
    o1, l1 = ref.attention_of(b, tree_mask=zero, mask_indptr=np.array([0, 1, 2, 3], np.int32))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("cap", [0.0, 5.0])
def test_tree_mask_equals_dense_attention_over_prefix_and_ancestors(cap):
    """Brute force per query row: dense softmax over exactly the keys before
    the draft, the row's own key and its ancestors' keys (walked from the
    parent array, not from the bits)."""
    qo = [7, 2, 12, 1, 5]
    kv = [19, 2, 40, 6, 5]
    b, parents = _tree_batch(604, qo, kv, 4, cap=cap)
    o, lse = ref.attention_of(b)
    qi = b.qo_indptr
    for i in range(len(qo)):
        K, V = _keys_of(b, i)
        L, n = K.shape[0], qo[i]
        d0 = L - n
        for t in range(n):
            keep = list(range(d0))
            u = t
            while u >= 0:
                keep.append(d0 + u)
                u = int(parents[i][u])
            keep = np.array(sorted(keep))
            Q = b.q[qi[i] + t:qi[i] + t + 1].double().numpy()
            o_d, l_d = dense_ref(Q, K[keep].astype(np.float64), V[keep].astype(np.float64),
                                 b.sm_scale, cap, causal=False)
            assert np.allclose(o[qi[i] + t], o_d[0], rtol=0, atol=1e-12), (i, t)
            assert np.allclose(lse[qi[i] + t], l_d[0], rtol=0, atol=1e-12), (i, t)


def test_tree_mask_with_no_bits_sees_the_prefix_and_itself():
    qo = [4, 6]
    kv = [4, 13]
    b, _ = _tree_batch(605, qo, kv, 2)
    bits, ind = _lower_block(qo, lambda i, t, u: False)
    o, lse = ref.attention_of(b, tree_mask=bits, mask_indptr=ind)
    qi = b.qo_indptr
    for i in range(2):
        K, V = _keys_of(b, i)
        d0 = K.shape[0] - qo[i]
        for t in range(qo[i]):
            keep = np.array(list(range(d0)) + [d0 + t])
            Q = b.q[qi[i] + t:qi[i] + t + 1].double().numpy()
            o_d, l_d = dense_ref(Q, K[keep].astype(np.float64), V[keep].astype(np.float64),
                                 b.sm_scale, 0.0, causal=False)
            assert np.allclose(o[qi[i] + t], o_d[0], rtol=0, atol=1e-12)
            assert np.allclose(lse[qi[i] + t], l_d[0], rtol=0, atol=1e-12)


def test_tree_mask_is_invariant_under_page_permutation():
    b, _ = _tree_batch(606, [9, 3], [25, 11], 4)
    o0, l0 = ref.attention_of(b)
    rng = np.random.default_rng(8)
    sigma = rng.permutation(b.pool_pages)
    pool2 = torch.empty_like(b.kv_pool)
    pool2[torch.from_numpy(sigma)] = b.kv_pool
    b.kv_pool = pool2
    b.kv_indices = sigma[b.kv_indices].astype(np.int32)
    o1, l1 = ref.attention_of(b)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_tree_mask_rejects_non_causal_and_bad_offsets():
    b, _ = _tree_batch(607, [3, 2], [5, 9], 4)
    with pytest.raises(ref.OracleError):
        ref.attention_of(b, causal=False)
    with pytest.raises(ref.OracleError):
        ref.attention_of(b, mask_indptr=np.array([0, 9, 12], np.int32))


def test_tree_mask_matches_torch_sdpa_with_a_boolean_mask():
    """The library routine as a second pin: torch's fp64 scaled-dot-product
    attention over the request's gathered keys with the boolean mask built
    from the parent array (prefix columns all true, draft columns true for
    the row's own token and its ancestors)."""
    import workloads as wl
    qo, kv = [9, 4], [30, 4]
    b, parents = _tree_batch(608, qo, kv, 4, D=16)
    o, lse = ref.attention_of(b)
    F = torch.nn.functional
    qi = b.qo_indptr
    for i in range(2):
        K, V = _keys_of(b, i)
        n, L = qo[i], K.shape[0]
        m = torch.zeros(n, L, dtype=torch.bool)
        m[:, :L - n] = True
        for t in range(n):
            u = t
            while u >= 0:
                m[t, L - n + u] = True
                u = int(parents[i][u])
        Q = b.q[qi[i]:qi[i] + n].double().permute(1, 0, 2)[None]                  # [1, Hq, n, D]
        Kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)[None].repeat_interleave(2, dim=1)
        Vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)[None].repeat_interleave(2, dim=1)
        out = F.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=m, scale=b.sm_scale)
        np.testing.assert_allclose(o[qi[i]:qi[i] + n], out[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        s = torch.einsum("bhtd,bhjd->bhtj", Q, Kt) * b.sm_scale
        s = s.masked_fill(~m, -math.inf)
        np.testing.assert_allclose(lse[qi[i]:qi[i] + n], torch.logsumexp(s, dim=-1)[0].T.numpy(),
                                   rtol=0, atol=1e-12)
