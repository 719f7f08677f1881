"""Pins of the paged KV append oracle (oracle/append_ref.py), on the CPU.

- the pages' own page-table example (tests/golden/page_table_example.json):
  every token lands on the page and slot the example lists;
- appending a whole request into an empty pool, then concatenating its pages
  in page-table order, gives back the appended rows (the pages' "tokens fill
  the pages in order"), and nothing outside those slots changes;
- appending in two steps (the page table growing in between) equals
  appending once, across page boundaries;
- a new token with no place (the request does not hold it, or its page id
  is outside the pool) is refused: the pages define no such input.
"""
import json
import os

import numpy as np
import pytest

from oracle import append_ref as ap

HERE = os.path.dirname(os.path.abspath(__file__))


def _indptr(counts):
    out = np.zeros(len(counts) + 1, np.int32)
    out[1:] = np.cumsum(counts)
    return out


def test_token_slots_of_the_pages_example():
    g = json.load(open(os.path.join(HERE, "golden", "page_table_example.json")))
    P = g["page_size"]
    tables = [r["page_table"] for r in g["requests"]]
    kv_indptr = _indptr([len(t) for t in tables])
    kv_indices = np.concatenate([np.asarray(t, np.int32) for t in tables])
    last = np.asarray(g["expected_last_page_len"], np.int32)
    for i, r in enumerate(g["requests"]):
        assert ap.kv_len(kv_indptr, last, P, i) == g["expected_kv_len"][i]
        for lo, hi, page in r["ranges"]:
            for pos in range(lo, hi + 1):
                assert ap.slot_of(kv_indptr, kv_indices, P, i, pos) == (page, pos - lo)
    # request 1's last five tokens (96..100) go to page 7, slots 32..36
    pool = np.zeros((16, 2, P, 1, 2))
    k = np.arange(10, dtype=np.float64).reshape(5, 1, 2) + 1.0
    out = ap.append(pool, k, -k, np.array([0, 0, 5], np.int32), kv_indptr, kv_indices, last, P)
    assert np.array_equal(out[7, 0, 32:37], k) and np.array_equal(out[7, 1, 32:37], -k)
    out[7, :, 32:37] = 0.0
    assert not out.any()


def test_whole_requests_read_back_through_their_pages():
    rng = np.random.default_rng(9101)
    for P in (1, 3, 16):
        lens = [0, 1, P, P + 1, 5 * P - 2, 37]
        counts = [(L + P - 1) // P for L in lens]
        pool_pages = sum(counts) + 7
        perm = rng.permutation(pool_pages).astype(np.int32)
        kv_indptr = _indptr(counts)
        kv_indices = perm[: sum(counts)]
        last = np.array([L - (c - 1) * P if c else 0 for L, c in zip(lens, counts)], np.int32)
        Hk, D = 2, 4
        k = rng.standard_normal((sum(lens), Hk, D))
        v = rng.standard_normal((sum(lens), Hk, D))
        pool = rng.standard_normal((pool_pages, 2, P, Hk, D))
        out = ap.append(pool, k, v, _indptr(lens), kv_indptr, kv_indices, last, P)
        written = np.zeros(out.shape[:3], bool)
        a = 0
        for i, L in enumerate(lens):
            pages = kv_indices[kv_indptr[i]:kv_indptr[i + 1]]
            if L:
                seq_k = np.concatenate([out[p, 0] for p in pages])[:L]
                seq_v = np.concatenate([out[p, 1] for p in pages])[:L]
                assert np.array_equal(seq_k, k[a:a + L]) and np.array_equal(seq_v, v[a:a + L])
                for j, p in enumerate(pages):
                    written[p, :, : min(P, L - j * P)] = True
            a += L
        assert np.array_equal(out[~written], pool[~written])


def test_two_appends_equal_one():
    rng = np.random.default_rng(9102)
    P, Hk, D = 4, 1, 3
    lens = [9, 4, 13]            # after the second append
    first = [6, 1, 8]            # after the first
    counts = [(L + P - 1) // P for L in lens]
    kv_indices = rng.permutation(sum(counts) + 3)[: sum(counts)].astype(np.int32)
    kv_indptr = _indptr(counts)
    last = np.array([L - (c - 1) * P for L, c in zip(lens, counts)], np.int32)
    k = rng.standard_normal((sum(lens), Hk, D))
    pool = np.zeros((len(kv_indices) + 3, 2, P, Hk, D))
    once = ap.append(pool, k, k, _indptr(lens), kv_indptr, kv_indices, last, P)
    # step 1: the first tokens of each request, with the page table of that moment
    c1 = [(L + P - 1) // P for L in first]
    idx1 = np.concatenate([kv_indices[kv_indptr[i]:kv_indptr[i] + c1[i]] for i in range(3)])
    last1 = np.array([L - (c - 1) * P for L, c in zip(first, c1)], np.int32)
    starts = _indptr(lens)[:-1]
    k1 = np.concatenate([k[s:s + f] for s, f in zip(starts, first)])
    step1 = ap.append(pool, k1, k1, _indptr(first), _indptr(c1), idx1, last1, P)
    # step 2: the rest, with the final page table
    rest = [L - f for L, f in zip(lens, first)]
    k2 = np.concatenate([k[s + f:s + L] for s, f, L in zip(starts, first, lens)])
    step2 = ap.append(step1, k2, k2, _indptr(rest), kv_indptr, kv_indices, last, P)
    assert np.array_equal(step2, once)


def test_tokens_without_a_place_are_refused():
    """The pages define where a new token goes only when the request holds it
    and its page-table entry names a page of the pool; the oracle raises on
    anything else rather than pick a behaviour."""
    P = 4
    kv_indptr, kv_indices, last = _indptr([1]), np.array([2], np.int32), np.array([3], np.int32)
    k = np.arange(5, dtype=np.float64).reshape(5, 1, 1) + 1.0
    pool = np.zeros((4, 2, P, 1, 1))
    with pytest.raises(ap.Unplaceable):   # 5 new tokens, 3 held
        ap.append(pool, k, k, np.array([0, 5], np.int32), kv_indptr, kv_indices, last, P)
    with pytest.raises(ap.Unplaceable):   # a page id outside the pool
        ap.append(pool, k[:2], k[:2], np.array([0, 2], np.int32), kv_indptr, np.array([9], np.int32), last, P)
    out = ap.append(pool, k[:3], k[:3], np.array([0, 3], np.int32), kv_indptr, kv_indices, last, P)
    assert np.array_equal(out[2, 0, :3, 0, 0], [1.0, 2.0, 3.0])
