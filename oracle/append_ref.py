"""Paged KV append, written out in numpy.

TEST INFRASTRUCTURE ONLY: used by tests/ and nothing on the product path.

What it follows.
- Talk page, Background, "Dynamic Problem Shapes": the append stage adds a
  step's new tokens to the KV cache.
- Serving-engine page, "Page-Level Attention": a request's tokens fill the
  pages of its page table in order, page_size tokens per page, and the last
  page holds kv_last_page_len of them.

Reading (the pages give no call for it).  The index arrays describe each
request's pages after the append, and request i's n_i new tokens are its last
n_i tokens: new token t sits at position kv_len_i - n_i + t.

The oracle places only tokens that have a place: a position inside the
request and a page-table entry that names a page of the pool.  The pages say
nothing about other inputs, so the oracle raises on them; what the library
does with them is its own contract, stated in its header and tested as such,
not as parity with the method.
"""
from __future__ import annotations

import numpy as np


def kv_len(kv_indptr, kv_last_page_len, page_size, i) -> int:
    """Tokens of request i from its page count and last-page length."""
    n = int(kv_indptr[i + 1]) - int(kv_indptr[i])
    return 0 if n == 0 else (n - 1) * page_size + int(kv_last_page_len[i])


def slot_of(kv_indptr, kv_indices, page_size, i, pos):
    """(page id, slot) of position `pos` of request i, or None if the page
    table has no entry for it."""
    e = int(kv_indptr[i]) + pos // page_size
    if pos < 0 or e < 0 or e >= len(kv_indices):
        return None
    return int(kv_indices[e]), pos % page_size


class Unplaceable(ValueError):
    """A new token with no place in the pool (the pages define none)."""


def append(pool, k, v, append_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size):
    """A copy of `pool` ([pages, 2, page_size, Hk, D]) with the rows of `k`
    and `v` ([n_tokens, Hk, D]) written into their slots.  A token without a
    place raises ``Unplaceable``."""
    out = np.array(pool, copy=True)
    B = len(append_indptr) - 1
    for i in range(B):
        a0, a1 = int(append_indptr[i]), int(append_indptr[i + 1])
        n = a1 - a0
        L = kv_len(kv_indptr, kv_last_page_len, page_size, i)
        for t in range(n):
            ps = slot_of(kv_indptr, kv_indices, page_size, i, L - n + t)
            if ps is None or not 0 <= ps[0] < out.shape[0]:
                raise Unplaceable(f"request {i}, new token {t}: no slot in the pool")
            page, slot = ps
            out[page, 0, slot] = k[a0 + t]
            out[page, 1, slot] = v[a0 + t]
    return out
