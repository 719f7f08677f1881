"""Seeded synthetic inputs for batched attention over a paged KV cache.

This module only draws lengths, page permutations and random values, and
builds the page-table index arrays (kv_indptr / kv_indices / kv_last_page_len,
qo_indptr) that describe them.  It holds none of the attention arithmetic: both
the fp64 oracle and the GPU library consume what it produces.

Layout of the page pool (FlashInfer MLSys 2025 pages, "Page-Level Attention"):
``[num_pages, 2, page_size, num_kv_heads, head_dim]``, axis 1 index 0 = K,
1 = V (the NHD layout of the tiny decode workload).  Request ``i`` owns pages
``kv_indices[kv_indptr[i]:kv_indptr[i+1]]`` in logical order; its last page
holds ``kv_last_page_len[i]`` valid tokens.

Random draws happen in a fixed order: (1) lengths, (2) the page permutation of
the pool, (3) Q, (4) pool K/V.  Values are N(0, 1) drawn in fp32 and rounded to
the storage dtype (round-to-nearest-even for bf16); the oracle consumes exactly
those rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = [
    "PagedBatch",
    "CascadeBatch",
    "make_batch",
    "tiny_decode_fp32",
    "llama8b_decode",
    "skewed_long_decode",
    "mixed_ragged_step",
    "shared_prefix_cascade",
    "WORKLOADS",
]


@dataclass
class PagedBatch:
    """One batch of requests over a paged KV pool (host tensors)."""

    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    causal: bool
    sm_scale: float
    soft_cap: float
    qo_lens: np.ndarray            # int64 [B]
    kv_lens: np.ndarray            # int64 [B]
    qo_indptr: Optional[np.ndarray]  # int32 [B+1]; None means every qo_len is 1 (decode)
    kv_indptr: np.ndarray          # int32 [B+1]
    kv_indices: np.ndarray         # int32 [nnz pages]
    kv_last_page_len: np.ndarray   # int32 [B]
    q: torch.Tensor                # [sum(qo_lens), Hq, D]
    kv_pool: torch.Tensor          # [pool_pages, 2, P, Hk, D]
    name: str = ""
    meta: dict = field(default_factory=dict)
    window_left: int = -1          # sliding window (keys before the query's own); -1 = none
    tree_mask: Optional[np.ndarray] = None    # uint8 bits (speculative-decoding token trees); None = none
    mask_indptr: Optional[np.ndarray] = None  # int32 [B+1]: bit offset of request i's qo x qo block

    @property
    def batch_size(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def total_qo(self) -> int:
        return int(self.q.shape[0])

    @property
    def pool_pages(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def group_size(self) -> int:
        return self.num_qo_heads // self.num_kv_heads


@dataclass
class CascadeBatch:
    """A batch whose requests share one prefix, with flat and two-level index arrays.

    ``flat`` lists, for every request, the shared prefix pages followed by its
    own suffix pages.  ``level0`` stacks all requests' queries as one request
    over the prefix pages; ``level1`` holds each request's suffix pages.  Both
    views index the same pool: only the index arrays differ.
    """

    flat: PagedBatch
    level0: PagedBatch
    level1: PagedBatch
    prefix_len: int
    suffix_lens: np.ndarray


def _pages_for(kv_len: int, page_size: int) -> int:
    return (kv_len + page_size - 1) // page_size


def _last_len(kv_len: int, page_size: int) -> int:
    """Valid tokens on the last page (0 when the request has no pages)."""
    if kv_len == 0:
        return 0
    return kv_len - (_pages_for(kv_len, page_size) - 1) * page_size


def _draw_values(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    return x.to(dtype)


def _index_arrays(kv_lens, page_size, perm, start=0):
    """Assign each request the next ceil(kv_len/P) pages of ``perm``."""
    B = len(kv_lens)
    kv_indptr = np.zeros(B + 1, dtype=np.int32)
    last = np.zeros(B, dtype=np.int32)
    idx = []
    pos = start
    for i, L in enumerate(kv_lens):
        n = _pages_for(int(L), page_size)
        idx.append(perm[pos:pos + n])
        pos += n
        kv_indptr[i + 1] = kv_indptr[i] + n
        last[i] = _last_len(int(L), page_size)
    kv_indices = (np.concatenate(idx) if idx else np.zeros(0, np.int64)).astype(np.int32)
    return kv_indptr, kv_indices, last, pos


def _poison(pool: torch.Tensor, kv_indptr, kv_indices, last, page_size):
    """Fill every unreferenced page and every slot past a request's last
    valid token with NaN (they must never influence a result)."""
    used = np.zeros(pool.shape[0], dtype=bool)
    used[kv_indices] = True
    pool[torch.from_numpy(~used)] = float("nan")
    for i in range(len(last)):
        n = kv_indptr[i + 1] - kv_indptr[i]
        if n > 0 and last[i] < page_size:
            pool[int(kv_indices[kv_indptr[i + 1] - 1]), :, int(last[i]):] = float("nan")


def make_batch(seed: int, qo_lens, kv_lens, *, page_size=16, num_qo_heads=32,
               num_kv_heads=8, head_dim=128, dtype=torch.bfloat16, causal=True,
               decode=False, pool_factor=1.25, pool_pages=None, soft_cap=0.0,
               sm_scale=None, nan_poison=False, identity_pages=False,
               name="", window_left=-1) -> PagedBatch:
    """Generic seeded batch.  ``decode=True`` means qo_indptr is None and every
    request has exactly one query token."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    qo_lens = np.ones_like(kv_lens) if decode else np.asarray(qo_lens, dtype=np.int64)
    b = _assemble(rng, qo_lens, kv_lens, page_size, num_qo_heads, num_kv_heads,
                  head_dim, dtype, causal, decode, pool_factor, pool_pages,
                  soft_cap, sm_scale, nan_poison, identity_pages, name)
    b.window_left = int(window_left)
    return b


def _assemble(rng, qo_lens, kv_lens, P, Hq, Hk, D, dtype, causal, decode,
              pool_factor, pool_pages, soft_cap, sm_scale, nan_poison,
              identity_pages, name, meta=None) -> PagedBatch:
    need = sum(_pages_for(int(L), P) for L in kv_lens)
    if pool_pages is None:
        pool_pages = max(1, int(math.ceil(pool_factor * need)))
    assert pool_pages >= need
    perm = np.arange(pool_pages) if identity_pages else rng.permutation(pool_pages)
    kv_indptr, kv_indices, last, _ = _index_arrays(kv_lens, P, perm)
    total_qo = int(qo_lens.sum())
    q = _draw_values(rng, (total_qo, Hq, D), dtype)
    pool = _draw_values(rng, (pool_pages, 2, P, Hk, D), dtype)
    if nan_poison:
        _poison(pool, kv_indptr, kv_indices, last, P)
    qo_indptr = None
    if not decode:
        qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(qo_lens)
    return PagedBatch(
        page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=D, dtype=dtype,
        causal=bool(causal), sm_scale=(1.0 / math.sqrt(D)) if sm_scale is None else float(sm_scale),
        soft_cap=float(soft_cap), qo_lens=np.asarray(qo_lens, np.int64),
        kv_lens=np.asarray(kv_lens, np.int64), qo_indptr=qo_indptr, kv_indptr=kv_indptr,
        kv_indices=kv_indices, kv_last_page_len=last, q=q, kv_pool=pool, name=name,
        meta=meta or {})


# --------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------

def tiny_decode_fp32(nan_poison=False) -> PagedBatch:
    """Tiny fp32 decode: batch 4, 8 query / 2 KV heads, D=64, P=16,
    kv_lens {17, 64, 100, 3}, a randomly permuted pool of 32 pages."""
    rng = np.random.default_rng(1001)
    kv = np.array([17, 64, 100, 3], dtype=np.int64)
    return _assemble(rng, np.ones(4, np.int64), kv, 16, 8, 2, 64, torch.float32,
                     True, True, 1.0, 32, 0.0, 1.0 / 8.0, nan_poison, False,
                     "tiny_decode_fp32")


def llama8b_decode(nan_poison=False, identity_pages=False) -> PagedBatch:
    """Batch decode, Llama-3-8B attention shape: batch 64, 32/8 heads, D=128,
    bf16, P=16, kv_len uniform in [512, 4096], pool = ceil(1.25 x pages)."""
    rng = np.random.default_rng(1002)
    kv = rng.integers(512, 4096, size=64, endpoint=True).astype(np.int64)
    return _assemble(rng, np.ones(64, np.int64), kv, 16, 32, 8, 128, torch.bfloat16,
                     True, True, 1.25, None, 0.0, None, nan_poison, identity_pages,
                     "llama8b_decode")


def skewed_long_decode(nan_poison=False) -> PagedBatch:
    """Skewed long-context decode: batch 32, request 0 has 131072 tokens, the
    other 31 are lognormal(median 1024, sigma 1) clipped to [128, 4096]."""
    rng = np.random.default_rng(1003)
    rest = np.clip(np.rint(np.exp(rng.normal(math.log(1024.0), 1.0, size=31))), 128, 4096)
    kv = np.concatenate([[131072], rest]).astype(np.int64)
    return _assemble(rng, np.ones(32, np.int64), kv, 16, 32, 8, 128, torch.bfloat16,
                     True, True, 1.25, None, 0.0, None, nan_poison, False,
                     "skewed_long_decode")


def mixed_ragged_step(nan_poison=False) -> PagedBatch:
    """Mixed ragged step: 16 causal prefills with qo_len in {64,128,256,512}
    over a cached prefix uniform in [0, 2048] (kv_len = prefix + qo_len), then
    48 decodes with kv_len uniform in [256, 8192], in one batch."""
    rng = np.random.default_rng(1004)
    qo_p = rng.choice(np.array([64, 128, 256, 512]), size=16)
    prefix = rng.integers(0, 2048, size=16, endpoint=True)
    kv_d = rng.integers(256, 8192, size=48, endpoint=True)
    qo = np.concatenate([qo_p, np.ones(48, np.int64)]).astype(np.int64)
    kv = np.concatenate([prefix + qo_p, kv_d]).astype(np.int64)
    return _assemble(rng, qo, kv, 16, 32, 8, 128, torch.bfloat16, True, False, 1.25,
                     None, 0.0, None, nan_poison, False, "mixed_ragged_step",
                     meta={"num_prefill": 16, "num_decode": 48})


def shared_prefix_cascade(nan_poison=False, num_requests=64, prefix_len=2048,
                          suffix_lo=50, suffix_hi=200, seed=1005,
                          num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          page_size=16, dtype=torch.bfloat16,
                          soft_cap=30.0) -> CascadeBatch:
    """Cascade decode: every request shares one prefix (stored once) and has
    its own suffix (uniform in [suffix_lo, suffix_hi]) on fresh pages; logits
    soft-capped as cap*tanh(s/cap)."""
    assert prefix_len % page_size == 0, "the shared prefix must fill whole pages"
    rng = np.random.default_rng(seed)
    P, Hq, Hk, D = page_size, num_qo_heads, num_kv_heads, head_dim
    suffix = rng.integers(suffix_lo, suffix_hi, size=num_requests, endpoint=True).astype(np.int64)
    n_prefix = prefix_len // P
    need = n_prefix + sum(_pages_for(int(s), P) for s in suffix)
    pool_pages = int(math.ceil(1.25 * need))
    perm = rng.permutation(pool_pages)
    prefix_ids = perm[:n_prefix].astype(np.int32)
    s_indptr, s_indices, s_last, _ = _index_arrays(suffix, P, perm, start=n_prefix)
    q = _draw_values(rng, (num_requests, Hq, D), dtype)
    pool = _draw_values(rng, (pool_pages, 2, P, Hk, D), dtype)

    f_indptr = np.zeros(num_requests + 1, np.int32)
    f_idx = []
    for i in range(num_requests):
        own = s_indices[s_indptr[i]:s_indptr[i + 1]]
        f_idx.append(np.concatenate([prefix_ids, own]))
        f_indptr[i + 1] = f_indptr[i] + n_prefix + len(own)
    f_indices = np.concatenate(f_idx).astype(np.int32)
    # an empty suffix leaves the (full) last prefix page as the flat view's last page
    f_last = np.where(suffix > 0, s_last, P).astype(np.int32)
    if nan_poison:
        _poison(pool, f_indptr, f_indices, f_last, P)
    common = dict(page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=D, dtype=dtype,
                  sm_scale=1.0 / math.sqrt(D), soft_cap=float(soft_cap), q=q, kv_pool=pool)
    ones = np.ones(num_requests, np.int64)
    flat = PagedBatch(causal=True, qo_lens=ones, kv_lens=prefix_len + suffix, qo_indptr=None,
                      kv_indptr=f_indptr, kv_indices=f_indices, kv_last_page_len=f_last,
                      name="shared_prefix_cascade/flat", **common)
    level0 = PagedBatch(causal=False, qo_lens=np.array([num_requests], np.int64),
                        kv_lens=np.array([prefix_len], np.int64),
                        qo_indptr=np.array([0, num_requests], np.int32),
                        kv_indptr=np.array([0, n_prefix], np.int32), kv_indices=prefix_ids.copy(),
                        kv_last_page_len=np.array([P], np.int32),
                        name="shared_prefix_cascade/level0", **common)
    level1 = PagedBatch(causal=True, qo_lens=ones, kv_lens=suffix.copy(), qo_indptr=None,
                        kv_indptr=s_indptr, kv_indices=s_indices, kv_last_page_len=s_last,
                        name="shared_prefix_cascade/level1", **common)
    return CascadeBatch(flat=flat, level0=level0, level1=level1, prefix_len=prefix_len,
                        suffix_lens=suffix)


WORKLOADS = {
    "tiny_decode_fp32": tiny_decode_fp32,
    "llama8b_decode": llama8b_decode,
    "skewed_long_decode": skewed_long_decode,
    "mixed_ragged_step": mixed_ragged_step,
    "shared_prefix_cascade": shared_prefix_cascade,
}


# --------------------------------------------------------------------------
# Token trees of speculative decoding (input structure only).
# --------------------------------------------------------------------------

def random_tree_parents(rng: np.random.Generator, n: int, max_children: int = 4) -> np.ndarray:
    """Parent of each of n draft tokens in topological order: token 0 is the
    root (parent -1); token t > 0 hangs under a random earlier token that has
    fewer than ``max_children`` children."""
    parent = np.full(n, -1, np.int64)
    kids = np.zeros(n, np.int64)
    for t in range(1, n):
        while True:
            p = int(rng.integers(0, t))
            if kids[p] < max_children:
                break
        parent[t] = p
        kids[p] += 1
    return parent


def tree_mask_bits(parents_per_request, qo_lens):
    """Pack per-request ancestor masks: bit t * n + u of request i's block is
    set iff draft token u is token t or one of its ancestors.  Returns (bits
    as uint8, little-endian within a byte; mask_indptr int32 [B+1] of bit
    offsets).  A request with qo_len <= 1 gets its qo_len^2 bits set."""
    blocks = []
    for par, n in zip(parents_per_request, qo_lens):
        n = int(n)
        m = np.zeros((n, n), bool)
        for t in range(n):
            u = t
            while u >= 0:
                m[t, u] = True
                u = int(par[u]) if par is not None else -1
        blocks.append(m.reshape(-1))
    flat = np.concatenate(blocks) if blocks else np.zeros(0, bool)
    indptr = np.zeros(len(blocks) + 1, np.int32)
    indptr[1:] = np.cumsum([b.size for b in blocks])
    return np.packbits(flat, bitorder="little"), indptr


def speculative_verify(seed: int = 1006, num_requests: int = 32, draft_lens=(16, 32, 64),
                       prefix_range=(512, 4096), page_size=16, nan_poison=False) -> PagedBatch:
    """Speculative-decoding verification step: each request checks a random
    draft token tree of 16, 32 or 64 tokens on top of a cached prefix
    (uniform in [512, 4096]); 32/8 heads, D = 128, bf16, page 16.  The draft
    tokens are the request's last keys; the tree mask lets each one see its
    ancestors."""
    rng = np.random.default_rng(seed)
    qo = rng.choice(np.asarray(draft_lens), size=num_requests).astype(np.int64)
    prefix = rng.integers(prefix_range[0], prefix_range[1], size=num_requests, endpoint=True)
    parents = [random_tree_parents(rng, int(n)) for n in qo]
    b = make_batch(seed, qo, prefix + qo, page_size=page_size, nan_poison=nan_poison,
                   name="speculative_verify")
    b.tree_mask, b.mask_indptr = tree_mask_bits(parents, qo)
    return b
