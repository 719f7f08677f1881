"""The seeded generators build the shapes and index arrays the workloads name."""
import numpy as np
import torch

import workloads as wl


def _consistent(b, shared_pages=False):
    P = b.page_size
    npg = np.diff(b.kv_indptr)
    assert np.array_equal(npg, -(-b.kv_lens // P))
    assert np.all(b.kv_last_page_len[npg > 0] >= 1) and np.all(b.kv_last_page_len <= P)
    kv = np.where(npg > 0, (npg - 1) * P + b.kv_last_page_len, 0)
    assert np.array_equal(kv, b.kv_lens)
    if not shared_pages:
        assert len(np.unique(b.kv_indices)) == len(b.kv_indices)  # no page shared in these views
    assert b.kv_indices.max(initial=-1) < b.pool_pages
    assert b.q.shape == (int(b.qo_lens.sum()), b.num_qo_heads, b.head_dim)
    assert b.kv_pool.shape == (b.pool_pages, 2, P, b.num_kv_heads, b.head_dim)


def test_tiny_decode_fp32_shapes():
    b = wl.tiny_decode_fp32()
    _consistent(b)
    assert list(b.kv_lens) == [17, 64, 100, 3]
    assert list(np.diff(b.kv_indptr)) == [2, 4, 7, 1]
    assert list(b.kv_last_page_len) == [1, 16, 4, 3]
    assert list(b.kv_indptr) == [0, 2, 6, 13, 14]
    assert b.kv_pool.shape == (32, 2, 16, 2, 64) and b.kv_pool.dtype == torch.float32
    assert b.sm_scale == 1.0 / 8.0 and b.qo_indptr is None


def test_generators_are_deterministic():
    a, b = wl.tiny_decode_fp32(), wl.tiny_decode_fp32()
    assert torch.equal(a.q, b.q) and torch.equal(a.kv_pool, b.kv_pool)
    assert np.array_equal(a.kv_indices, b.kv_indices)


def test_small_mixed_and_cascade_views():
    b = wl.make_batch(5, [1, 7, 0, 3], [9, 7, 5, 40], page_size=4, num_qo_heads=8,
                      num_kv_heads=2, head_dim=64, causal=True)
    _consistent(b)
    assert list(b.qo_indptr) == [0, 1, 8, 8, 11]
    cb = wl.shared_prefix_cascade(num_requests=6, prefix_len=64, suffix_lo=3, suffix_hi=20,
                                  seed=3, head_dim=64, num_qo_heads=8, num_kv_heads=2)
    for i in range(6):
        fl = cb.flat.kv_indices[cb.flat.kv_indptr[i]:cb.flat.kv_indptr[i + 1]]
        assert np.array_equal(fl[:4], cb.level0.kv_indices)
        assert np.array_equal(fl[4:], cb.level1.kv_indices[cb.level1.kv_indptr[i]:cb.level1.kv_indptr[i + 1]])
    assert np.array_equal(cb.flat.kv_lens, 64 + cb.suffix_lens)
    assert list(cb.level0.qo_indptr) == [0, 6] and not cb.level0.causal


def test_cascade_views_with_empty_suffix():
    cb = wl.shared_prefix_cascade(num_requests=20, prefix_len=32, suffix_lo=0, suffix_hi=2, seed=8,
                                  head_dim=64, num_qo_heads=4, num_kv_heads=2, page_size=16)
    assert (cb.suffix_lens == 0).any()
    _consistent(cb.flat, shared_pages=True)
    npg = np.diff(cb.flat.kv_indptr)
    kv = (npg - 1) * 16 + cb.flat.kv_last_page_len
    assert np.array_equal(kv, 32 + cb.suffix_lens)
