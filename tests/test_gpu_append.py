"""GPU parity of the paged KV append (fi_append_paged_kv) against the numpy
oracle (oracle/append_ref.py): the whole pool after the append must be
bit-exactly the oracle's, through the C ABI."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import append_ref as ap

from gpu_util import note

pytestmark = pytest.mark.gpu


def _indptr(counts):
    out = np.zeros(len(counts) + 1, np.int32)
    out[1:] = np.cumsum(counts)
    return out


def _case(rng, P, Hk, D, dtype, kv_lens, new, pool_extra=5, bad_pages=()):
    counts = [(int(L) + P - 1) // P for L in kv_lens]
    pool_pages = sum(counts) + pool_extra
    kv_indices = rng.permutation(pool_pages)[: sum(counts)].astype(np.int32)
    for e, page in bad_pages:
        kv_indices[e] = page
    kv_indptr = _indptr(counts)
    last = np.array([int(L) - (c - 1) * P if c else 0 for L, c in zip(kv_lens, counts)], np.int32)
    n = int(sum(new))
    pool = torch.from_numpy(rng.standard_normal((pool_pages, 2, P, Hk, D), dtype=np.float32)).to(dtype)
    k = torch.from_numpy(rng.standard_normal((n, Hk, D), dtype=np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((n, Hk, D), dtype=np.float32)).to(dtype)
    return pool, k, v, _indptr(new), kv_indptr, kv_indices, last


def _check(pool, k, v, append_indptr, kv_indptr, kv_indices, last, what):
    P = pool.shape[2]
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    pool_d = pool.cuda()
    note(f"append {what}: {k.shape[0]} tokens into {pool.shape[0]} pages, P={P}, {pool.dtype}")
    fi.fi_append_paged_kv(k.cuda(), v.cuda(), i32(append_indptr), pool_d, i32(kv_indptr), i32(kv_indices),
                          i32(last))
    torch.cuda.synchronize()
    # the oracle on the raw bits: rows are moved, never converted
    as_bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()
    want = ap.append(as_bits(pool), as_bits(k), as_bits(v), append_indptr, kv_indptr, kv_indices, last, P)
    got = as_bits(pool_d.cpu())
    assert np.array_equal(got, want), f"append {what}: pool differs from the oracle"


SWEEP = [(dt, D, Hk, P) for dt in (torch.bfloat16, torch.float32) for D in (64, 128) for Hk in (1, 8)
         for P in (1, 3, 16)]


@pytest.mark.parametrize("dtype,D,Hk,P", SWEEP)
def test_append_sweep(dtype, D, Hk, P):
    rng = np.random.default_rng(8100 + D + 7 * Hk + 3 * P + (dtype == torch.float32))
    kv_lens = [1, 17, 0, 2 * P, 50, 3 * P + 1, 9]
    new = [1, 5, 0, 2 * P, 50, P + 2, 1]        # single tokens, page-crossing runs, whole requests
    _check(*_case(rng, P, Hk, D, dtype, kv_lens, new), f"sweep D={D} Hk={Hk} P={P}")


def test_append_contract_for_tokens_without_a_place():
    """Library contract (the pages define no such input): a new token that
    the request does not hold, or whose page id lies outside the pool, is not
    written and nothing else changes.  Expected pool: the oracle on the same
    batch made placeable -- request 0 keeps only the new tokens it holds (the
    last 5 of 9, whose positions do not change), and the two bad page-table
    entries name a scratch page added past the pool, dropped afterwards."""
    rng = np.random.default_rng(8201)
    P = 16
    kv_lens = [5, 40, 33]
    new = [9, 3, 4]                          # request 0: 9 new tokens but only 5 held
    pool, k, v, a_ip, kv_ip, kv_idx, last = _case(rng, P, 2, 64, torch.bfloat16, kv_lens, new,
                                                  bad_pages=[(3, 10 ** 6), (5, -7)])
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    pool_d = pool.cuda()
    note("append contract: 4 tokens past the request's start, 2 out-of-pool page ids")
    fi.fi_append_paged_kv(k.cuda(), v.cuda(), i32(a_ip), pool_d, i32(kv_ip), i32(kv_idx), i32(last))
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).numpy()
    n_pages = pool.shape[0]
    ext = np.concatenate([bits(pool), np.zeros((1,) + tuple(pool.shape[1:]), np.int16)])
    idx = kv_idx.copy()
    idx[3] = idx[5] = n_pages                # the scratch page
    keep = np.r_[4:int(a_ip[-1])]            # drop request 0's first 4 new tokens
    want = ap.append(ext, bits(k)[keep], bits(v)[keep], a_ip - np.array([0, 4, 4, 4], np.int32),
                     kv_ip, idx, last, P)[:n_pages]
    assert np.array_equal(bits(pool_d.cpu()), want), "append contract: pool differs"


def test_append_mixed_step_new_tokens_full_size():
    b = wl.mixed_ragged_step()
    rng = np.random.default_rng(8301)
    n = int(b.qo_lens.sum())
    Hk, D = b.num_kv_heads, b.head_dim
    k = torch.from_numpy(rng.standard_normal((n, Hk, D), dtype=np.float32)).to(b.dtype)
    v = torch.from_numpy(rng.standard_normal((n, Hk, D), dtype=np.float32)).to(b.dtype)
    _check(b.kv_pool, k, v, _indptr(b.qo_lens), b.kv_indptr, b.kv_indices, b.kv_last_page_len,
           "mixed_ragged_step new tokens")


def test_append_long_run_uses_the_grid_stride():
    rng = np.random.default_rng(8401)
    kv_lens = [40000, 3]
    new = [40000, 2]                          # more tokens than one pass of the grid covers
    _check(*_case(rng, 16, 2, 64, torch.bfloat16, kv_lens, new), "40002 tokens")
