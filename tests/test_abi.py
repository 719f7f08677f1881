"""Host-side checks of the C-ABI library (no GPU needed).

- libfi.so loads and exports every function include/fi.h declares;
- fi_plan (C++) equals the plan oracle (pure Python) bit-exactly on every
  int32 word, over seeded random batches and the named workloads;
- error codes for invalid inputs, plan capacity, fi_plan_bounds.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_block_bsr_amd as fi
import workloads
from oracle import plan_ref as pr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Tests that hand the run calls made-up device addresses (16, 64, ...) to
# check that the host validation rejects a call before any launch.  Where a
# GPU is visible, a check that regressed would launch kernels on those
# addresses, so these run only where none is.
fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses: host-only test")


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fi_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = fi.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(fi.EXPORTS)
    assert fi.fi_version() >= 100


def test_default_workers():
    assert fi.fi_default_workers(fi.FI_KIND_DECODE, 256, 8) >= 1
    assert fi.fi_default_workers(fi.FI_KIND_PREFILL, 256, 8) >= 1
    assert fi.fi_default_workers(fi.FI_KIND_DECODE, 0, 8) == 1


def _compare(qo_indptr, kv_indptr, last, **kw):
    code, res = pr.plan(qo_indptr, kv_indptr, last, **kw)
    assert code == 0, res
    plan = fi.fi_plan(qo_indptr, kv_indptr, last, **kw)
    got = plan.buf[:plan.ints]
    assert plan.ints == len(res["buf"])
    assert np.array_equal(got, np.asarray(res["buf"], np.int32))
    d = fi.decode_plan_buffer(got)
    for name in ("decode", "prefill"):
        st = res[name]
        assert d[name]["rows"] == [tuple(r) for r in st["rows"]]
        assert d[name]["items"] == [tuple(r) for r in st["items"]]
        assert d[name]["wip"] == st["wip"]
        assert d[name]["merge_indptr"] == st["merge_indptr"]
        assert d[name]["split_rows"] == st["split_rows"]
        assert d[name]["item_meta"] == [tuple(m) for m in st["item_meta"]]
    assert plan.float_ws_bytes == 4 * res["ws_floats"]
    return plan, res


@pytest.mark.parametrize("seed", range(60))
def test_fi_plan_bit_exact_vs_oracle_random(seed):
    rng = np.random.default_rng(1000 + seed)
    P = int(rng.choice([1, 3, 16, 32]))
    causal = bool(rng.integers(0, 2))
    B = int(rng.integers(0, 20))
    qo = rng.integers(0, 70, size=B)
    kv = np.array([rng.integers(q if (causal and q >= 2) else 0, max(q, 600) + 1) for q in qo],
                  dtype=np.int64)
    npg = -(-kv // P)
    last = np.where(npg > 0, kv - (npg - 1) * P, 0).astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    Hk = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    decode_only = bool(rng.integers(0, 3) == 0)
    _compare(None if decode_only else qo_indptr, kv_indptr, last, page_size=P,
             num_qo_heads=Hk * G, num_kv_heads=Hk, head_dim=int(rng.choice([64, 128])),
             causal=causal, workers_decode=int(rng.integers(1, 40)),
             workers_prefill=int(rng.integers(1, 40)), min_seg_pages=int(rng.integers(1, 10)),
             br_override=int(rng.choice([0, 0, 16, 64])), no_split=int(rng.integers(0, 2)),
             window_left=int(rng.choice([-1, -1, 0, 3, 50, 400])))


@pytest.mark.parametrize("name", ["tiny_decode_fp32", "llama8b_decode", "skewed_long_decode",
                                  "mixed_ragged_step"])
def test_fi_plan_bit_exact_on_named_workloads(name, monkeypatch):
    # only the index arrays matter: build them without drawing the pools
    rng = np.random.default_rng(7)
    if name == "tiny_decode_fp32":
        kv, qo, P, Hq, Hk, D = np.array([17, 64, 100, 3]), None, 16, 8, 2, 64
    elif name == "llama8b_decode":
        kv, qo, P, Hq, Hk, D = rng.integers(512, 4097, 64), None, 16, 32, 8, 128
    elif name == "skewed_long_decode":
        kv = np.concatenate([[131072], np.clip(np.rint(np.exp(rng.normal(np.log(1024), 1, 31))), 128, 4096)]).astype(np.int64)
        qo, P, Hq, Hk, D = None, 16, 32, 8, 128
    else:
        qp = rng.choice([64, 128, 256, 512], 16)
        kv = np.concatenate([rng.integers(0, 2049, 16) + qp, rng.integers(256, 8193, 48)])
        qo = np.concatenate([[0], np.cumsum(np.concatenate([qp, np.ones(48, int)]))]).astype(np.int32)
        P, Hq, Hk, D = 16, 32, 8, 128
    npg = -(-kv // P)
    last = (kv - (npg - 1) * P).astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    for wd, wp in ((1, 1), (64, 32), (128, 64), (256, 128)):
        _compare(qo, kv_indptr, last, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=D,
                 causal=True, workers_decode=wd, workers_prefill=wp)


@pytest.mark.parametrize("bad,code", [
    (dict(page_size=0), fi.binding.FI_ERR_INVALID_ARG),
    (dict(num_qo_heads=6, num_kv_heads=4), fi.binding.FI_ERR_INVALID_ARG),
    (dict(head_dim=96), fi.binding.FI_ERR_UNSUPPORTED),
    (dict(num_qo_heads=48, num_kv_heads=3), fi.binding.FI_ERR_UNSUPPORTED),
    (dict(workers_decode=0), fi.binding.FI_ERR_INVALID_ARG),
    (dict(min_seg_pages=0), fi.binding.FI_ERR_INVALID_ARG),
    # a segment of more than 2^31 - 1 cost units (min_seg plus the fixed cost)
    (dict(min_seg_pages=2 ** 31 - 1), fi.binding.FI_ERR_INVALID_ARG),
    (dict(br_override=24), fi.binding.FI_ERR_INVALID_ARG),
    (dict(kv_last_page_len=[0, 3]), fi.binding.FI_ERR_INVALID_ARG),
    (dict(kv_last_page_len=[5, 3]), fi.binding.FI_ERR_INVALID_ARG),
    (dict(kv_indptr=[1, 2, 3]), fi.binding.FI_ERR_INVALID_ARG),
    (dict(kv_indptr=[0, 2, 1]), fi.binding.FI_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 9, 10]), fi.binding.FI_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 2, 1]), fi.binding.FI_ERR_INVALID_ARG),
    (dict(window_left=-2), fi.binding.FI_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 2, 3], kv_indptr=[0, 2 ** 28, 2 ** 28 + 1],
          kv_last_page_len=[4, 3], window_left=5), fi.binding.FI_ERR_UNSUPPORTED),
])
def test_fi_plan_error_codes_match_oracle(bad, code):
    kw = dict(qo_indptr=[0, 2, 3], kv_indptr=[0, 2, 3], kv_last_page_len=[4, 3], page_size=4,
              num_qo_heads=8, num_kv_heads=2, head_dim=64, causal=True, workers_decode=2,
              workers_prefill=2)
    kw.update(bad)
    args = (kw.pop("qo_indptr"), kw.pop("kv_indptr"), kw.pop("kv_last_page_len"))
    ocode, _ = pr.plan(*args, **kw)
    assert ocode == code
    with pytest.raises(fi.FIError) as e:
        fi.fi_plan(*args, **kw)
    assert e.value.code == code
    assert fi.fi_last_error()


def test_fi_plan_capacity_and_bounds():
    kv_indptr = [0, 3, 10]
    last = [5, 16]
    with pytest.raises(fi.FIError) as e:
        fi.fi_plan(None, kv_indptr, last, page_size=16, num_qo_heads=8, num_kv_heads=2,
                   head_dim=128, causal=True, workers_decode=4, capacity=10)
    assert e.value.code == fi.binding.FI_ERR_WORKSPACE_TOO_SMALL
    rng = np.random.default_rng(5)
    for _ in range(30):
        B = int(rng.integers(1, 12))
        qo = rng.integers(0, 300, B)
        kv = qo + rng.integers(0, 500, B)
        npg = -(-kv // 16)
        lastp = np.where(npg > 0, kv - (npg - 1) * 16, 0)
        kvi = np.concatenate([[0], np.cumsum(npg)])
        qoi = np.concatenate([[0], np.cumsum(qo)])
        wd, wp = int(rng.integers(1, 50)), int(rng.integers(1, 50))
        ints, ws = fi.fi_plan_bounds(B, int(qoi[-1]), 32, 8, 128, wd, wp)
        p = fi.fi_plan(qoi, kvi, lastp, page_size=16, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, causal=True, workers_decode=wd, workers_prefill=wp,
                       min_seg_pages=1, br_override=16)
        assert p.ints <= ints and p.float_ws_bytes <= ws


@fake_addresses
def test_run_calls_reject_bad_arguments_without_a_gpu():
    """Argument and plan checks happen on the host before any launch."""
    plan = fi.fi_plan(None, [0, 2], [3], page_size=16, num_qo_heads=8, num_kv_heads=2,
                      head_dim=128, causal=True, workers_decode=2)
    L = fi.lib()
    params = fi.make_params(__import__("torch").bfloat16, __import__("torch").bfloat16, 8, 2, 64, 16)
    rc = L.fi_batch_decode_paged(plan.host_ptr(), 16, ctypes.byref(params), 16, 16, 10, 16, 16, 16,
                                 16, None, 16, 1 << 20, None)
    assert rc == fi.binding.FI_ERR_PLAN_MISMATCH  # plan built for head_dim 128
    params = fi.make_params(__import__("torch").bfloat16, __import__("torch").bfloat16, 8, 2, 128, 16)
    rc = L.fi_batch_decode_paged(plan.host_ptr(), 16, ctypes.byref(params), 16, 16, 10, 16, 16, 16,
                                 16, None, 16, 0, None)
    assert rc == fi.binding.FI_ERR_WORKSPACE_TOO_SMALL  # checked before any launch
    bad = np.zeros(64, np.int32)
    rc = L.fi_batch_decode_paged(bad.ctypes.data, 16, ctypes.byref(params), 16, 16, 10, 16, 16, 16,
                                 16, None, 16, 1 << 20, None)
    assert rc == fi.binding.FI_ERR_PLAN_MISMATCH


@fake_addresses
def test_cascade_rejects_windowed_plans_without_a_gpu():
    torch = __import__("torch")
    kw = dict(page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128, workers_decode=2,
              workers_prefill=2, window_left=8)
    p0 = fi.fi_plan([0, 1], [0, 2], [3], causal=False, **kw)
    p1 = fi.fi_plan([0, 1], [0, 1], [5], causal=True, **kw)
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 16)
    rc = fi.lib().fi_cascade(p0.host_ptr(), 16, 16, 16, 16, 16, p1.host_ptr(), 16, 16, 16, 16, 16,
                             ctypes.byref(params), 16, 16, 10, 16, None, 16, 1 << 24, None)
    assert rc == fi.binding.FI_ERR_UNSUPPORTED and "window" in fi.fi_last_error()


@fake_addresses
def test_rope_arguments_are_checked_without_a_gpu():
    torch = __import__("torch")
    plan = fi.fi_plan(None, [0, 2], [3], page_size=16, num_qo_heads=8, num_kv_heads=2,
                      head_dim=128, causal=True, workers_decode=2)
    L = fi.lib()
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 16, rope_theta=float("inf"))
    rc = L.fi_batch_decode_paged(plan.host_ptr(), 16, ctypes.byref(params), 16, 16, 10, 16, 16, 16,
                                 16, None, 16, 1 << 20, None)
    assert rc == fi.binding.FI_ERR_INVALID_ARG and "rope" in fi.fi_last_error()
    kw = dict(page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128, workers_decode=2,
              workers_prefill=2)
    p0 = fi.fi_plan([0, 1], [0, 2], [3], causal=False, **kw)
    p1 = fi.fi_plan([0, 1], [0, 1], [5], causal=True, **kw)
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 16, rope_theta=10000.0)
    rc = L.fi_cascade(p0.host_ptr(), 16, 16, 16, 16, 16, p1.host_ptr(), 16, 16, 16, 16, 16,
                      ctypes.byref(params), 16, 16, 10, 16, None, 16, 1 << 24, None)
    assert rc == fi.binding.FI_ERR_UNSUPPORTED and "rotary" in fi.fi_last_error()


def test_append_rejects_bad_arguments():
    L = fi.lib()
    args = lambda dtype=fi.FI_BF16, n=5, hk=8, d=128: (None, None, dtype, None, 1, n, None, 1, 16, hk, d,
                                                        None, None, 1, None, None)
    assert L.fi_append_paged_kv(*args(dtype=7)) == -2            # dtype
    assert L.fi_append_paged_kv(*args(n=-1)) == -1               # negative size
    assert L.fi_append_paged_kv(*args(n=0)) == 0                 # nothing to write: no launch
    assert L.fi_append_paged_kv(*args()) == -1                   # null pointers with tokens
    assert L.fi_append_paged_kv(*args(hk=1, d=4)) == -2          # 8-byte rows
    assert "token row" in fi.fi_last_error()


@fake_addresses
def test_tree_mask_arguments_are_checked_without_a_gpu():
    """Tree-mask checks happen on the host before any launch: mask_indptr and
    a bit count in [1, 2^31), word alignment, no rotary embedding, a causal
    plan without a window, and no cascade."""
    torch = __import__("torch")
    L = fi.lib()
    kw = dict(page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128, workers_decode=2,
              workers_prefill=2)
    plan = fi.fi_plan([0, 3], [0, 2], [3], causal=True, **kw)

    def prefill(params, p=plan):
        return L.fi_batch_prefill_paged(p.host_ptr(), 16, ctypes.byref(params), 16, 16, 10, 16, 16,
                                        16, 16, 16, None, 16, 1 << 24, None)

    mk = lambda **k: fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 16, **k)
    assert prefill(mk(tree_mask=64, mask_indptr=None, mask_bits=9)) == fi.binding.FI_ERR_INVALID_ARG
    assert prefill(mk(tree_mask=64, mask_indptr=64, mask_bits=0)) == fi.binding.FI_ERR_INVALID_ARG
    assert prefill(mk(tree_mask=64, mask_indptr=64, mask_bits=1 << 31)) == fi.binding.FI_ERR_INVALID_ARG
    assert prefill(mk(tree_mask=66, mask_indptr=64, mask_bits=9)) == fi.binding.FI_ERR_INVALID_ARG
    assert "aligned" in fi.fi_last_error()
    assert prefill(mk(tree_mask=64, mask_indptr=64, mask_bits=9, rope_theta=1e4)) == fi.binding.FI_ERR_UNSUPPORTED
    nc = fi.fi_plan([0, 3], [0, 2], [3], causal=False, **kw)
    assert prefill(mk(tree_mask=64, mask_indptr=64, mask_bits=9), nc) == fi.binding.FI_ERR_UNSUPPORTED
    win = fi.fi_plan([0, 3], [0, 2], [3], causal=True, window_left=4, **kw)
    assert prefill(mk(tree_mask=64, mask_indptr=64, mask_bits=9), win) == fi.binding.FI_ERR_UNSUPPORTED
    p0 = fi.fi_plan([0, 1], [0, 2], [3], causal=False, **kw)
    p1 = fi.fi_plan([0, 1], [0, 1], [5], causal=True, **kw)
    rc = L.fi_cascade(p0.host_ptr(), 16, 16, 16, 16, 16, p1.host_ptr(), 16, 16, 16, 16, 16,
                      ctypes.byref(mk(tree_mask=64, mask_indptr=64, mask_bits=1)), 16, 16, 10, 16,
                      None, 16, 1 << 24, None)
    assert rc == fi.binding.FI_ERR_UNSUPPORTED and "tree" in fi.fi_last_error()


@fake_addresses
def test_run_calls_need_the_pool_and_page_table_when_the_plan_reads_pages():
    """A plan in which some row sees a KV page makes the kernels read
    kv_indices and the pool (and page 0, which stands in for an out-of-pool
    id): pool_pages < 1 or a null pool / page table is refused on the host."""
    torch = __import__("torch")
    L = fi.lib()
    plan = fi.fi_plan(None, [0, 2], [3], page_size=16, num_qo_heads=8, num_kv_heads=2,
                      head_dim=128, causal=True, workers_decode=2)
    assert plan.buf[53] == 1
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 16)
    big = 1 << 24

    def decode(pool, pool_pages, kv_indices):
        return L.fi_batch_decode_paged(plan.host_ptr(), 16, ctypes.byref(params), 16, pool, pool_pages,
                                       16, kv_indices, 16, 16, None, 16, big, None)

    for args in ((16, 0, 16), (None, 10, 16), (16, 10, None), (16, -1, 16)):
        assert decode(*args) == fi.binding.FI_ERR_INVALID_ARG, args
    assert "pool" in fi.fi_last_error()
    # the workspace (control region included) is always needed
    rc = L.fi_batch_decode_paged(plan.host_ptr(), 16, ctypes.byref(params), 16, 16, 10, 16, 16, 16, 16,
                                 None, None, 0, None)
    assert rc == fi.binding.FI_ERR_WORKSPACE_TOO_SMALL


@fake_addresses
def test_prefill_with_other_pages_refuses_pools_of_2_31_tokens_or_more():
    """Pages that are not a power of two >= 16 tokens: the prefill kernel
    addresses the pool in 32-bit token rows, so a pool of 2^31 tokens or more
    is refused on the host."""
    torch = __import__("torch")
    L = fi.lib()
    plan = fi.fi_plan([0, 4], [0, 2], [3], page_size=3, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                      causal=True, workers_decode=2, workers_prefill=2)
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 3)

    def prefill(pool_pages):
        return L.fi_batch_prefill_paged(plan.host_ptr(), 16, ctypes.byref(params), 16, 16, pool_pages, 16, 16,
                                        16, 16, 16, None, 16, plan.float_ws_bytes, None)

    assert prefill((1 << 31) // 3 + 1) == fi.binding.FI_ERR_UNSUPPORTED
    assert "2^31 tokens" in fi.fi_last_error()


@fake_addresses
def test_cascade_checks_both_levels_index_arrays():
    torch = __import__("torch")
    L = fi.lib()
    kw = dict(page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128, workers_decode=2,
              workers_prefill=2)
    p0 = fi.fi_plan([0, 3], [0, 2], [3], causal=False, **kw)
    p1 = fi.fi_plan([0, 2, 3], [0, 1, 2], [5, 4], causal=True, **kw)  # request 0 has 2 queries
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 8, 2, 128, 16)
    big = 1 << 26

    def cascade(l0, l1, pool_pages=10, pool=16):
        return L.fi_cascade(p0.host_ptr(), 16, *l0, p1.host_ptr(), 16, *l1, ctypes.byref(params), 16, pool,
                            pool_pages, 16, None, 16, big, None)

    good = (16, 16, 16, 16)
    for k in range(4):
        bad = list(good)
        bad[k] = None
        assert cascade(tuple(bad), good) == fi.binding.FI_ERR_INVALID_ARG, ("level 0", k)
        assert cascade(good, tuple(bad)) == fi.binding.FI_ERR_INVALID_ARG, ("level 1", k)
    assert cascade(good, good, pool_pages=0) == fi.binding.FI_ERR_INVALID_ARG
    assert cascade(good, good, pool=None) == fi.binding.FI_ERR_INVALID_ARG


def test_read_status_rejects_a_null_status_pointer():
    assert fi.lib().fi_read_status(16, None, 0, None) == fi.binding.FI_ERR_INVALID_ARG


def test_noalloc_decode_refuses_plans_larger_than_its_scratch_on_the_host():
    """The size check comes before any device call: 599 x 2 partial slots of
    32 heads x 128 dims do not fit the 16 MiB static scratch."""
    torch = __import__("torch")
    plan = fi.fi_plan(None, [0, 2, 5], [3, 9], page_size=16, num_qo_heads=32, num_kv_heads=8,
                      head_dim=128, causal=True, workers_decode=600, min_seg_pages=1)
    params = fi.make_params(torch.bfloat16, torch.bfloat16, 32, 8, 128, 16)
    rc = fi.lib().fi_batch_decode_paged_noalloc(plan.host_ptr(), None, ctypes.byref(params), None, None, 0,
                                                None, None, None, None, None, None)
    assert rc == fi.binding.FI_ERR_WORKSPACE_TOO_SMALL and "scratch" in fi.fi_last_error()
