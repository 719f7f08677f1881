"""Helpers of the GPU parity tests: run a batch through the C ABI and compare
with the fp64 oracle.  Tolerances: |o - o_ref| <= 2e-3 + 2e-2 |o_ref| per
element, |lse - lse_ref| <= 1e-3, and rows without visible keys must give
exactly o = 0, lse = -inf."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_block_bsr_amd as fi

ATOL, RTOL, LSE_ATOL = 2e-3, 2e-2, 1e-3
NUM_CUS = 256


def note(msg: str):
    """Name the case on stdout before a GPU step, flushed."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _dev_i32(a):
    a = np.asarray(a, dtype=np.int32)
    if a.size == 0:
        a = np.zeros(1, np.int32)
    return torch.from_numpy(a.copy()).cuda()


class DeviceBatch:
    def __init__(self, b):
        self.b = b
        self.q = b.q.cuda()
        self.pool = b.kv_pool.cuda()
        self.qo_indptr = None if b.qo_indptr is None else _dev_i32(b.qo_indptr)
        self.kv_indptr = _dev_i32(b.kv_indptr)
        self.kv_indices = _dev_i32(b.kv_indices)
        self.last = _dev_i32(b.kv_last_page_len)
        self.mask = self.mask_indptr = None
        self.mask_bits = 0
        if getattr(b, "tree_mask", None) is not None:
            self.mask = torch.from_numpy(fi.tree_mask_words(b.tree_mask)).cuda()
            self.mask_indptr = _dev_i32(b.mask_indptr)
            self.mask_bits = int(b.mask_indptr[-1])


def plan_for(b, workers_decode, workers_prefill=1, min_seg_pages=8, no_split=0, br_override=0,
             decode_only=None):
    qo = None if (decode_only or (decode_only is None and b.qo_indptr is None)) else b.qo_indptr
    return fi.fi_plan(qo, b.kv_indptr, b.kv_last_page_len, page_size=b.page_size,
                      num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                      head_dim=b.head_dim, causal=b.causal, workers_decode=workers_decode,
                      workers_prefill=workers_prefill, min_seg_pages=min_seg_pages,
                      br_override=br_override, no_split=no_split,
                      window_left=getattr(b, "window_left", -1))


def run(b, workers_decode=None, workers_prefill=None, min_seg_pages=8, no_split=0,
        out_dtype=None, br_override=0, dev=None, with_lse=True, ws=None):
    """Run decode (qo_indptr None) or prefill; returns (o float32 cpu, lse cpu).
    ``ws``: a workspace to use (else a fresh zero-filled one)."""
    Hk = b.num_kv_heads
    wd = workers_decode or fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk)
    wp = workers_prefill or fi.fi_default_workers(fi.FI_KIND_PREFILL, NUM_CUS, Hk)
    plan = plan_for(b, wd, wp, min_seg_pages, no_split, br_override)
    d = dev or DeviceBatch(b)
    plan_dev = plan.to_device()
    out_dtype = out_dtype or b.dtype
    o = torch.full(tuple(b.q.shape), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(tuple(b.q.shape[:2]), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    if ws is None:
        ws = fi.workspace(plan.float_ws_bytes)
    params = fi.make_params(b.dtype, out_dtype, b.num_qo_heads, Hk, b.head_dim, b.page_size,
                            b.sm_scale, b.soft_cap, tree_mask=d.mask, mask_indptr=d.mask_indptr,
                            mask_bits=d.mask_bits)
    if b.qo_indptr is None:
        fi.fi_batch_decode_paged(plan, plan_dev, params, d.q, d.pool, d.kv_indptr, d.kv_indices,
                                 d.last, o, lse, ws)
    else:
        fi.fi_batch_prefill_paged(plan, plan_dev, params, d.q, d.pool, d.qo_indptr, d.kv_indptr,
                                  d.kv_indices, d.last, o, lse, ws)
    torch.cuda.synchronize()
    return o.float().cpu(), (lse.cpu() if with_lse else None), plan


def assert_close(o, lse, o_ref, lse_ref, what="", atol=ATOL, rtol=RTOL, lse_atol=LSE_ATOL):
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    empty = ~np.isfinite(lse_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    bound = atol + rtol * np.abs(o_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs outside tolerance; "
                             f"max err {err.max():.3e}; first {idx.tolist()}")
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf lse rows differ"
        if (~empty).any():
            lerr = np.abs(lse[~empty] - lse_ref[~empty]).max()
            assert lerr <= lse_atol, f"{what}: lse err {lerr:.3e}"
        if empty.any():
            assert np.all(o[empty] == 0.0), f"{what}: empty rows must have o = 0"
    return float(err.max()) if err.size else 0.0


def run_cascade(cb, workers_decode=None, workers_prefill=None, min_seg_pages=8, out_dtype=None):
    """fi_cascade over a CascadeBatch: level 0 (groups over the shared pages,
    non-causal) merged with level 1 (each request's own pages)."""
    l0, l1 = cb.level0, cb.level1
    Hk = l0.num_kv_heads
    wd = workers_decode or fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk)
    wp = workers_prefill or fi.fi_default_workers(fi.FI_KIND_PREFILL, NUM_CUS, Hk)
    kw = dict(page_size=l0.page_size, num_qo_heads=l0.num_qo_heads, num_kv_heads=Hk,
              head_dim=l0.head_dim, workers_decode=wd, workers_prefill=wp,
              min_seg_pages=min_seg_pages)
    plan0 = fi.fi_plan(l0.qo_indptr, l0.kv_indptr, l0.kv_last_page_len, causal=False, **kw)
    plan1 = fi.fi_plan(l1.qo_indptr, l1.kv_indptr, l1.kv_last_page_len, causal=l1.causal, **kw)
    d0, d1 = DeviceBatch(l0), DeviceBatch(l1)
    d1.q, d1.pool = d0.q, d0.pool  # one query tensor and one pool: only the index arrays differ
    out_dtype = out_dtype or l0.dtype
    o = torch.full(tuple(l0.q.shape), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(tuple(l0.q.shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = fi.fi_cascade_workspace_bytes(plan0, plan1)
    ws = fi.workspace(nbytes)
    params = fi.make_params(l0.dtype, out_dtype, l0.num_qo_heads, Hk, l0.head_dim, l0.page_size,
                            l0.sm_scale, l0.soft_cap)
    fi.fi_cascade(plan0, plan0.to_device(), d0.qo_indptr, d0.kv_indptr, d0.kv_indices, d0.last,
                  plan1, plan1.to_device(), d1.qo_indptr, d1.kv_indptr, d1.kv_indices, d1.last,
                  params, d0.q, d0.pool, o, lse, ws)
    torch.cuda.synchronize()
    return o.float().cpu(), lse.cpu()
