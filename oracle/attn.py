"""ctypes front end of the fp64 C oracle (``attn_ref.c``).

TEST INFRASTRUCTURE ONLY.

Every function takes plain numpy arrays (index arrays int32, values float64)
and returns float64 results.  Values in other dtypes are upcast exactly
(fp32 and bf16 are subsets of fp64).
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from . import build as _build

_lock = threading.Lock()
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):
                _build.build()
            L = ctypes.CDLL(_build.LIB)
            L.oref_last_error.restype = ctypes.c_char_p
            L.oref_num_threads.restype = ctypes.c_int
            L.oref_set_num_threads.restype = None
            L.oref_set_num_threads.argtypes = [ctypes.c_int]
            L.oref_validate.restype = ctypes.c_int
            L.oref_validate.argtypes = [ctypes.c_int, _i32p, _i32p, _i32p, _i32p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64]
            L.oref_token_location.restype = ctypes.c_int
            L.oref_token_location.argtypes = [_i32p, _i32p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int64, _i32p, _i32p]
            L.oref_attention_rows.restype = ctypes.c_int
            L.oref_attention_rows.argtypes = [
                ctypes.c_int, _i32p, _i32p, _i32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                ctypes.c_double, ctypes.c_double, _u8p, _i32p, _f64p, _f64p, ctypes.c_int64,
                ctypes.c_int64, _i32p, _i32p, _i32p, _f64p, _f64p]
            L.oref_attention.restype = ctypes.c_int
            L.oref_attention.argtypes = [
                ctypes.c_int, _i32p, _i32p, _i32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                ctypes.c_double, ctypes.c_double, _u8p, _i32p, _f64p, _f64p, ctypes.c_int64,
                _f64p, _f64p]
            L.oref_merge_states.restype = ctypes.c_int
            L.oref_merge_states.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, _f64p,
                                            _f64p, _f64p, _f64p]
            _lib = L
    return _lib


class OracleError(ValueError):
    pass


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(lib().oref_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later calls."""
    lib().oref_set_num_threads(int(n))


def _i32(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


def _f64(a):
    if hasattr(a, "detach"):  # a torch tensor: upcast exactly on the CPU
        a = a.detach().to("cpu").double().numpy()
    a = np.ascontiguousarray(np.asarray(a), dtype=np.float64)
    return a, a.ctypes.data_as(_f64p)


def _check(rc):
    if rc != 0:
        raise OracleError(lib().oref_last_error().decode())


def validate(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size, num_qo_heads,
             num_kv_heads, head_dim, causal, pool_pages):
    B = len(kv_indptr) - 1
    qo, qo_p = _i32(qo_indptr)
    kp, kp_p = _i32(kv_indptr)
    ki, ki_p = _i32(kv_indices if len(kv_indices) else np.zeros(1, np.int32))
    kl, kl_p = _i32(kv_last_page_len if len(kv_last_page_len) else np.zeros(1, np.int32))
    _check(lib().oref_validate(B, qo_p, kp_p, ki_p, kl_p, page_size, num_qo_heads, num_kv_heads,
                               head_dim, int(causal), int(pool_pages)))


def _mask(tree_mask, mask_indptr):
    """ctypes views of the optional tree mask (NULL pointers when absent)."""
    if tree_mask is None:
        return None, ctypes.cast(None, _u8p), None, ctypes.cast(None, _i32p)
    tm = np.ascontiguousarray(np.asarray(tree_mask, dtype=np.uint8).reshape(-1))
    if tm.size == 0:
        tm = np.zeros(1, np.uint8)
    mi = np.ascontiguousarray(np.asarray(mask_indptr, dtype=np.int32))
    return tm, tm.ctypes.data_as(_u8p), mi, mi.ctypes.data_as(_i32p)


def token_location(kv_indptr, kv_indices, page_size, request, token):
    """(page id, slot) of logical token ``token`` of request ``request``."""
    kp, kp_p = _i32(kv_indptr)
    ki, ki_p = _i32(kv_indices)
    page = ctypes.c_int32()
    slot = ctypes.c_int32()
    _check(lib().oref_token_location(kp_p, ki_p, page_size, request, token, ctypes.byref(page),
                                     ctypes.byref(slot)))
    return page.value, slot.value


def attention(q, kv_pool, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, *, page_size,
              num_qo_heads, num_kv_heads, head_dim, causal, sm_scale, soft_cap=0.0,
              window_left=-1, rope_theta=0.0, rope_scale=1.0, tree_mask=None, mask_indptr=None):
    """Exact attention for every query row.

    q: [total_qo, Hq, D]; kv_pool: [pages, 2, P, Hk, D]; qo_indptr None means
    one query per request.  Returns (o [total_qo, Hq, D], lse [total_qo, Hq]),
    float64, lse in natural log (-inf where no key is visible).  window_left
    >= 0: the query at position kv_len - qo_len + t sees no key more than
    window_left positions before it.  rope_theta > 0: rotary embedding of q
    (at position kv_len - qo_len + t) and k (at position j), rotate-half form
    with angle pos / rope_scale * rope_theta^(-2d/D).  tree_mask (uint8
    bits, little-endian within a byte) with mask_indptr (bit offset of each
    request's qo_len x qo_len block): draft token t sees draft token u <= t
    iff bit t * qo_len + u is set (always itself), and every key before the
    draft.
    """
    B = len(kv_indptr) - 1
    tm, tm_p, mi, mi_p = _mask(tree_mask, mask_indptr)
    qa, q_p = _f64(q)
    pa, p_p = _f64(kv_pool)
    qo, qo_p = _i32(qo_indptr)
    kp, kp_p = _i32(kv_indptr)
    ki, ki_p = _i32(kv_indices if len(kv_indices) else np.zeros(1, np.int32))
    kl, kl_p = _i32(kv_last_page_len if len(kv_last_page_len) else np.zeros(1, np.int32))
    total = qa.shape[0]
    o = np.zeros((total, num_qo_heads, head_dim), np.float64)
    lse = np.zeros((total, num_qo_heads), np.float64)
    _check(lib().oref_attention(B, qo_p, kp_p, ki_p, kl_p, page_size, num_qo_heads, num_kv_heads,
                                head_dim, int(causal), float(sm_scale), float(soft_cap),
                                int(window_left), float(rope_theta), float(rope_scale), tm_p, mi_p,
                                q_p, p_p, int(pa.shape[0]), o.ctypes.data_as(_f64p),
                                lse.ctypes.data_as(_f64p)))
    return o, lse


def attention_rows(q, kv_pool, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, rows, *,
                   page_size, num_qo_heads, num_kv_heads, head_dim, causal, sm_scale,
                   soft_cap=0.0, window_left=-1, rope_theta=0.0, rope_scale=1.0, tree_mask=None,
                   mask_indptr=None):
    """Exact attention for selected rows.  ``rows`` is an int array [n, 3] of
    (request, token-in-request, query head).  Returns (o [n, D], lse [n])."""
    B = len(kv_indptr) - 1
    tm, tm_p, mi, mi_p = _mask(tree_mask, mask_indptr)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    rq, rq_p = _i32(rows[:, 0].copy())
    rt, rt_p = _i32(rows[:, 1].copy())
    rh, rh_p = _i32(rows[:, 2].copy())
    qa, q_p = _f64(q)
    pa, p_p = _f64(kv_pool)
    qo, qo_p = _i32(qo_indptr)
    kp, kp_p = _i32(kv_indptr)
    ki, ki_p = _i32(kv_indices if len(kv_indices) else np.zeros(1, np.int32))
    kl, kl_p = _i32(kv_last_page_len if len(kv_last_page_len) else np.zeros(1, np.int32))
    n = rows.shape[0]
    o = np.zeros((n, head_dim), np.float64)
    lse = np.zeros((n,), np.float64)
    _check(lib().oref_attention_rows(B, qo_p, kp_p, ki_p, kl_p, page_size, num_qo_heads,
                                     num_kv_heads, head_dim, int(causal), float(sm_scale),
                                     float(soft_cap), int(window_left), float(rope_theta),
                                     float(rope_scale), tm_p, mi_p, q_p, p_p, int(pa.shape[0]), n,
                                     rq_p, rt_p,
                                     rh_p, o.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p)))
    return o, lse


def merge_states(o_parts, lse_parts):
    """n-way log-sum-exp merge.  o_parts [k, ..., D], lse_parts [k, ...]."""
    oa, o_p = _f64(o_parts)
    la, l_p = _f64(lse_parts)
    k = oa.shape[0]
    D = oa.shape[-1]
    lead = la.shape[1:]
    n = int(np.prod(lead)) if len(lead) else 1
    assert oa.shape[1:-1] == lead
    o = np.zeros(lead + (D,), np.float64)
    lse = np.zeros(lead, np.float64)
    _check(lib().oref_merge_states(k, n, D, o_p, l_p, o.ctypes.data_as(_f64p),
                                   lse.ctypes.data_as(_f64p)))
    return o, lse


def attention_of(batch, **overrides):
    """``attention`` on any object carrying the batch fields (q, kv_pool,
    qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size,
    num_qo_heads, num_kv_heads, head_dim, causal, sm_scale, soft_cap)."""
    kw = dict(page_size=batch.page_size, num_qo_heads=batch.num_qo_heads,
              num_kv_heads=batch.num_kv_heads, head_dim=batch.head_dim, causal=batch.causal,
              sm_scale=batch.sm_scale, soft_cap=batch.soft_cap,
              window_left=getattr(batch, "window_left", -1),
              rope_theta=getattr(batch, "rope_theta", 0.0), rope_scale=getattr(batch, "rope_scale", 1.0),
              tree_mask=getattr(batch, "tree_mask", None), mask_indptr=getattr(batch, "mask_indptr", None))
    kw.update(overrides)
    return attention(batch.q, batch.kv_pool, batch.qo_indptr, batch.kv_indptr, batch.kv_indices,
                     batch.kv_last_page_len, **kw)


def attention_rows_of(batch, rows, **overrides):
    kw = dict(page_size=batch.page_size, num_qo_heads=batch.num_qo_heads,
              num_kv_heads=batch.num_kv_heads, head_dim=batch.head_dim, causal=batch.causal,
              sm_scale=batch.sm_scale, soft_cap=batch.soft_cap,
              window_left=getattr(batch, "window_left", -1),
              rope_theta=getattr(batch, "rope_theta", 0.0), rope_scale=getattr(batch, "rope_scale", 1.0),
              tree_mask=getattr(batch, "tree_mask", None), mask_indptr=getattr(batch, "mask_indptr", None))
    kw.update(overrides)
    return attention_rows(batch.q, batch.kv_pool, batch.qo_indptr, batch.kv_indptr,
                          batch.kv_indices, batch.kv_last_page_len, rows, **kw)


def cascade_of(level0, level1, level0_rows_of_query):
    """Two-level (shared prefix, then per-request suffix) attention.

    Level 0 attends the stacked queries of a group to the shared pages, level
    1 attends each request's query to its own pages, and the two states are
    merged by log-sum-exp composition (cascade code block of the
    serving-engine page; composable formats paragraph).
    ``level0_rows_of_query[k]`` is the level-0 query row holding level-1
    query ``k`` (identity when the group stacks the queries in order).
    """
    o0, l0 = attention_of(level0)
    o1, l1 = attention_of(level1)
    sel = np.asarray(level0_rows_of_query)
    return merge_states(np.stack([o0[sel], o1]), np.stack([l0[sel], l1]))
