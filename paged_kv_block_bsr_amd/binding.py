"""ctypes binding of ``libfi.so``: the C ABI of ``include/fi.h`` under the same
names, with torch tensors marshalled to raw pointers.

Argument marshalling only: every step of the attention path (plan, page
gather, softmax, merge) runs inside the library.  PyTorch supplies device
memory (``data_ptr()``) and the current HIP stream.  If the library is missing
every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfi.so")

FI_OK = 0
FI_ERR_INVALID_ARG = -1
FI_ERR_UNSUPPORTED = -2
FI_ERR_WORKSPACE_TOO_SMALL = -3
FI_ERR_PLAN_MISMATCH = -4
FI_ERR_HIP = -5

FI_F32 = 0
FI_BF16 = 1
FI_KIND_DECODE = 0
FI_KIND_PREFILL = 1

# plan buffer layout (see csrc/plan_format.h)
H_MAGIC, H_SIZE, H_BATCH, H_TOTAL_QO, H_CAUSAL, H_WS_FLOATS = 0, 2, 3, 4, 9, 11
H_STREAM0, H_STREAM1 = 12, 32
(S_W, S_SEG, S_TILE, S_NROWS, S_NITEMS, S_NSLOTS, S_NSPLIT, S_SLOTCAP, S_OFF_ROWS, S_OFF_ITEMS,
 S_OFF_WIP, S_OFF_MERGE, S_OFF_SPLIT, S_WS_O, S_WS_LSE, S_KIND, S_OFF_META, S_OFF_SREC) = range(18)

EXPORTS = ["fi_plan", "fi_plan_bounds", "fi_batch_decode_paged", "fi_batch_prefill_paged",
           "fi_merge_state", "fi_cascade", "fi_cascade_workspace_bytes", "fi_append_paged_kv",
           "fi_read_status", "fi_last_error", "fi_version", "fi_default_workers",
           "fi_batch_decode_paged_noalloc"]

# status word bits (fi_read_status)
FI_STATUS_BAD_PAGE = 1


class FIError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class fi_plan_in(ctypes.Structure):
    _fields_ = [("batch_size", ctypes.c_int32),
                ("qo_indptr", ctypes.c_void_p),         # const int32_t*
                ("kv_indptr", ctypes.c_void_p),         # const int32_t*
                ("kv_last_page_len", ctypes.c_void_p),  # const int32_t*
                ("page_size", ctypes.c_int32),
                ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("causal", ctypes.c_int32),
                ("workers_decode", ctypes.c_int32),
                ("workers_prefill", ctypes.c_int32),
                ("min_seg_pages", ctypes.c_int32),
                ("br_override", ctypes.c_int32),
                ("no_split", ctypes.c_int32),
                ("window_left", ctypes.c_int32)]


class fi_plan_info(ctypes.Structure):
    _fields_ = [("plan_ints", ctypes.c_int64),
                ("float_ws_bytes", ctypes.c_int64),
                ("decode_rows", ctypes.c_int32), ("decode_items", ctypes.c_int32),
                ("decode_slots", ctypes.c_int32), ("decode_segment_pages", ctypes.c_int32),
                ("prefill_rows", ctypes.c_int32), ("prefill_items", ctypes.c_int32),
                ("prefill_slots", ctypes.c_int32), ("prefill_segment_pages", ctypes.c_int32),
                ("prefill_tile_rows", ctypes.c_int32)]


class fi_attn_params(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int),
                ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32),
                ("sm_scale", ctypes.c_float),
                ("logits_soft_cap", ctypes.c_float),
                ("graph_safe", ctypes.c_int32),
                ("rope_theta", ctypes.c_float),
                ("rope_scale", ctypes.c_float),
                ("tree_mask", ctypes.c_void_p),
                ("mask_indptr", ctypes.c_void_p),
                ("mask_bits", ctypes.c_int64)]


_lib = None


def lib():
    """Load libfi.so (built in-tree by ``paged_kv_block_bsr_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FIError(FI_ERR_HIP, f"{LIB_PATH} is not built; run paged_kv_block_bsr_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        L.fi_plan.argtypes = [ctypes.POINTER(fi_plan_in), vp, ctypes.c_int64,
                              ctypes.POINTER(fi_plan_info)]
        L.fi_plan_bounds.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i64p, i64p]
        L.fi_batch_decode_paged.argtypes = [vp, vp, ctypes.POINTER(fi_attn_params), vp, vp,
                                            ctypes.c_int64, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp]
        L.fi_batch_prefill_paged.argtypes = [vp, vp, ctypes.POINTER(fi_attn_params), vp, vp,
                                             ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_int64, vp]
        L.fi_merge_state.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int, vp]
        L.fi_cascade.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.POINTER(fi_attn_params), vp, vp, ctypes.c_int64, vp, vp, vp,
                                 ctypes.c_int64, vp]
        L.fi_cascade_workspace_bytes.argtypes = [vp, vp]
        L.fi_append_paged_kv.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int32, ctypes.c_int64, vp,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         vp, vp, ctypes.c_int64, vp, vp]
        L.fi_read_status.argtypes = [vp, i32p, ctypes.c_int32, vp]
        L.fi_batch_decode_paged_noalloc.argtypes = [vp, vp, ctypes.POINTER(fi_attn_params), vp, vp,
                                                    ctypes.c_int64, vp, vp, vp, vp, vp, vp]
        L.fi_cascade_workspace_bytes.restype = ctypes.c_int64
        L.fi_last_error.restype = ctypes.c_char_p
        L.fi_default_workers.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        for name in EXPORTS:
            if name not in ("fi_cascade_workspace_bytes", "fi_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != FI_OK:
        raise FIError(rc, lib().fi_last_error().decode())


def _i32_host(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if type(a) is np.ndarray and a.dtype == np.int32 and a.flags.c_contiguous:
        return a
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return FI_F32
    if dt == torch.bfloat16:
        return FI_BF16
    raise FIError(FI_ERR_UNSUPPORTED, f"dtype {dt}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Plan:
    """A host plan buffer (int32) with its summary."""

    buf: np.ndarray
    info: fi_plan_info

    @property
    def ints(self) -> int:
        return int(self.info.plan_ints)

    @property
    def float_ws_bytes(self) -> int:
        return int(self.info.float_ws_bytes)

    def host_ptr(self) -> int:
        return self.buf.ctypes.data

    def to_device(self, device="cuda", out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Copy the plan to device memory (``out`` if given, else a new tensor)."""
        src = torch.from_numpy(self.buf[: self.ints])
        if out is None:
            return src.to(device)
        out[: self.ints].copy_(src, non_blocking=False)
        return out


def fi_plan(qo_indptr, kv_indptr, kv_last_page_len, *, page_size, num_qo_heads, num_kv_heads,
            head_dim, causal, workers_decode, workers_prefill=1, min_seg_pages=8,
            br_override=0, no_split=0, window_left=-1, capacity: Optional[int] = None,
            out: Optional[np.ndarray] = None) -> Plan:
    """Build a plan on the host from host index arrays (``fi_plan``).
    ``window_left`` >= 0: sliding-window attention (-1: none)."""
    kp = _i32_host(kv_indptr)
    kl = _i32_host(kv_last_page_len)
    qo = _i32_host(qo_indptr)
    B = len(kp) - 1
    if kl is None or len(kl) == 0:
        kl = np.zeros(max(B, 1), np.int32)
    total_qo = B if qo is None else int(qo[-1])
    if capacity is None and out is not None:
        capacity = len(out)  # fi_plan itself rejects a buffer that is too small
    if capacity is None:
        ints = ctypes.c_int64()
        _check(lib().fi_plan_bounds(B, total_qo, num_qo_heads, num_kv_heads, head_dim,
                                    max(1, workers_decode), max(1, workers_prefill),
                                    ctypes.byref(ints), None))
        capacity = int(ints.value)
    buf = out if out is not None else np.zeros(capacity, np.int32)
    pin = fi_plan_in(B, qo.ctypes.data if qo is not None else None, kp.ctypes.data, kl.ctypes.data,
                     page_size, num_qo_heads, num_kv_heads, head_dim, int(bool(causal)),
                     workers_decode, workers_prefill, min_seg_pages, br_override, no_split,
                     window_left)
    info = fi_plan_info()
    _check(lib().fi_plan(ctypes.byref(pin), buf.ctypes.data, len(buf), ctypes.byref(info)))
    return Plan(buf=buf, info=info)


def fi_plan_bounds(batch_size, total_qo, num_qo_heads, num_kv_heads, head_dim, workers_decode,
                   workers_prefill):
    ints, ws = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().fi_plan_bounds(batch_size, total_qo, num_qo_heads, num_kv_heads, head_dim,
                                workers_decode, workers_prefill, ctypes.byref(ints),
                                ctypes.byref(ws)))
    return int(ints.value), int(ws.value)


def make_params(q_dtype, out_dtype, num_qo_heads, num_kv_heads, head_dim, page_size, sm_scale=0.0,
                logits_soft_cap=0.0, graph_safe=False, rope_theta=0.0, rope_scale=1.0,
                tree_mask=None, mask_indptr=None, mask_bits=0) -> fi_attn_params:
    """``graph_safe``: launch every kernel of a call whatever the plan, so a
    call captured into a graph stays valid for later plans of the same shapes.
    ``rope_theta`` > 0: fused rotary embedding of q and k (``rope_scale``
    divides the positions).  ``tree_mask`` (device int32 / uint32 words of
    the bit stream, see :func:`tree_mask_words`), ``mask_indptr`` (device
    int32) and ``mask_bits``: the speculative-decoding tree mask of a prefill
    call.  The params hold raw device addresses: keep those tensors alive
    while the params are used."""
    return fi_attn_params(_dtype_code(q_dtype), _dtype_code(out_dtype), num_qo_heads,
                          num_kv_heads, head_dim, page_size, float(sm_scale),
                          float(logits_soft_cap), int(bool(graph_safe)), float(rope_theta),
                          float(rope_scale), _ptr(tree_mask) if tree_mask is not None else None,
                          _ptr(mask_indptr) if mask_indptr is not None else None, int(mask_bits))


def tree_mask_words(bits_u8) -> np.ndarray:
    """A little-endian byte stream of mask bits as int32 words (padded with
    zero bytes to whole words), the layout the tree-mask parameter takes."""
    b = np.asarray(bits_u8, dtype=np.uint8).reshape(-1)
    pad = (-b.size) % 4
    if pad or b.size == 0:
        b = np.concatenate([b, np.zeros(pad if b.size else 4, np.uint8)])
    return b.view(np.int32).copy()


def fi_batch_decode_paged(plan: Plan, plan_dev, params: fi_attn_params, q, kv_pool,
                          kv_indptr, kv_indices, kv_last_page_len, o, lse, float_ws,
                          stream=None):
    _check(lib().fi_batch_decode_paged(
        plan.host_ptr(), _ptr(plan_dev), ctypes.byref(params), _ptr(q), _ptr(kv_pool),
        kv_pool.shape[0], _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(o),
        _ptr(lse), _ptr(float_ws), float_ws.numel() * float_ws.element_size(), _stream(stream)))


def fi_batch_decode_paged_noalloc(plan: Plan, plan_dev, params: fi_attn_params, q, kv_pool,
                                  kv_indptr, kv_indices, kv_last_page_len, o, lse, stream=None):
    """Batch decode with the library's static scratch as its workspace
    (``fi_batch_decode_paged_noalloc``): no workspace argument, nothing
    allocated."""
    _check(lib().fi_batch_decode_paged_noalloc(
        plan.host_ptr(), _ptr(plan_dev), ctypes.byref(params), _ptr(q), _ptr(kv_pool),
        kv_pool.shape[0], _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(o),
        _ptr(lse), _stream(stream)))


def fi_batch_prefill_paged(plan: Plan, plan_dev, params: fi_attn_params, q, kv_pool, qo_indptr,
                           kv_indptr, kv_indices, kv_last_page_len, o, lse, float_ws,
                           stream=None):
    _check(lib().fi_batch_prefill_paged(
        plan.host_ptr(), _ptr(plan_dev), ctypes.byref(params), _ptr(q), _ptr(kv_pool),
        kv_pool.shape[0], _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
        _ptr(kv_last_page_len), _ptr(o), _ptr(lse), _ptr(float_ws),
        float_ws.numel() * float_ws.element_size(), _stream(stream)))


def fi_merge_state(v_a, s_a, v_b, s_b, v_out, s_out, stream=None):
    """Two-way log-sum-exp merge; v: [n_tokens, n_heads, head_dim], s: [n_tokens, n_heads]."""
    n, h, d = v_a.shape
    _check(lib().fi_merge_state(_ptr(v_a), _ptr(s_a), _ptr(v_b), _ptr(s_b), _ptr(v_out),
                                _ptr(s_out), n, h, d, _dtype_code(v_a.dtype), _stream(stream)))


def fi_cascade_workspace_bytes(plan0: Plan, plan1: Plan) -> int:
    n = int(lib().fi_cascade_workspace_bytes(plan0.host_ptr(), plan1.host_ptr()))
    if n < 0:
        _check(n)
    return n


def fi_cascade(plan0: Plan, plan0_dev, qo_indptr0, kv_indptr0, kv_indices0, kv_last_page_len0,
               plan1: Plan, plan1_dev, qo_indptr1, kv_indptr1, kv_indices1, kv_last_page_len1,
               params: fi_attn_params, q, kv_pool, o, lse, float_ws, stream=None):
    _check(lib().fi_cascade(
        plan0.host_ptr(), _ptr(plan0_dev), _ptr(qo_indptr0), _ptr(kv_indptr0), _ptr(kv_indices0),
        _ptr(kv_last_page_len0), plan1.host_ptr(), _ptr(plan1_dev), _ptr(qo_indptr1),
        _ptr(kv_indptr1), _ptr(kv_indices1), _ptr(kv_last_page_len1), ctypes.byref(params),
        _ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(o), _ptr(lse), _ptr(float_ws),
        float_ws.numel() * float_ws.element_size(), _stream(stream)))


def fi_append_paged_kv(append_k, append_v, append_indptr, kv_pool, kv_indptr, kv_indices,
                       kv_last_page_len, stream=None):
    """Write new K/V rows ``[n_tokens, Hk, D]`` into their pages of ``kv_pool``
    ``[pages, 2, P, Hk, D]`` (``fi_append_paged_kv``); index arrays are device int32."""
    n, hk, d = append_k.shape
    pages, two, page_size, hk2, d2 = kv_pool.shape
    if (append_v.shape != append_k.shape or two != 2 or (hk2, d2) != (hk, d)
            or append_v.dtype != append_k.dtype or kv_pool.dtype != append_k.dtype):
        raise FIError(FI_ERR_INVALID_ARG, "fi_append_paged_kv: shapes or dtypes disagree")
    for t in (append_k, append_v, kv_pool, append_indptr, kv_indptr, kv_indices, kv_last_page_len):
        if not t.is_contiguous():
            raise FIError(FI_ERR_INVALID_ARG, "fi_append_paged_kv: tensors must be contiguous")
    _check(lib().fi_append_paged_kv(_ptr(append_k), _ptr(append_v), _dtype_code(append_k.dtype),
                                    _ptr(append_indptr), append_indptr.numel() - 1, n, _ptr(kv_pool),
                                    pages, page_size, hk, d, _ptr(kv_indptr), _ptr(kv_indices),
                                    kv_indices.numel(), _ptr(kv_last_page_len), _stream(stream)))


def workspace(nbytes: int, device="cuda") -> "torch.Tensor":
    """A float workspace of at least ``nbytes`` bytes, zero-filled: its control
    region (the status word) must be zero when first used."""
    return torch.zeros(max(int(nbytes), 4) // 4 + 64, dtype=torch.float32, device=device)


def fi_read_status(float_ws, clear: bool = False, stream=None) -> int:
    """The status word of a workspace (``fi_read_status``; None: the static
    scratch of the no-alloc decode on the current device): bit
    ``FI_STATUS_BAD_PAGE`` is set once a run call has met a page id outside the
    pool.  Synchronises ``stream``; ``clear`` resets the word afterwards."""
    out = ctypes.c_int32()
    ws = None if float_ws is None else _ptr(float_ws)
    _check(lib().fi_read_status(ws, ctypes.byref(out), int(bool(clear)), _stream(stream)))
    return int(out.value)


def fi_last_error() -> str:
    return lib().fi_last_error().decode()


def fi_version() -> int:
    return int(lib().fi_version())


def fi_default_workers(kind: int, num_cus: int, num_kv_heads: int) -> int:
    return int(lib().fi_default_workers(kind, num_cus, num_kv_heads))


def decode_plan_buffer(buf) -> dict:
    """Split a plan buffer into its arrays (used to compare plans)."""
    b = np.asarray(buf)
    out = {"header": b[:12].tolist()}
    for name, at in (("decode", H_STREAM0), ("prefill", H_STREAM1)):
        d = b[at:at + 20]
        W, nr, ni, ns = int(d[S_W]), int(d[S_NROWS]), int(d[S_NITEMS]), int(d[S_NSPLIT])
        out[name] = dict(
            W=W, S=int(d[S_SEG]), BR=int(d[S_TILE]), n_slots=int(d[S_NSLOTS]),
            slot_cap=int(d[S_SLOTCAP]), ws_off_o=int(d[S_WS_O]), ws_off_lse=int(d[S_WS_LSE]),
            rows=[tuple(x) for x in b[d[S_OFF_ROWS]:d[S_OFF_ROWS] + 4 * nr].reshape(-1, 4).tolist()],
            items=[tuple(x) for x in b[d[S_OFF_ITEMS]:d[S_OFF_ITEMS] + 4 * ni].reshape(-1, 4).tolist()],
            wip=b[d[S_OFF_WIP]:d[S_OFF_WIP] + W + 1].tolist(),
            merge_indptr=b[d[S_OFF_MERGE]:d[S_OFF_MERGE] + nr + 1].tolist(),
            split_rows=b[d[S_OFF_SPLIT]:d[S_OFF_SPLIT] + ns].tolist(),
            item_meta=[tuple(x) for x in b[d[S_OFF_META]:d[S_OFF_META] + 8 * ni].reshape(-1, 8).tolist()],
            split_records=[tuple(x) for x in b[d[S_OFF_SREC]:d[S_OFF_SREC] + 4 * ns].reshape(-1, 4).tolist()])
    return out
