"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = the whole path over one batch: the host plan (fi_plan), its upload
to the device, and the run call (persistent decode kernel + partial merge),
with inputs resident in HBM.  Default workload: batch decode of the
Llama-3-8B attention shape (batch 64, 32 query / 8 KV heads, head_dim 128,
bf16, page 16, kv_len uniform in [512, 4096], random page permutation).

Prints one JSON line.  ``value`` is algorithmic GB/s of the whole step
(K/V once per KV head for valid tokens, plus Q, O, LSE and index arrays) over
the step's wall time; ``roofline.achieved`` is the same bytes over the run
call's average duration measured with HIP events on its stream;
``cpu_baseline`` times the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode HBM GB/s & causal prefill TFLOP/s (bf16), % of MI355X peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
NUM_CUS = 256


def log(*a):
    print(*a, file=sys.stderr, flush=True)


EVENT_EVERY = 8  # timed steps per HIP-event sample of the call duration

PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_mfma_kernel_llama8b_decode_pmc.json")


def counter_traffic(workload):
    """HBM bytes per decode-kernel dispatch from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, scaled by the copy-kernel calibration;
    None when that summary was taken on another workload or on a decode
    kernel source that has changed since."""
    import hashlib
    try:
        d = json.load(open(PMC_SUMMARY))
        src = open(os.path.join(ROOT, d["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != d["source_sha256_16"]:
        return None
    if workload != "llama8b_decode":
        return None
    return int(d["traffic_bytes_per_dispatch"])


def decode_bytes(b, window_left=-1) -> int:
    """Algorithmic bytes of one decode pass (the method's own traffic).  With a
    sliding window only the keys inside it, and the page-table entries of
    their pages, are counted."""
    esz = 2 if b.dtype.itemsize == 2 else 4
    kv_lens = b.kv_lens.astype(np.int64)
    if window_left >= 0:
        first = np.maximum(kv_lens - 1 - window_left, 0)
        keys = int((kv_lens - first).sum())
        P = b.page_size
        pages = int((-(-kv_lens // P) - first // P).sum())
    else:
        keys, pages = int(kv_lens.sum()), len(b.kv_indices)
    kv = keys * b.num_kv_heads * 2 * b.head_dim * esz
    qo = 2 * b.total_qo * b.num_qo_heads * b.head_dim * esz
    lse = b.total_qo * b.num_qo_heads * 4
    idx = 4 * (pages + len(b.kv_indptr) + len(b.kv_last_page_len))
    return kv + qo + lse + idx


def run_decode_bench(args):
    import torch

    import paged_kv_block_bsr_amd as fi
    import workloads as wl

    b = getattr(wl, args.workload)()
    B, Hq, Hk, D, P = b.batch_size, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.page_size
    wd = args.workers_decode or fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ncopy = max(1, args.pool_copies)
    pools = [b.kv_pool.to(dev) for _ in range(ncopy)]  # rotated so a step cannot hit caches warmed by the last
    q = b.q.to(dev)
    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to(dev)
    kv_indptr_d, kv_indices_d, last_d = i32(b.kv_indptr), i32(b.kv_indices), i32(b.kv_last_page_len)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    cap_ints, ws_bytes = fi.fi_plan_bounds(B, B, Hq, Hk, D, wd, 1)
    ws = fi.workspace(ws_bytes, dev)
    pinned = [torch.empty(cap_ints, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    plan_dev = [torch.empty(cap_ints, dtype=torch.int32, device=dev) for _ in range(2)]
    copied = [torch.cuda.Event() for _ in range(2)]
    for e in copied:
        e.record()
    params = fi.make_params(b.dtype, b.dtype, Hq, Hk, D, P, b.sm_scale, b.soft_cap)
    kv_indptr_h = np.ascontiguousarray(b.kv_indptr, np.int32)
    last_h = np.ascontiguousarray(b.kv_last_page_len, np.int32)

    # The call's duration is sampled with HIP events on every EVENT_EVERY-th
    # timed step: timing events around every call add ~7.5 us to each step.
    sampled = list(range(0, args.steps, EVENT_EVERY))
    starts = {k: torch.cuda.Event(enable_timing=True) for k in sampled}
    ends = {k: torch.cuda.Event(enable_timing=True) for k in sampled}
    info = {}

    def step(k, timed_idx=None):
        j = k % 2
        copied[j].synchronize()  # the upload that last read this pinned buffer is done
        plan = fi.fi_plan(None, kv_indptr_h, last_h, page_size=P, num_qo_heads=Hq,
                          num_kv_heads=Hk, head_dim=D, causal=True, workers_decode=wd,
                          workers_prefill=1, min_seg_pages=args.min_seg_pages,
                          out=pinned[j].numpy())
        info["plan"] = plan
        # only the plan's own ints: a copy of a few KiB runs as a short blit
        # on the stream, where the whole capacity buffer (> 16 KiB with many
        # workers) went to the DMA engine and left a ~20 us gap per step
        n = plan.ints
        plan_dev[j][:n].copy_(pinned[j][:n], non_blocking=True)
        copied[j].record()
        if timed_idx in starts:
            starts[timed_idx].record()
        fi.fi_batch_decode_paged(plan, plan_dev[j], params, q, pools[k % ncopy], kv_indptr_d,
                                 kv_indices_d, last_d, o, lse, ws)
        if timed_idx in ends:
            ends[timed_idx].record()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    call_ms = float(np.mean([starts[k].elapsed_time(ends[k]) for k in sampled]))
    nbytes = decode_bytes(b)
    plan = info["plan"]
    result = {
        "metric": METRIC,
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if b.dtype.itemsize == 2 else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": B, "num_qo_heads": Hq, "num_kv_heads": Hk,
            "head_dim": D, "page_size": P, "sum_kv_len": int(b.kv_lens.sum()),
            "pool_pages": b.pool_pages, "workers_decode": wd,
            "decode_items": int(plan.info.decode_items), "decode_slots": int(plan.info.decode_slots),
            "algorithmic_bytes_per_step": nbytes,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(nbytes / (call_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic(args.workload),
            "kernel_ms": round(call_ms, 5),
            "kernel": "decode_kernel + merge_partials_kernel (one fi_batch_decode_paged call)",
        },
    }
    return result, b, nbytes


def prefill_flops(b, window_left=-1) -> int:
    """Visible flops: 4 D per (query head, visible key) pair (QK^T and PV).
    Query t of a request sees keys up to p = kv - qo + t (causal) or kv - 1,
    and with a sliding window none before p - window_left."""
    tot = 0
    for qo, kv in zip(b.qo_lens.tolist(), b.kv_lens.tolist()):
        p = kv - qo + np.arange(qo, dtype=np.int64)
        hi = p + 1 if b.causal else np.full(qo, kv, np.int64)
        lo = np.maximum(p - window_left, 0) if window_left >= 0 else np.zeros(qo, np.int64)
        tot += int(np.maximum(hi - lo, 0).sum())
    return 4 * b.head_dim * b.num_qo_heads * tot


def tree_flops(b) -> int:
    """Visible flops under a tree mask: 4 D per (query head, visible key)
    pair, where draft token t sees the keys before the draft, itself and the
    draft tokens its bits name (u < t)."""
    bits = np.unpackbits(np.asarray(b.tree_mask, np.uint8), bitorder="little")
    tot = 0
    for i, (qo, kv) in enumerate(zip(b.qo_lens.tolist(), b.kv_lens.tolist())):
        blk = bits[b.mask_indptr[i]:b.mask_indptr[i] + qo * qo].reshape(qo, qo).astype(bool)
        vis = np.tril(blk, -1).sum(axis=1) + 1 + (kv - qo)
        tot += int(vis.sum())
    return 4 * b.head_dim * b.num_qo_heads * tot


def prefill_slice(b):
    """The batch restricted to its multi-query requests (same pool and values)."""
    import workloads as wl
    keep = [i for i, q in enumerate(b.qo_lens.tolist()) if q >= 2]
    qo = b.qo_lens[keep]
    kv_indptr = [0]
    idx = []
    qrows = []
    for i in keep:
        pages = b.kv_indices[b.kv_indptr[i]:b.kv_indptr[i + 1]]
        idx.append(pages)
        kv_indptr.append(kv_indptr[-1] + len(pages))
        qrows.append(b.q[b.qo_indptr[i]:b.qo_indptr[i + 1]])
    qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    import torch
    return wl.PagedBatch(page_size=b.page_size, num_qo_heads=b.num_qo_heads,
                         num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype,
                         causal=b.causal, sm_scale=b.sm_scale, soft_cap=b.soft_cap, qo_lens=qo,
                         kv_lens=b.kv_lens[keep], qo_indptr=qo_indptr,
                         kv_indptr=np.asarray(kv_indptr, np.int32),
                         kv_indices=np.concatenate(idx).astype(np.int32),
                         kv_last_page_len=b.kv_last_page_len[keep].copy(),
                         q=torch.cat(qrows), kv_pool=b.kv_pool, name=b.name + "/prefill_slice")


def time_batch_call(b, steps, warmup, workers_decode=0, workers_prefill=0, pool_copies=2,
                    window_left=-1, rope_theta=0.0, no_split=0):
    """Plan once, then time the run call (decode/prefill kernels + merges) with
    HIP events on its stream.  Returns (mean ms, plan)."""
    import torch

    import paged_kv_block_bsr_amd as fi
    dev = torch.device("cuda", 0)
    Hk = b.num_kv_heads
    wd = workers_decode or fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk)
    wp = workers_prefill or fi.fi_default_workers(fi.FI_KIND_PREFILL, NUM_CUS, Hk)
    plan = fi.fi_plan(b.qo_indptr, b.kv_indptr, b.kv_last_page_len, page_size=b.page_size,
                      num_qo_heads=b.num_qo_heads, num_kv_heads=Hk, head_dim=b.head_dim,
                      causal=b.causal, workers_decode=wd, workers_prefill=wp,
                      window_left=window_left, no_split=no_split)
    plan_dev = plan.to_device(dev)
    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to(dev)
    pools = [b.kv_pool.to(dev) for _ in range(max(1, pool_copies))]
    q = b.q.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = fi.workspace(plan.float_ws_bytes, dev)
    mask = mask_ip = None
    if getattr(b, "tree_mask", None) is not None:
        mask = torch.from_numpy(fi.tree_mask_words(b.tree_mask)).to(dev)
        mask_ip = i32(b.mask_indptr)
    params = fi.make_params(b.dtype, b.dtype, b.num_qo_heads, Hk, b.head_dim, b.page_size,
                            b.sm_scale, b.soft_cap, rope_theta=rope_theta, tree_mask=mask,
                            mask_indptr=mask_ip,
                            mask_bits=0 if mask is None else int(b.mask_indptr[-1]))
    qo_d, kvp_d, kvi_d, last_d = (None if b.qo_indptr is None else i32(b.qo_indptr),
                                  i32(b.kv_indptr), i32(b.kv_indices), i32(b.kv_last_page_len))

    def call(k):
        if b.qo_indptr is None:
            fi.fi_batch_decode_paged(plan, plan_dev, params, q, pools[k % len(pools)], kvp_d,
                                     kvi_d, last_d, o, lse, ws)
        else:
            fi.fi_batch_prefill_paged(plan, plan_dev, params, q, pools[k % len(pools)], qo_d,
                                      kvp_d, kvi_d, last_d, o, lse, ws)

    for k in range(warmup):
        call(k)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record()
        call(k)
        ev[k][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    del pools
    return ms, plan


def secondary_measurements(args):
    """Prefill slice TFLOP/s, whole mixed step and cascade vs flat (context for
    the headline decode figure; same kernels, other workloads)."""
    import workloads as wl
    out = {}
    out["skewed_long_decode"] = skewed_measurements(args.side_steps)
    out["page_order"] = page_order_measurements(args.side_steps)
    out["plan_host"] = plan_host_times()
    b = wl.mixed_ragged_step()
    ps = prefill_slice(b)
    ms, plan = time_batch_call(ps, args.side_steps, 3)
    fl = prefill_flops(ps)
    out["prefill_slice"] = {
        "workload": "mixed_ragged_step prefill requests (16 causal prefills)",
        "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "peak_tflops": BF16_PEAK_TFLOPS,
        "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4), "ms": round(ms, 4),
        "flops": fl, "tile_rows": int(plan.info.prefill_tile_rows),
        "prefill_items": int(plan.info.prefill_items)}
    ms, plan = time_batch_call(b, args.side_steps, 3)
    nb = decode_bytes(b)
    fl = prefill_flops(b)
    out["mixed_step"] = {
        "workload": "mixed_ragged_step (16 prefills + 48 decodes, one call)",
        "ms": round(ms, 4), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
        "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
        "roofline_frac": round(max(nb / (HBM_PEAK_GBS * 1e9), fl / (BF16_PEAK_TFLOPS * 1e12)) / (ms * 1e-3), 4)}
    out["prefill_page_sizes"] = prefill_page_size_measurements(ps, args.side_steps)
    out["append"] = time_append(b, args.side_steps)
    out["window"] = window_measurements(ps, args.side_steps)
    out["rope"] = rope_measurements(ps, args.side_steps)
    del b, ps
    sv = wl.speculative_verify()
    ms, plan = time_batch_call(sv, args.side_steps, 3)
    fl = tree_flops(sv)
    out["tree_mask"] = {"workload": "speculative_verify (32 requests, draft trees of 16/32/64 tokens "
                                    "over prefixes U[512, 4096], tree mask)",
                        "ms": round(ms, 4), "flops": fl, "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                        "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "bytes": decode_bytes(sv),
                        "gbs": round(decode_bytes(sv) / (ms * 1e-3) / 1e9, 1)}
    del sv
    cb = wl.shared_prefix_cascade()
    ms_flat, _ = time_batch_call(cb.flat, args.side_steps, 3)
    # level 1 holds only short suffixes (50-200 tokens): segments of 2 pages
    # spread them over the workers (8-page segments leave most of them idle)
    ms_casc = time_cascade(cb, args.side_steps, 3, min_seg1=2)
    out["cascade"] = {"workload": "shared_prefix_cascade (64 requests, 2048-token prefix, soft-cap 30)",
                      "cascade_us": round(ms_casc * 1e3, 2), "flat_us": round(ms_flat * 1e3, 2),
                      "speedup": round(ms_flat / ms_casc, 3)}
    return out


def prefill_page_size_measurements(ps, steps):
    """The prefill slice's 16 requests (same query and KV lengths) stored with
    pages of 1, 4, 16 and 64 tokens (pages of 1 token: the column-vector
    BSR of the pages), each batch drawn by the same generator, so only the
    page size differs.
    The page sizes are timed in turn, five rounds (fresh device copies of the
    pools each time, so their placement in memory varies), and each reports its
    median round, so that a drift of the clock during the leg does not land
    on one page size only."""
    import workloads as wl
    fl = prefill_flops(ps)
    out = {"workload": "mixed_ragged_step prefill requests, page size 1 / 4 / 16 / 64", "flops": fl,
           "rounds": 5}
    sizes = (1, 4, 16, 64)
    batches = {P: wl.make_batch(1009, ps.qo_lens, ps.kv_lens, page_size=P, num_qo_heads=ps.num_qo_heads,
                                num_kv_heads=ps.num_kv_heads, head_dim=ps.head_dim, dtype=ps.dtype,
                                causal=True, name=f"prefill_slice_P{P}") for P in sizes}
    times = {P: [] for P in sizes}
    for _ in range(out["rounds"]):
        for P in sizes:
            times[P].append(time_batch_call(batches[P], steps, 3)[0])
    for P in sizes:
        ms = float(np.median(times[P]))
        out[f"P{P}"] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
    out["P1_over_P16"] = round(out["P1"]["ms"] / out["P16"]["ms"], 3)
    return out


def skewed_measurements(steps):
    """Skewed long-context decode (batch 32: one 131072-token request, 31 of
    lognormal length): the plan's split of the long request into segments of equal cost
    with the merge of its partial states, against the same call with every
    row on one worker (no_split), which leaves the long request to a single
    wave."""
    import workloads as wl
    sb = wl.skewed_long_decode()
    nb = decode_bytes(sb)
    out = {"workload": "skewed_long_decode (batch 32, one 131072-token request)", "bytes": nb}
    for name, ns in (("split", 0), ("no_split", 1)):
        ms, plan = time_batch_call(sb, steps, 3, no_split=ns)
        out[name] = {"us": round(ms * 1e3, 2), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                     "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "decode_items": int(plan.info.decode_items),
                     "decode_slots": int(plan.info.decode_slots)}
    out["split_speedup"] = round(out["no_split"]["us"] / out["split"]["us"], 2)
    return out


def page_order_measurements(steps):
    """llama8b_decode with its pages randomly permuted over the pool (the
    bench workload) and with the identity page table (request i's pages
    contiguous, in order): how much the scattered gather costs."""
    import workloads as wl
    out = {"workload": "llama8b_decode call, random vs identity page table"}
    for name, ident in (("random", False), ("identity", True)):
        db = wl.llama8b_decode(identity_pages=ident)
        nb = decode_bytes(db)
        ms, _ = time_batch_call(db, steps, 3)
        out[name] = {"us": round(ms * 1e3, 2), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                     "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del db
    return out


def plan_host_times(reps=100):
    """Host time of fi_plan (the CPU-side inspector), median of ``reps`` calls
    into a preallocated buffer, for the bench workloads."""
    import paged_kv_block_bsr_amd as fi
    import workloads as wl
    out = {"reps": reps}
    for b in (wl.llama8b_decode(), wl.skewed_long_decode(), wl.mixed_ragged_step()):
        Hk = b.num_kv_heads
        kw = dict(page_size=b.page_size, num_qo_heads=b.num_qo_heads, num_kv_heads=Hk, head_dim=b.head_dim,
                  causal=b.causal, workers_decode=fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk),
                  workers_prefill=fi.fi_default_workers(fi.FI_KIND_PREFILL, NUM_CUS, Hk))
        qo = b.qo_indptr
        total_qo = int(b.total_qo)
        cap, _ = fi.fi_plan_bounds(b.batch_size, total_qo, b.num_qo_heads, Hk, b.head_dim,
                                   kw["workers_decode"], kw["workers_prefill"])
        buf = np.empty(cap, np.int32)
        ip, last = np.ascontiguousarray(b.kv_indptr, np.int32), np.ascontiguousarray(b.kv_last_page_len, np.int32)
        ts = []
        for _ in range(reps + 3):
            t0 = time.perf_counter()
            fi.fi_plan(qo, ip, last, out=buf, **kw)
            ts.append(time.perf_counter() - t0)
        ts = np.array(ts[3:]) * 1e6
        out[b.name] = {"median_us": round(float(np.median(ts)), 1), "p90_us": round(float(np.percentile(ts, 90)), 1),
                       "batch": b.batch_size, "total_qo": total_qo}
    return out


WINDOW = 1023  # keys a query sees before its own (a 1024-key sliding window)


def window_measurements(ps, steps):
    """Sliding-window attention with a 1024-key window: the decode workload
    (each request reads its last <= 1024 keys) and the prefill slice of the
    mixed step.  Only keys inside the window count as work."""
    import workloads as wl
    db = wl.llama8b_decode()
    ms, plan = time_batch_call(db, steps, 3, window_left=WINDOW)
    nb = decode_bytes(db, WINDOW)
    out = {"window_left": WINDOW,
           "decode": {"workload": "llama8b_decode, window 1023", "us": round(ms * 1e3, 2),
                      "bytes": nb, "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                      "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    del db
    ms, plan = time_batch_call(ps, steps, 3, window_left=WINDOW)
    fl = prefill_flops(ps, WINDOW)
    out["prefill_slice"] = {"workload": "mixed_ragged_step prefill requests, window 1023",
                            "ms": round(ms, 4), "flops": fl,
                            "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                            "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return out


ROPE_THETA = 500000.0  # rotary base of the Llama-3 family


def rope_measurements(ps, steps):
    """Fused rotary embedding on q and k: the decode workload (the default
    worker count and 8 per CU, as many as the rotary decode kernel's two waves
    per SIMD hold) and the prefill slice of the mixed step.  Same algorithmic
    bytes and flops as without it."""
    import workloads as wl
    import paged_kv_block_bsr_amd as fi
    db = wl.llama8b_decode()
    nb = decode_bytes(db)
    out = {"rope_theta": ROPE_THETA, "decode": {"workload": "llama8b_decode, rotary embedding"}}
    for w in (fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, db.num_kv_heads), 8 * NUM_CUS // db.num_kv_heads):
        ms, _ = time_batch_call(db, steps, 3, workers_decode=w, rope_theta=ROPE_THETA)
        out["decode"][f"workers_{w}"] = {"us": round(ms * 1e3, 2), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                                         "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del db
    ms, _ = time_batch_call(ps, steps, 3, rope_theta=ROPE_THETA)
    fl = prefill_flops(ps)
    out["prefill_slice"] = {"workload": "mixed_ragged_step prefill requests, rotary embedding",
                            "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                            "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return out


def time_append(b, steps):
    """Paged KV append of a step's new tokens (fi_append_paged_kv), timed with
    HIP events on its stream: the mixed step's new tokens (every query
    token's K/V row) into its pool, and one 32768-token prefill's.  Bytes =
    each token row read once and written once, for K and V."""
    import torch

    import paged_kv_block_bsr_amd as fi
    dev = torch.device("cuda", 0)
    Hk, D, P = b.num_kv_heads, b.head_dim, b.page_size
    esz = 2 if b.dtype == torch.bfloat16 else 4
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    rng = np.random.default_rng(1006)
    res = {}
    long_pages = 32768 // P
    cases = {
        "mixed_step_new_tokens": (b.qo_lens, b.kv_indptr, b.kv_indices, b.kv_last_page_len, b.kv_pool.to(dev)),
        "prefill_32768": (np.array([32768]), np.array([0, long_pages], np.int32),
                          rng.permutation(long_pages + 8)[:long_pages].astype(np.int32), np.array([P], np.int32),
                          torch.zeros((long_pages + 8, 2, P, Hk, D), dtype=b.dtype, device=dev)),
    }
    for name, (new, kv_ip, kv_idx, last, pool) in cases.items():
        n = int(np.sum(new))
        a_ip = np.zeros(len(new) + 1, np.int32)
        a_ip[1:] = np.cumsum(new)
        k = torch.randn((n, Hk, D), device=dev).to(b.dtype)
        v = torch.randn((n, Hk, D), device=dev).to(b.dtype)
        args = (k, v, i32(a_ip), pool, i32(kv_ip), i32(kv_idx), i32(last))
        for _ in range(3):
            fi.fi_append_paged_kv(*args)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for s, e in ev:
            s.record()
            fi.fi_append_paged_kv(*args)
            e.record()
        torch.cuda.synchronize()
        ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
        nbytes = 2 * 2 * n * Hk * D * esz
        res[name] = {"tokens": n, "bytes": nbytes, "us": round(ms * 1e3, 2),
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del args, pool
    return res


def prefill_only(args):
    """The prefill slice of the mixed ragged step alone, timed like the side
    measurement (one plan, then the run call on its stream)."""
    import workloads as wl
    ps = prefill_slice(wl.mixed_ragged_step())
    ms, plan = time_batch_call(ps, args.side_steps, 3)
    fl = prefill_flops(ps)
    return {"workload": "mixed_ragged_step prefill requests (16 causal prefills)", "ms": round(ms, 4),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "flops": fl,
            "prefill_items": int(plan.info.prefill_items), "steps": args.side_steps}


def side_only(args):
    """One side measurement alone (``--mode mixed | cascade | skewed | pages | append``)."""
    import workloads as wl
    if args.mode == "append":
        return time_append(wl.mixed_ragged_step(), args.side_steps)
    if args.mode == "skewed":
        return skewed_measurements(args.side_steps)
    if args.mode == "pages":
        return prefill_page_size_measurements(prefill_slice(wl.mixed_ragged_step()), args.side_steps)
    if args.mode == "mixed":
        b = wl.mixed_ragged_step()
        ms, _ = time_batch_call(b, args.side_steps, 3)
        nb, fl = decode_bytes(b), prefill_flops(b)
        return {"workload": "mixed_ragged_step (16 prefills + 48 decodes, one call)", "ms": round(ms, 4),
                "gbs": round(nb / (ms * 1e-3) / 1e9, 1), "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
    cb = wl.shared_prefix_cascade()
    ms_flat, _ = time_batch_call(cb.flat, args.side_steps, 3)
    ms_casc = time_cascade(cb, args.side_steps, 3, min_seg1=2)
    return {"workload": "shared_prefix_cascade (64 requests, 2048-token prefix, soft-cap 30)",
            "cascade_us": round(ms_casc * 1e3, 2), "flat_us": round(ms_flat * 1e3, 2)}


def time_cascade(cb, steps, warmup, min_seg0=8, min_seg1=8):
    import torch

    import paged_kv_block_bsr_amd as fi
    dev = torch.device("cuda", 0)
    l0, l1 = cb.level0, cb.level1
    Hk = l0.num_kv_heads
    kw = dict(page_size=l0.page_size, num_qo_heads=l0.num_qo_heads, num_kv_heads=Hk,
              head_dim=l0.head_dim, workers_decode=fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk),
              workers_prefill=fi.fi_default_workers(fi.FI_KIND_PREFILL, NUM_CUS, Hk))
    p0 = fi.fi_plan(l0.qo_indptr, l0.kv_indptr, l0.kv_last_page_len, causal=False,
                    min_seg_pages=min_seg0, **kw)
    p1 = fi.fi_plan(None, l1.kv_indptr, l1.kv_last_page_len, causal=True, min_seg_pages=min_seg1,
                    **kw)
    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to(dev)
    q, pool = l0.q.to(dev), l0.kv_pool.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = fi.workspace(fi.fi_cascade_workspace_bytes(p0, p1), dev)
    params = fi.make_params(l0.dtype, l0.dtype, l0.num_qo_heads, Hk, l0.head_dim, l0.page_size,
                            l0.sm_scale, l0.soft_cap)
    a0 = (p0, p0.to_device(dev), i32(l0.qo_indptr), i32(l0.kv_indptr), i32(l0.kv_indices),
          i32(l0.kv_last_page_len))
    a1 = (p1, p1.to_device(dev), None, i32(l1.kv_indptr), i32(l1.kv_indices),
          i32(l1.kv_last_page_len))

    def call():
        fi.fi_cascade(*a0, *a1, params, q, pool, o, lse, ws)

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record()
        call()
        ev[k][1].record()
    torch.cuda.synchronize()
    return float(np.mean([s.elapsed_time(e) for s, e in ev]))


def calibrate(reps=10):
    """Plain torch copy (1 GiB read + 1 GiB written) and a streaming sum over
    2 GiB: the achievable-bandwidth context and the known-size kernels that
    scale the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda", 0)
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    big = torch.ones(n // 2, dtype=torch.float32, device=dev)  # 2 GiB
    out = {}
    for name, fn, moved in (("copy_1GiB", lambda: dst.copy_(src), 2 * n),
                            ("sum_2GiB", lambda: big.sum(), 2 * n)):
        for _ in range(3):
            fn()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(reps):
            fn()
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / reps
        out[name] = {"us": round(ms * 1e3, 2), "gbs": round(moved / (ms * 1e-3) / 1e9, 1)}
    return out


def host_cpu():
    """The host's CPU model (first 'model name' of /proc/cpuinfo), its
    logical CPUs and those this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(b, nbytes, budget_s=12.0, single_budget_s=4.0):
    """The fp64 oracle on the host cores over the whole batch (the sample),
    then with one thread over the first requests of the batch (the requests
    that fit its time budget), so the per-core rate is on record too."""
    from oracle import attn as ref

    q64 = b.q.double().numpy()
    pool64 = b.kv_pool.double().numpy()
    kw = dict(page_size=b.page_size, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
              head_dim=b.head_dim, causal=b.causal, sm_scale=b.sm_scale, soft_cap=b.soft_cap)
    times = []
    while True:
        t0 = time.perf_counter()
        ref.attention(q64, pool64, b.qo_indptr, b.kv_indptr, b.kv_indices, b.kv_last_page_len, **kw)
        times.append(time.perf_counter() - t0)
        log(f"[bench] oracle pass {len(times)}: {times[-1]:.2f} s")
        if sum(times) >= budget_s or len(times) >= 30:
            break
    t = float(np.mean(times))
    threads = ref.num_threads()
    out = {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"whole {b.name} batch (all {b.total_qo * b.num_qo_heads} query rows), "
                     f"{len(times)} passes, mean {t:.2f} s per pass", **host_cpu()}
    # one thread: decode requests 0 .. k-1, k grown until the pass takes a
    # second or more (bytes counted for those requests alone)
    assert b.qo_indptr is None, "the single-thread leg samples decode requests"
    ref.set_num_threads(1)
    try:
        k, t1 = 1, 0.0
        while True:
            sub_ip = np.ascontiguousarray(b.kv_indptr[:k + 1])
            t0 = time.perf_counter()
            ref.attention(q64[:k], pool64, None, sub_ip, b.kv_indices, b.kv_last_page_len[:k], **kw)
            t1 = time.perf_counter() - t0
            if t1 >= single_budget_s / 4 or k == b.batch_size:
                break
            k = min(b.batch_size, 2 * k)
        kv = b.kv_lens[:k].astype(np.int64)
        esz = 2 if b.dtype.itemsize == 2 else 4
        sub_bytes = (int(kv.sum()) * b.num_kv_heads * 2 * b.head_dim * esz +
                     k * b.num_qo_heads * (2 * b.head_dim * esz + 4) +
                     4 * (int(b.kv_indptr[k]) + 2 * k + 1))
        out["single_thread"] = {"value": round(sub_bytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "sample": f"requests 0..{k - 1} of {b.name}, one pass, {t1:.2f} s"}
    finally:
        ref.set_num_threads(threads)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_decode",
                    choices=["llama8b_decode", "skewed_long_decode", "tiny_decode_fp32"])
    ap.add_argument("--workers-decode", type=int, default=0)
    ap.add_argument("--min-seg-pages", type=int, default=8)
    ap.add_argument("--pool-copies", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the prefill / mixed / cascade side measurements")
    ap.add_argument("--side-steps", type=int, default=20)
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "secondary", "prefill", "mixed", "cascade", "skewed", "pages", "append",
                             "calibrate"],
                    help="secondary: only the side measurements; prefill / mixed / cascade / skewed / pages / append: "
                         "only that timing (for profiling its kernels): the prefill slice, the whole "
                         "mixed step, the cascade (and its flat equivalent), skewed_long_decode split "
                         "and unsplit, the prefill slice at page sizes 1 / 4 / 16 / 64; calibrate: only "
                         "the plain copy / streaming-sum kernels")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    if args.mode == "secondary":
        print(json.dumps(secondary_measurements(args)), flush=True)
        return
    if args.mode == "calibrate":
        print(json.dumps(calibrate()), flush=True)
        return
    if args.mode == "prefill":
        print(json.dumps(prefill_only(args)), flush=True)
        return
    if args.mode in ("mixed", "cascade", "skewed", "pages", "append"):
        print(json.dumps(side_only(args)), flush=True)
        return
    result, b, nbytes = run_decode_bench(args)
    if not args.no_secondary:
        result["secondary"] = secondary_measurements(args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(b, nbytes)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
