"""A whole step captured once into a HIP graph and replayed with changing
lengths (serving-engine page, "How FlashInfer Works": a host plan per step,
persistent fixed-grid kernels inside a captured graph).

The graph holds the uploads of the plan, the index arrays and the queries
from fixed pinned host buffers, then one run call made with graph_safe set.
Each step refills the host buffers (new lengths, new page tables, a new plan)
and replays.  Every replay is checked bit-exactly against an eager call on
the same inputs, with eager work and synchronisation between replays, and
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import assert_close, note

pytestmark = pytest.mark.gpu

P, HQ, HK, D = 16, 32, 8, 128


def _step_batch(rng, pool, qo_lens, kv_lens, ragged):
    """A batch over the fixed pool: each request takes fresh random pages.
    ``ragged``: always carry qo_indptr (the prefill call's batches, also when
    every request has one query)."""
    qo_lens = np.asarray(qo_lens, np.int64)
    kv_lens = np.asarray(kv_lens, np.int64)
    pages = [(int(L) + P - 1) // P for L in kv_lens]
    perm = rng.permutation(pool.shape[0])[: sum(pages)].astype(np.int32)
    kv_indptr = np.zeros(len(kv_lens) + 1, np.int32)
    kv_indptr[1:] = np.cumsum(pages)
    last = np.array([int(L) - (n - 1) * P if n else 0 for L, n in zip(kv_lens, pages)], np.int32)
    q = torch.from_numpy(rng.standard_normal((int(qo_lens.sum()), HQ, D), dtype=np.float32)).to(torch.bfloat16)
    qo_indptr = None
    if ragged:
        qo_indptr = np.zeros(len(qo_lens) + 1, np.int32)
        qo_indptr[1:] = np.cumsum(qo_lens)
    return wl.PagedBatch(page_size=P, num_qo_heads=HQ, num_kv_heads=HK, head_dim=D,
                         dtype=torch.bfloat16, causal=True, sm_scale=1.0 / np.sqrt(D), soft_cap=0.0,
                         qo_lens=qo_lens, kv_lens=kv_lens, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                         kv_indices=perm, kv_last_page_len=last, q=q, kv_pool=pool, name="graph step")


class _Fixed:
    """Device buffers and pinned host staging buffers that never move."""

    def __init__(self, B, max_qo, max_pages, cap_ints, ws_bytes, mixed):
        pin = lambda n, dt=torch.int32: torch.zeros(n, dtype=dt, pin_memory=True)
        self.mixed = mixed
        self.plan_h, self.plan_d = pin(cap_ints), torch.zeros(cap_ints, dtype=torch.int32, device="cuda")
        self.qo_h, self.qo_d = pin(B + 1), torch.zeros(B + 1, dtype=torch.int32, device="cuda")
        self.kvp_h, self.kvp_d = pin(B + 1), torch.zeros(B + 1, dtype=torch.int32, device="cuda")
        self.kvi_h, self.kvi_d = pin(max_pages), torch.zeros(max_pages, dtype=torch.int32, device="cuda")
        self.last_h, self.last_d = pin(B), torch.zeros(B, dtype=torch.int32, device="cuda")
        self.q_h = torch.zeros((max_qo, HQ, D), dtype=torch.bfloat16, pin_memory=True)
        self.q_d = torch.zeros((max_qo, HQ, D), dtype=torch.bfloat16, device="cuda")
        self.o = torch.zeros((max_qo, HQ, D), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.zeros((max_qo, HQ), dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")

    def fill(self, b, W_d, W_p, min_seg):
        """Host side of a step: index arrays, queries and the plan into the pinned buffers."""
        self.kvp_h.numpy()[:] = b.kv_indptr
        self.kvi_h.numpy()[:] = 0
        self.kvi_h.numpy()[: len(b.kv_indices)] = b.kv_indices
        self.last_h.numpy()[:] = b.kv_last_page_len
        if b.qo_indptr is not None:
            self.qo_h.numpy()[:] = b.qo_indptr
        self.q_h[: b.total_qo].copy_(b.q)
        return fi.fi_plan(b.qo_indptr if self.mixed else None, b.kv_indptr, b.kv_last_page_len,
                          page_size=P, num_qo_heads=HQ, num_kv_heads=HK, head_dim=D, causal=True,
                          workers_decode=W_d, workers_prefill=W_p, min_seg_pages=min_seg,
                          out=self.plan_h.numpy())

    def body(self, plan, params, pool):
        """The captured step: uploads, then one run call."""
        for h, d in ((self.plan_h, self.plan_d), (self.kvp_h, self.kvp_d), (self.kvi_h, self.kvi_d),
                     (self.last_h, self.last_d), (self.q_h, self.q_d), (self.qo_h, self.qo_d)):
            d.copy_(h, non_blocking=True)
        if self.mixed:
            fi.fi_batch_prefill_paged(plan, self.plan_d, params, self.q_d, pool, self.qo_d, self.kvp_d,
                                      self.kvi_d, self.last_d, self.o, self.lse, self.ws)
        else:
            fi.fi_batch_decode_paged(plan, self.plan_d, params, self.q_d, pool, self.kvp_d, self.kvi_d,
                                     self.last_d, self.o, self.lse, self.ws)


def _eager(b, pool, W_d, W_p, mixed, min_seg):
    """The same step through ordinary (non-graph) calls on buffers of its own."""
    plan = fi.fi_plan(b.qo_indptr if mixed else None, b.kv_indptr, b.kv_last_page_len, page_size=P,
                      num_qo_heads=HQ, num_kv_heads=HK, head_dim=D, causal=True, workers_decode=W_d,
                      workers_prefill=W_p, min_seg_pages=min_seg)
    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32).copy()).cuda()
    q = b.q.cuda()
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:2], dtype=torch.float32, device="cuda")
    ws = torch.zeros(plan.float_ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    params = fi.make_params(torch.bfloat16, torch.bfloat16, HQ, HK, D, P, b.sm_scale, 0.0)
    if mixed:
        fi.fi_batch_prefill_paged(plan, plan.to_device(), params, q, pool, i32(b.qo_indptr),
                                  i32(b.kv_indptr), i32(b.kv_indices), i32(b.kv_last_page_len), o, lse, ws)
    else:
        fi.fi_batch_decode_paged(plan, plan.to_device(), params, q, pool, i32(b.kv_indptr),
                                 i32(b.kv_indices), i32(b.kv_last_page_len), o, lse, ws)
    torch.cuda.synchronize()
    return o, lse, plan


def _run_steps(seed, steps, W_d, W_p, mixed, min_seg):
    rng = np.random.default_rng(seed)
    B = len(steps[0][0])
    max_qo = max(int(np.sum(q)) for q, _ in steps)
    max_pages = max(sum((int(L) + P - 1) // P for L in kv) for _, kv in steps)
    pool_pages = int(1.25 * max_pages) + 1
    pool_h = torch.from_numpy(rng.standard_normal((pool_pages, 2, P, HK, D), dtype=np.float32)).to(torch.bfloat16)
    pool = pool_h.cuda()
    cap, ws_bytes = fi.fi_plan_bounds(B, max_qo, HQ, HK, D, W_d, W_p)
    fx = _Fixed(B, max_qo, max_pages, cap, ws_bytes, mixed)
    batches = [_step_batch(rng, pool_h, q, kv, mixed) for q, kv in steps]
    params = fi.make_params(torch.bfloat16, torch.bfloat16, HQ, HK, D, P, 1.0 / np.sqrt(D), 0.0,
                            graph_safe=True)
    # capture on step 0 (the host plan is read at capture only; replays use the device copy)
    plan0 = fx.fill(batches[0], W_d, W_p, min_seg)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fx.body(plan0, params, pool)
    torch.cuda.synchronize()
    splits = []
    for s, b in enumerate(batches):
        plan = fx.fill(b, W_d, W_p, min_seg)
        kinds = (plan.info.decode_slots, plan.info.prefill_rows, plan.info.prefill_slots)
        splits.append(kinds)
        note(f"graph replay {'mixed' if mixed else 'decode'} step {s}: total_qo {b.total_qo}, "
             f"(decode slots, prefill rows, prefill slots) = {kinds}")
        graph.replay()
        torch.cuda.synchronize()
        n = b.total_qo
        o_g, l_g = fx.o[:n].clone(), fx.lse[:n].clone()
        o_e, l_e, _ = _eager(b, pool, W_d, W_p, mixed, min_seg)  # eager work between replays
        assert torch.equal(o_g, o_e), f"step {s}: replay and eager outputs differ"
        assert torch.equal(l_g, l_e), f"step {s}: replay and eager lse differ"
        o_ref, l_ref = ref.attention_of(b)
        assert_close(o_g.float().cpu(), l_g.cpu(), o_ref, l_ref, f"graph step {s}")
    return splits


def test_decode_step_graph_replays_with_changing_lengths():
    # step 0 (captured) has no split rows; later steps do, so the merge
    # captured under graph_safe must run for them
    steps = [([1] * 12, [40, 17, 3, 64, 30, 9, 55, 1, 16, 33, 48, 20]),
             ([1] * 12, [900, 17, 1300, 64, 2048, 9, 555, 1, 16, 733, 48, 1200]),
             ([1] * 12, [901, 18, 1301, 65, 2049, 10, 556, 2, 17, 734, 49, 1201]),
             ([1] * 12, [5, 2000, 7, 1999, 11, 13, 1024, 640, 16, 15, 1500, 3])]
    splits = _run_steps(7001, steps, W_d=16, W_p=1, mixed=False, min_seg=64)
    assert splits[0][0] == 0 and all(k[0] > 0 for k in splits[1:]), splits


def test_mixed_step_graph_replays_with_changing_lengths():
    # prefill rows come and go between steps; captured on a step with none
    steps = [([1, 1, 1, 1, 1, 1], [30, 70, 5, 300, 64, 9]),
             ([37, 1, 100, 1, 5, 1], [437, 700, 100, 300, 1005, 9]),
             ([2, 64, 1, 1, 130, 1], [40, 600, 17, 1200, 130, 900]),
             ([1, 1, 1, 1, 1, 1], [31, 71, 6, 301, 65, 10])]
    splits = _run_steps(7002, steps, W_d=8, W_p=6, mixed=True, min_seg=1)
    assert splits[0][1] == 0 and splits[1][1] > 0 and splits[3][1] == 0, splits


def test_cascade_graph_replays_bit_exactly():
    """fi_cascade (level 0, level 1, their split merges and the final merge)
    captured once with graph_safe and replayed: replays, with eager work and
    synchronisation between them, match the eager call bit for bit and the
    fp64 oracle of the flat batch."""
    cb = wl.shared_prefix_cascade(num_requests=24, prefix_len=640, seed=7003)
    l0, l1 = cb.level0, cb.level1
    kw = dict(page_size=l0.page_size, num_qo_heads=l0.num_qo_heads, num_kv_heads=l0.num_kv_heads,
              head_dim=l0.head_dim, workers_decode=48, workers_prefill=16, min_seg_pages=2)
    plan0 = fi.fi_plan(l0.qo_indptr, l0.kv_indptr, l0.kv_last_page_len, causal=False, **kw)
    plan1 = fi.fi_plan(l1.qo_indptr, l1.kv_indptr, l1.kv_last_page_len, causal=l1.causal, **kw)
    assert plan0.info.prefill_slots > 0 and plan1.info.decode_slots > 0  # both levels split and merge
    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32).copy()).cuda()
    dev0 = (plan0.to_device(), i32(l0.qo_indptr), i32(l0.kv_indptr), i32(l0.kv_indices), i32(l0.kv_last_page_len))
    dev1 = (plan1.to_device(), None if l1.qo_indptr is None else i32(l1.qo_indptr), i32(l1.kv_indptr),
            i32(l1.kv_indices), i32(l1.kv_last_page_len))
    q, pool = l0.q.cuda(), l0.kv_pool.cuda()

    def call(graph_safe, o, lse, ws):
        params = fi.make_params(l0.dtype, l0.dtype, l0.num_qo_heads, l0.num_kv_heads, l0.head_dim,
                                l0.page_size, l0.sm_scale, l0.soft_cap, graph_safe=graph_safe)
        fi.fi_cascade(plan0, *dev0, plan1, *dev1, params, q, pool, o, lse, ws)

    nbytes = fi.fi_cascade_workspace_bytes(plan0, plan1)
    o_g, l_g = torch.zeros_like(q), torch.zeros(q.shape[:2], dtype=torch.float32, device="cuda")
    ws_g = fi.workspace(nbytes)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(True, o_g, l_g, ws_g)
    torch.cuda.synchronize()
    o_e, l_e = torch.zeros_like(q), torch.zeros(q.shape[:2], dtype=torch.float32, device="cuda")
    ws_e = fi.workspace(nbytes)
    o_ref, l_ref = ref.attention_of(cb.flat)
    for k in range(3):
        note(f"cascade graph replay {k}")
        o_g.zero_()
        l_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        call(False, o_e, l_e, ws_e)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {k}: output differs from the eager call"
        assert torch.equal(l_g, l_e), f"replay {k}: lse differs from the eager call"
        assert_close(o_g.float().cpu(), l_g.cpu(), o_ref, l_ref, f"cascade replay {k}")
