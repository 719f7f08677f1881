"""GPU test of the allocation-free decode entry point
(fi_batch_decode_paged_noalloc): two calls in a row, the second on a smaller
batch, each against fi_batch_decode_paged with a caller workspace on the
same inputs (bit for bit: same plan, same kernels) and against the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import NUM_CUS, DeviceBatch, assert_close, note, plan_for

pytestmark = pytest.mark.gpu


def _decode_both(b, workers, min_seg_pages):
    plan = plan_for(b, workers, 1, min_seg_pages)
    d = DeviceBatch(b)
    plan_dev = plan.to_device()
    params = fi.make_params(b.dtype, b.dtype, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.page_size,
                            b.sm_scale, b.soft_cap)
    outs = []
    for kind in ("workspace", "noalloc"):
        o = torch.full(tuple(b.q.shape), float("nan"), dtype=b.dtype, device="cuda")
        lse = torch.full(tuple(b.q.shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
        note(f"{kind} decode: {b.batch_size} requests, {workers} workers, "
             f"{plan.info.decode_slots} partial slots")
        if kind == "workspace":
            ws = fi.workspace(plan.float_ws_bytes)
            fi.fi_batch_decode_paged(plan, plan_dev, params, d.q, d.pool, d.kv_indptr, d.kv_indices, d.last,
                                     o, lse, ws)
        else:
            fi.fi_batch_decode_paged_noalloc(plan, plan_dev, params, d.q, d.pool, d.kv_indptr, d.kv_indices,
                                             d.last, o, lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    return outs, plan


def test_noalloc_decode_equals_the_workspace_call_on_two_calls():
    b1 = wl.llama8b_decode(nan_poison=True)
    b2 = wl.make_batch(31, None, [5, 700, 64, 1, 2100, 33], page_size=16, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, dtype=torch.bfloat16, decode=True, nan_poison=True)
    wd = fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, 8)
    for b, workers, ms in ((b1, wd, 8), (b2, 16, 1)):
        outs, plan = _decode_both(b, workers, ms)
        (ow, lw), (on, ln) = outs
        assert plan.info.decode_slots > 0, "the case must exercise the partial slots"
        assert torch.equal(on, ow) and torch.equal(ln, lw), f"{b.batch_size} requests: differs from the workspace call"
        o_ref, l_ref = ref.attention_of(b)
        assert_close(on.float(), ln, o_ref, l_ref, f"noalloc decode, {b.batch_size} requests")
    assert fi.fi_read_status(None) == 0


def test_noalloc_refuses_plans_larger_than_its_scratch():
    b = wl.make_batch(32, None, [100, 200], page_size=16, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                      dtype=torch.bfloat16, decode=True)
    plan = plan_for(b, 600, 1, 1)   # 1198 slots x 32 heads x 128 dims x 4 B > 16 MiB
    d = DeviceBatch(b)
    params = fi.make_params(b.dtype, b.dtype, 32, 8, 128, 16, b.sm_scale)
    o = torch.empty_like(d.q)
    with pytest.raises(fi.FIError) as e:
        fi.fi_batch_decode_paged_noalloc(plan, plan.to_device(), params, d.q, d.pool, d.kv_indptr, d.kv_indices,
                                         d.last, o, None)
    assert e.value.code == fi.binding.FI_ERR_WORKSPACE_TOO_SMALL and "scratch" in str(e.value)
