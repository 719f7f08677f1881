"""GPU parity of the fused rotary embedding against the fp64 oracle, through
the C ABI (paper page: fused rotary embeddings among the attention variants
of its opening paragraph; "Customizable attention": query / key transforms).
Rotate-half form, key j at position j, query t at kv_len - qo_len + t.
Covered: both decode kernels (bf16 matrix-core, generic bf16 / fp32), prefill
and mixed batches, split and unsplit plans, page sizes on and off the fast
paths, causal and non-causal prefill, with soft-cap and sliding window, long
requests (large positions), and the full-size decode and mixed workloads.
The kernels round rotated q and k to the storage type before the matrix-core
products; the tolerance is the same as without the rotation."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import DeviceBatch, NUM_CUS, assert_close, note, plan_for

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def run_rope(b, theta, scale, workers_decode=None, workers_prefill=None, min_seg_pages=8,
             no_split=0, br_override=0, dev=None):
    """Run decode (qo_indptr None) or prefill with the rotary embedding on."""
    Hk = b.num_kv_heads
    wd = workers_decode or fi.fi_default_workers(fi.FI_KIND_DECODE, NUM_CUS, Hk)
    wp = workers_prefill or fi.fi_default_workers(fi.FI_KIND_PREFILL, NUM_CUS, Hk)
    plan = plan_for(b, wd, wp, min_seg_pages, no_split, br_override)
    d = dev or DeviceBatch(b)
    o = torch.full(tuple(b.q.shape), float("nan"), dtype=b.dtype, device="cuda")
    lse = torch.full(tuple(b.q.shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    ws = fi.workspace(plan.float_ws_bytes)
    params = fi.make_params(b.dtype, b.dtype, b.num_qo_heads, Hk, b.head_dim, b.page_size, b.sm_scale,
                            b.soft_cap, rope_theta=theta, rope_scale=scale)
    if b.qo_indptr is None:
        fi.fi_batch_decode_paged(plan, plan.to_device(), params, d.q, d.pool, d.kv_indptr, d.kv_indices,
                                 d.last, o, lse, ws)
    else:
        fi.fi_batch_prefill_paged(plan, plan.to_device(), params, d.q, d.pool, d.qo_indptr, d.kv_indptr,
                                  d.kv_indices, d.last, o, lse, ws)
    torch.cuda.synchronize()
    return o.float().cpu(), lse.cpu(), plan


DECODE_SWEEP = [(dt, D, G, P) for dt in ("bf16", "f32") for D in (64, 128) for G in (1, 4, 8)
                for P in (1, 16)]


@pytest.mark.parametrize("dt,D,G,P", DECODE_SWEEP)
def test_rope_decode_sweep(dt, D, G, P):
    seed = 6000 + D + 7 * G + 3 * P + (dt == "f32")
    kv = [1, 2, 15, 16, 17, 100, 333, 2500, 0, 64]
    b = wl.make_batch(seed, None, kv, page_size=P, num_qo_heads=2 * G, num_kv_heads=2, head_dim=D,
                      dtype=DTYPES[dt], decode=True, nan_poison=True)
    dev = DeviceBatch(b)
    for theta, scale in ((10000.0, 1.0), (500000.0, 8.0)):
        o_ref, l_ref = ref.attention_of(b, rope_theta=theta, rope_scale=scale)
        for wd, ms, ns in ((5, 1, 0), (1, 8, 1)):
            note(f"rope decode {dt} D={D} G={G} P={P} theta={theta} scale={scale} Wd={wd} no_split={ns}")
            o, lse, _ = run_rope(b, theta, scale, workers_decode=wd, min_seg_pages=ms, no_split=ns, dev=dev)
            assert_close(o, lse, o_ref, l_ref, f"rope decode {dt} D={D} G={G} P={P} theta={theta}")


PREFILL_SWEEP = [(D, G, P) for D in (64, 128) for G in (1, 4) for P in (3, 16)]


@pytest.mark.parametrize("D,G,P", PREFILL_SWEEP)
def test_rope_prefill_sweep(D, G, P):
    seed = 6100 + D + 11 * G + 5 * P
    rng = np.random.default_rng(seed)
    qo = [2, 17, int(rng.integers(40, 140)), 1, 0, 33, 70]
    kv = [q + int(rng.integers(0, 300)) for q in qo]
    kv[4] = 5
    for causal in (True, False):
        for cap, window in ((0.0, -1), (30.0, -1), (0.0, 60), (50.0, 100)):
            b = wl.make_batch(seed + window + int(cap), qo, kv, page_size=P, num_qo_heads=2 * G,
                              num_kv_heads=2, head_dim=D, dtype=torch.bfloat16, causal=causal,
                              nan_poison=True, soft_cap=cap, window_left=window)
            o_ref, l_ref = ref.attention_of(b, rope_theta=10000.0, rope_scale=1.0)
            dev = DeviceBatch(b)
            for wp, ms, br in ((1, 8, 0), (5, 1, 16), (7, 2, 64)):
                note(f"rope prefill D={D} G={G} P={P} causal={causal} cap={cap} w={window} Wp={wp} br={br}")
                o, lse, _ = run_rope(b, 10000.0, 1.0, workers_decode=3, workers_prefill=wp,
                                     min_seg_pages=ms, br_override=br, dev=dev)
                assert_close(o, lse, o_ref, l_ref,
                             f"rope prefill D={D} G={G} P={P} causal={causal} cap={cap} w={window} Wp={wp}")


def test_rope_llama8b_decode_full():
    b = wl.llama8b_decode(nan_poison=True)
    note("llama8b_decode, rope theta 500000, default workers")
    o, lse, _ = run_rope(b, 500000.0, 1.0)
    o_ref, l_ref = ref.attention_of(b, rope_theta=500000.0)
    assert_close(o, lse, o_ref, l_ref, "llama8b decode rope")


def test_rope_long_request_positions():
    # positions up to 131071: the angle is taken modulo one turn exactly
    b = wl.make_batch(6201, None, [131072, 4000], page_size=16, num_qo_heads=32, num_kv_heads=8,
                      head_dim=128, dtype=torch.bfloat16, decode=True)
    note("rope decode, 131072-token request")
    o, lse, _ = run_rope(b, 500000.0, 1.0, workers_decode=64, min_seg_pages=1)
    o_ref, l_ref = ref.attention_of(b, rope_theta=500000.0)
    assert_close(o, lse, o_ref, l_ref, "rope long request")


def test_rope_mixed_ragged_step_full():
    b = wl.mixed_ragged_step(nan_poison=True)
    note("mixed_ragged_step, rope theta 10000, default workers")
    o, lse, plan = run_rope(b, 10000.0, 1.0)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    note(f"mixed_ragged_step rope oracle on all {b.total_qo * b.num_qo_heads} rows")
    o_ref, l_ref = ref.attention_of(b, rope_theta=10000.0)
    assert_close(o, lse, o_ref, l_ref, "mixed rope full")


def test_rope_mixed_ragged_step_sampled():
    b = wl.mixed_ragged_step(nan_poison=True)
    note("mixed_ragged_step, rope theta 10000, default workers")
    o, lse, plan = run_rope(b, 10000.0, 1.0)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    rows = []
    for i, q in enumerate(b.qo_lens):
        for t in sorted({0, 1, q // 2, q - 2, q - 1} & set(range(q))):
            for h in range(b.num_qo_heads):
                rows.append((i, t, h))
    rows = np.array(rows, np.int32)
    note(f"mixed_ragged_step rope oracle on {len(rows)} sampled rows")
    o_ref, l_ref = ref.attention_rows_of(b, rows, rope_theta=10000.0)
    g = b.qo_indptr[rows[:, 0]] + rows[:, 1]
    assert_close(o[g, rows[:, 2]].numpy(), lse[g, rows[:, 2]].numpy(), o_ref, l_ref, "mixed rope")
