"""GPU parity of sliding-window attention against the fp64 oracle, through the
C ABI.  The query at position p = kv_len - qo_len + t sees no key before
p - window_left (paper page: sliding windows among the attention variants of
its opening paragraph; "Customizable attention": a variant is a mask over the
logits).  Covered: both decode kernels (bf16 matrix-core, generic bf16 / fp32),
prefill and mixed batches, split and unsplit plans, soft-cap, page sizes on
and off the fast paths, causal and non-causal prefill, windows from 0 keys to
longer than every request, and the full-size decode and mixed workloads."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import DeviceBatch, assert_close, note, run

pytestmark = pytest.mark.gpu

DECODE_SWEEP = [(dt, D, G, P) for dt in ("bf16", "f32") for D in (64, 128) for G in (1, 4, 8)
                for P in (1, 16)]
DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("dt,D,G,P", DECODE_SWEEP)
def test_window_decode_sweep(dt, D, G, P):
    seed = 5000 + D + 7 * G + 3 * P + (dt == "f32")
    kv = [1, 2, 15, 16, 17, 100, 333, 1000, 0, 64]
    Hk = 2
    b = wl.make_batch(seed, None, kv, page_size=P, num_qo_heads=Hk * G, num_kv_heads=Hk,
                      head_dim=D, dtype=DTYPES[dt], decode=True, nan_poison=True)
    dev = DeviceBatch(b)
    for window in (0, 1, 15, 16, 100, 5000):
        b.window_left = window
        o_ref, l_ref = ref.attention_of(b)
        for wd, ms, ns in ((5, 1, 0), (1, 8, 1)):
            note(f"window decode {dt} D={D} G={G} P={P} w={window} Wd={wd} no_split={ns}")
            o, lse, _ = run(b, workers_decode=wd, min_seg_pages=ms, no_split=ns, dev=dev)
            assert_close(o, lse, o_ref, l_ref, f"window decode {dt} D={D} G={G} P={P} w={window}")


PREFILL_SWEEP = [(D, G, P) for D in (64, 128) for G in (1, 4) for P in (3, 16)]


@pytest.mark.parametrize("D,G,P", PREFILL_SWEEP)
def test_window_prefill_sweep(D, G, P):
    seed = 5100 + D + 11 * G + 5 * P
    rng = np.random.default_rng(seed)
    qo = [2, 17, int(rng.integers(40, 140)), 1, 0, 33, 70]
    kv = [q + int(rng.integers(0, 300)) for q in qo]
    kv[4] = 5
    Hk = 2
    for causal in (True, False):
        cap = 30.0 if causal and P == 16 else 0.0
        for window in (0, 5, 63, 64, 200, 5000):
            b = wl.make_batch(seed + window, qo, kv, page_size=P, num_qo_heads=Hk * G,
                              num_kv_heads=Hk, head_dim=D, dtype=torch.bfloat16, causal=causal,
                              nan_poison=True, soft_cap=cap, window_left=window)
            o_ref, l_ref = ref.attention_of(b)
            dev = DeviceBatch(b)
            for wp, ms, br in ((1, 8, 0), (5, 1, 16), (7, 2, 64)):
                note(f"window prefill D={D} G={G} P={P} causal={causal} cap={cap} w={window} "
                     f"Wp={wp} br={br}")
                o, lse, _ = run(b, workers_decode=3, workers_prefill=wp, min_seg_pages=ms,
                                br_override=br, dev=dev)
                assert_close(o, lse, o_ref, l_ref,
                             f"window prefill D={D} G={G} P={P} causal={causal} w={window} Wp={wp}")


def test_window_longer_than_every_request_is_bit_exact_without_one():
    """A window no request reaches hides nothing: the windowed kernels give
    the same bits as the ones without a window."""
    qo = [64, 1, 130, 7, 1, 300, 2, 1]
    kv = [64 + 500, 900, 130, 7 + 33, 17, 300 + 1200, 2, 3000]
    kw = dict(page_size=16, num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.bfloat16,
              causal=True)
    b0 = wl.make_batch(61, qo, kv, **kw)
    b1 = wl.make_batch(61, qo, kv, window_left=max(kv), **kw)
    dev = DeviceBatch(b0)
    for wd, wp, ms in ((None, None, 8), (3, 5, 1)):
        note(f"window >= kv_len vs none, W=({wd},{wp})")
        o0, l0, _ = run(b0, workers_decode=wd, workers_prefill=wp, min_seg_pages=ms, dev=dev)
        o1, l1, p1 = run(b1, workers_decode=wd, workers_prefill=wp, min_seg_pages=ms, dev=dev)
        assert p1.buf[52] == max(kv)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_window_llama8b_decode_full():
    b = wl.llama8b_decode(nan_poison=True)
    b.window_left = 1023
    note("llama8b_decode, window 1023, default workers")
    o, lse, plan = run(b)
    # pages outside every window are dropped from the plan
    assert sum(r[3] for r in fi.decode_plan_buffer(plan.buf)["decode"]["rows"]) <= 64 * (1024 // 16 + 1)
    o_ref, l_ref = ref.attention_of(b)
    assert_close(o, lse, o_ref, l_ref, "llama8b decode window 1023")


def test_window_mixed_ragged_step_full():
    b = wl.mixed_ragged_step(nan_poison=True)
    b.window_left = 1023
    note("mixed_ragged_step, window 1023, default workers")
    o, lse, plan = run(b)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    note(f"mixed_ragged_step window oracle on all {b.total_qo * b.num_qo_heads} rows")
    o_ref, l_ref = ref.attention_of(b)
    assert_close(o, lse, o_ref, l_ref, "mixed_ragged_step window 1023 full")


def test_window_mixed_ragged_step_sampled():
    b = wl.mixed_ragged_step(nan_poison=True)
    b.window_left = 1023
    note("mixed_ragged_step, window 1023, default workers")
    o, lse, plan = run(b)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rows = []
    for i, q in enumerate(b.qo_lens):
        for t in sorted({0, 1, q // 2, q - 2, q - 1} & set(range(q))):
            for h in range(b.num_qo_heads):
                rows.append((i, t, h))
    rows = np.array(rows, np.int32)
    note(f"mixed_ragged_step window oracle on {len(rows)} sampled rows")
    o_ref, l_ref = ref.attention_rows_of(b, rows)
    g = b.qo_indptr[rows[:, 0]] + rows[:, 1]
    assert_close(o[g, rows[:, 2]].numpy(), lse[g, rows[:, 2]].numpy(), o_ref, l_ref,
                 "mixed_ragged_step window 1023")
