"""GPU parity of ragged causal batch prefill (and mixed prefill + decode
batches) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import DeviceBatch, assert_close, note, run

pytestmark = pytest.mark.gpu


def _rows_for(b, tokens_per_req=None):
    """Sampled (request, token, head) rows: first, second, middle and last two
    tokens of each request, every head."""
    rows = []
    for i, qo in enumerate(b.qo_lens):
        toks = sorted({0, 1, qo // 2, qo - 2, qo - 1} & set(range(qo))) if tokens_per_req is None else range(qo)
        for t in toks:
            for h in range(b.num_qo_heads):
                rows.append((i, t, h))
    return np.array(rows, np.int32)


def _gather(o, lse, b, rows):
    g = b.qo_indptr[rows[:, 0]] + rows[:, 1]
    return o[g, rows[:, 2]].numpy(), lse[g, rows[:, 2]].numpy()


def test_mixed_ragged_step_sampled():
    b = wl.mixed_ragged_step(nan_poison=True)
    note("mixed_ragged_step gpu")
    o, lse, plan = run(b)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rows = _rows_for(b)
    note(f"mixed_ragged_step oracle on {len(rows)} sampled rows")
    o_ref, l_ref = ref.attention_rows_of(b, rows)
    og, lg = _gather(o, lse, b, rows)
    assert_close(og, lg, o_ref, l_ref, "mixed_ragged_step")


def test_mixed_ragged_step_full():
    """Every (token, head) row of the mixed step -- 16 causal prefills and 48
    decodes in one call -- against the oracle."""
    b = wl.mixed_ragged_step(nan_poison=True)
    note("mixed_ragged_step gpu, default workers")
    o, lse, plan = run(b)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    note(f"mixed_ragged_step oracle on all {b.total_qo * b.num_qo_heads} rows")
    o_ref, l_ref = ref.attention_of(b)
    assert_close(o, lse, o_ref, l_ref, "mixed_ragged_step full")


def test_mixed_ragged_step_page_size_1_full():
    """The mixed step stored one token per page (the column-vector layout),
    every row against the oracle."""
    m = wl.mixed_ragged_step()
    b = wl.make_batch(1004, m.qo_lens, m.kv_lens, page_size=1, nan_poison=True)
    note("mixed step P=1 gpu")
    o, lse, plan = run(b)
    assert plan.info.prefill_rows > 0 and plan.info.decode_rows == 48
    note(f"mixed step P=1 oracle on all {b.total_qo * b.num_qo_heads} rows")
    o_ref, l_ref = ref.attention_of(b)
    assert_close(o, lse, o_ref, l_ref, "mixed P=1 full")


def test_mixed_medium_full():
    qo = [64, 1, 130, 7, 1, 300, 2, 1]
    kv = [64 + 500, 900, 130, 7 + 33, 17, 300 + 1200, 2, 3000]
    b = wl.make_batch(21, qo, kv, page_size=16, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                      dtype=torch.bfloat16, causal=True, nan_poison=True)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wd, wp, ms in ((None, None, 8), (3, 5, 1), (1, 1, 8)):
        note(f"mixed medium W=({wd},{wp}) min_seg={ms}")
        o, lse, _ = run(b, workers_decode=wd, workers_prefill=wp, min_seg_pages=ms, dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"mixed medium W=({wd},{wp})")


SWEEP = [(D, G, P) for D in (64, 128) for G in (1, 2, 4, 8) for P in (1, 3, 16)]


@pytest.mark.parametrize("D,G,P", SWEEP)
def test_prefill_sweep(D, G, P):
    seed = 300 + D + 11 * G + 5 * P
    rng = np.random.default_rng(seed)
    causal = (G + P) % 2 == 0
    cap = 0.0 if (D + G) % 3 else 25.0
    qo = [2, 17, int(rng.integers(2, 90)), 1, 0, 33]
    kv = [q + int(rng.integers(0, 70)) for q in qo]
    kv[4] = 5
    Hk = 2
    b = wl.make_batch(seed, qo, kv, page_size=P, num_qo_heads=Hk * G, num_kv_heads=Hk, head_dim=D,
                      dtype=torch.bfloat16, causal=causal, nan_poison=True, soft_cap=cap)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wp, ms, br in ((1, 8, 0), (4, 1, 16), (7, 2, 64)):
        note(f"prefill sweep D={D} G={G} P={P} causal={causal} cap={cap} Wp={wp} br={br}")
        o, lse, _ = run(b, workers_decode=3, workers_prefill=wp, min_seg_pages=ms, br_override=br,
                        dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"prefill D={D} G={G} P={P} Wp={wp} br={br}")


@pytest.mark.parametrize("P", [2, 5, 7, 8, 12, 100])
def test_prefill_page_sizes(P):
    """The general page path divides key positions by P with a multiply-high
    and a shift (magic numbers from the host), for powers of two below 16
    and for other sizes alike."""
    seed = 700 + P
    rng = np.random.default_rng(seed)
    qo = [2, 17, int(rng.integers(2, 90)), 1, 0, 33, 130]
    kv = [q + int(rng.integers(0, 3 * P + 70)) for q in qo]
    kv[4] = 5
    b = wl.make_batch(seed, qo, kv, page_size=P, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, nan_poison=True)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wp, ms in ((1, 8), (5, 1)):
        note(f"prefill page size P={P} Wp={wp}")
        o, lse, _ = run(b, workers_decode=3, workers_prefill=wp, min_seg_pages=ms, dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"prefill P={P} Wp={wp}")


def test_prefill_non_causal_empty_cache_and_f32_out():
    b = wl.make_batch(41, [5, 40, 3], [0, 77, 9], page_size=16, num_qo_heads=8, num_kv_heads=2,
                      head_dim=128, dtype=torch.bfloat16, causal=False)
    o_ref, l_ref = ref.attention_of(b)
    note("non-causal prefill with an empty request, f32 out")
    o, lse, _ = run(b, workers_decode=2, workers_prefill=3, min_seg_pages=1,
                    out_dtype=torch.float32)
    assert_close(o, lse, o_ref, l_ref, "non-causal")
    assert torch.all(o[:5] == 0) and torch.all(torch.isneginf(lse[:5]))


def test_prefill_split_equals_unsplit():
    b = wl.make_batch(42, [256, 100], [2000, 1900], page_size=16, num_qo_heads=32,
                      num_kv_heads=8, head_dim=128, dtype=torch.bfloat16, causal=True)
    dev = DeviceBatch(b)
    note("prefill unsplit")
    o1, l1, p1 = run(b, workers_decode=1, workers_prefill=8, no_split=1, dev=dev)
    note("prefill split")
    o2, l2, p2 = run(b, workers_decode=1, workers_prefill=64, min_seg_pages=1, dev=dev)
    assert p1.info.prefill_slots == 0 and p2.info.prefill_slots > 0
    assert_close(o2, l2, o1.numpy(), l1.numpy().astype(np.float64), "split vs unsplit")
    rows = _rows_for(b)
    o_ref, l_ref = ref.attention_rows_of(b, rows)
    og, lg = _gather(o2, l2, b, rows)
    assert_close(og, lg, o_ref, l_ref, "split vs oracle")


def test_prefill_rejects_fp32_tiles():
    b = wl.make_batch(43, [4], [9], page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=64,
                      dtype=torch.float32, causal=True)
    with pytest.raises(fi.FIError) as e:
        run(b, workers_decode=1, workers_prefill=1)
    assert e.value.code == fi.binding.FI_ERR_UNSUPPORTED


def test_fp32_batch_of_single_queries_through_prefill_call():
    b = wl.make_batch(44, [1, 1, 0, 1], [9, 40, 3, 1], page_size=16, num_qo_heads=8,
                      num_kv_heads=2, head_dim=64, dtype=torch.float32, causal=True)
    o_ref, l_ref = ref.attention_of(b)
    note("fp32 single-query rows through fi_batch_prefill_paged")
    o, lse, _ = run(b, workers_decode=2, workers_prefill=2, min_seg_pages=1)
    assert_close(o, lse, o_ref, l_ref, "fp32 prefill call")


def test_prefill_repeats_bit_exactly_with_two_workgroups_per_cu():
    """64 tiles on 64 workers x 8 KV heads: 512 busy workgroups, two per CU.
    Repeated calls give identical bits (the kernel reads no matrix-core
    result before the wait states that must follow an MFMA, whatever the
    other wave on the SIMD does)."""
    b = wl.make_batch(71, [256] * 8, [1024 + 256] * 8, page_size=16, num_qo_heads=32,
                      num_kv_heads=8, head_dim=128, dtype=torch.bfloat16, causal=True)
    dev = DeviceBatch(b)
    outs = []
    for k in range(4):
        note(f"repeat {k}: 512 busy prefill workgroups")
        o, lse, plan = run(b, workers_decode=1, workers_prefill=64, no_split=1, dev=dev)
        outs.append((o, lse))
    assert plan.info.prefill_items == 64
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    rows = _rows_for(b)
    o_ref, l_ref = ref.attention_rows_of(b, rows)
    og, lg = _gather(outs[0][0], outs[0][1], b, rows)
    assert_close(og, lg, o_ref, l_ref, "512 busy workgroups")
