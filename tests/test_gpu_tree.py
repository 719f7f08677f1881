"""GPU parity of the speculative-decoding tree mask (batch prefill) against
the fp64 oracle, through the C ABI.  Marked gpu: run with -m gpu on an
MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
from paged_kv_block_bsr_amd.binding import FI_ERR_UNSUPPORTED
import workloads as wl
from oracle import attn as ref

from gpu_util import DeviceBatch, assert_close, note, plan_for, run

pytestmark = pytest.mark.gpu


def _tree_batch(seed, qo, kv, P, D, G, cap=0.0, full=False):
    Hk = 2
    b = wl.make_batch(seed, qo, kv, page_size=P, num_qo_heads=Hk * G, num_kv_heads=Hk, head_dim=D,
                      dtype=torch.bfloat16, causal=True, nan_poison=True, soft_cap=cap)
    rng = np.random.default_rng(seed + 1)
    parents = [None if full else wl.random_tree_parents(rng, int(n)) for n in qo]
    if full:  # every earlier draft token: the causal mask
        parents = [np.arange(int(n)) - 1 for n in qo]
    b.tree_mask, b.mask_indptr = wl.tree_mask_bits(parents, qo)
    return b


SWEEP = [(D, G, P) for D in (64, 128) for G in (1, 4) for P in (1, 3, 16)]


@pytest.mark.parametrize("D,G,P", SWEEP)
def test_tree_mask_sweep(D, G, P):
    seed = 800 + D + 11 * G + 3 * P
    rng = np.random.default_rng(seed)
    qo = [2, 17, 1, 64, int(rng.integers(2, 100)), 5, 130]
    kv = [q + int(rng.integers(0, 300)) for q in qo]
    kv[2] = 7
    cap = 0.0 if (D + G + P) % 2 else 20.0
    b = _tree_batch(seed, qo, kv, P, D, G, cap)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wp, ms, br in ((1, 8, 0), (5, 1, 16), (9, 2, 64)):
        note(f"tree mask D={D} G={G} P={P} cap={cap} Wp={wp} br={br}")
        o, lse, _ = run(b, workers_decode=3, workers_prefill=wp, min_seg_pages=ms, br_override=br,
                        dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"tree D={D} G={G} P={P} Wp={wp} br={br}")


def test_chain_tree_mask_matches_the_causal_kernel():
    qo = [40, 3, 100]
    kv = [300, 50, 100]
    b = _tree_batch(850, qo, kv, 16, 128, 4, full=True)
    note("chain tree mask")
    o1, l1, _ = run(b, workers_prefill=6, min_seg_pages=2)
    mask, ind = b.tree_mask, b.mask_indptr
    b.tree_mask = b.mask_indptr = None
    note("causal kernel")
    o0, l0, _ = run(b, workers_prefill=6, min_seg_pages=2)
    o_ref, l_ref = ref.attention_of(b)
    assert_close(o1, l1, o_ref, l_ref, "chain tree")
    assert_close(o0, l0, o_ref, l_ref, "causal")


def test_speculative_verify_full():
    b = wl.speculative_verify(nan_poison=True)
    note("speculative_verify oracle")
    o_ref, l_ref = ref.attention_of(b)
    note("speculative_verify gpu default workers")
    o, lse, plan = run(b)
    assert plan.info.prefill_rows > 0
    assert_close(o, lse, o_ref, l_ref, "speculative_verify")
    note("speculative_verify gpu unsplit")
    o2, l2, _ = run(b, workers_prefill=64, no_split=1)
    assert_close(o2, l2, o_ref, l_ref, "speculative_verify unsplit")


def test_tree_mask_errors():
    b = _tree_batch(860, [4, 2], [10, 8], 16, 128, 4)
    d = DeviceBatch(b)
    o = torch.empty(tuple(b.q.shape), dtype=b.dtype, device="cuda")
    lse = torch.empty(tuple(b.q.shape[:2]), dtype=torch.float32, device="cuda")
    for causal, window in ((False, -1), (True, 3)):
        plan = fi.fi_plan(b.qo_indptr, b.kv_indptr, b.kv_last_page_len, page_size=16,
                          num_qo_heads=8, num_kv_heads=2, head_dim=128, causal=causal,
                          workers_decode=2, workers_prefill=2, window_left=window)
        ws = fi.workspace(plan.float_ws_bytes)
        params = fi.make_params(b.dtype, b.dtype, 8, 2, 128, 16, b.sm_scale, 0.0, tree_mask=d.mask,
                                mask_indptr=d.mask_indptr, mask_bits=d.mask_bits)
        note(f"tree mask rejected: causal={causal} window={window}")
        with pytest.raises(fi.FIError) as e:
            fi.fi_batch_prefill_paged(plan, plan.to_device(), params, d.q, d.pool, d.qo_indptr,
                                      d.kv_indptr, d.kv_indices, d.last, o, lse, ws)
        assert e.value.code == FI_ERR_UNSUPPORTED
