"""GPU parity of batch decode (and the merge kernels) against the fp64 oracle,
through the C ABI.  Marked gpu: run with -m gpu on an MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import DeviceBatch, assert_close, note, run

pytestmark = pytest.mark.gpu


def test_tiny_decode_fp32_unsplit_and_split():
    b = wl.tiny_decode_fp32(nan_poison=True)
    o_ref, l_ref = ref.attention_of(b)
    for wd, ms, ns in ((1, 8, 1), (1, 8, 0), (8, 1, 0), (3, 2, 0)):
        note(f"tiny_decode_fp32 W={wd} min_seg={ms} no_split={ns}")
        o, lse, plan = run(b, workers_decode=wd, min_seg_pages=ms, no_split=ns)
        assert_close(o, lse, o_ref, l_ref, f"tiny W={wd}")
        if wd == 8:
            assert plan.info.decode_slots > 0  # the split path really ran


def test_llama8b_decode_full():
    b = wl.llama8b_decode()
    note("llama8b_decode oracle")
    o_ref, l_ref = ref.attention_of(b)
    note("llama8b_decode gpu default workers")
    o, lse, plan = run(b)
    assert_close(o, lse, o_ref, l_ref, "llama8b_decode")
    note("llama8b_decode gpu unsplit")
    o2, lse2, _ = run(b, workers_decode=64, no_split=1)
    assert_close(o2, lse2, o_ref, l_ref, "llama8b_decode unsplit")


def test_skewed_long_decode_full():
    b = wl.skewed_long_decode()
    note("skewed_long_decode oracle")
    o_ref, l_ref = ref.attention_of(b)
    note("skewed_long_decode gpu")
    o, lse, plan = run(b)
    assert plan.info.decode_slots >= 50  # the long request is split many ways
    assert_close(o, lse, o_ref, l_ref, "skewed_long_decode")


SWEEP = []
for _dt in (torch.float32, torch.bfloat16):
    for _D in (64, 128):
        for _G in (1, 2, 4, 8):
            for _P in (1, 3, 16, 32):
                SWEEP.append((_dt, _D, _G, _P))


@pytest.mark.parametrize("dt,D,G,P", SWEEP)
def test_decode_sweep(dt, D, G, P):
    seed = 100 + D + 7 * G + 13 * P + (0 if dt == torch.float32 else 1)
    rng = np.random.default_rng(seed)
    kv = [0, 1, max(P - 1, 1), P, P + 1, 2 * P + 3, int(rng.integers(1, 300)), int(rng.integers(1, 300))]
    Hk = 2
    cap = 0.0 if (G + P) % 2 else 20.0
    b = wl.make_batch(seed, None, kv, page_size=P, num_qo_heads=Hk * G, num_kv_heads=Hk,
                      head_dim=D, dtype=dt, decode=True, nan_poison=True, soft_cap=cap)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wd, ms in ((1, 8), (5, 1)):
        note(f"decode sweep dt={dt} D={D} G={G} P={P} W={wd}")
        o, lse, _ = run(b, workers_decode=wd, min_seg_pages=ms, dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"sweep {dt} D={D} G={G} P={P} W={wd}")


def test_decode_bf16_in_f32_out_and_no_lse():
    b = wl.make_batch(9, None, [5, 40, 333], page_size=16, num_qo_heads=8, num_kv_heads=2,
                      head_dim=128, dtype=torch.bfloat16, decode=True)
    o_ref, l_ref = ref.attention_of(b)
    note("bf16 in, f32 out")
    o, lse, _ = run(b, workers_decode=4, min_seg_pages=1, out_dtype=torch.float32)
    assert_close(o, lse, o_ref, l_ref, "f32 out")
    o, _, _ = run(b, workers_decode=4, min_seg_pages=1, with_lse=False)
    assert_close(o, None, o_ref, l_ref, "no lse")


def test_page_permutation_is_bit_exact_for_a_fixed_plan():
    b = wl.make_batch(11, None, [70, 3, 129, 16], page_size=16, num_qo_heads=16, num_kv_heads=4,
                      head_dim=128, dtype=torch.bfloat16, decode=True)
    note("page permutation: base")
    o1, l1, _ = run(b, workers_decode=3, min_seg_pages=2)
    rng = np.random.default_rng(3)
    sigma = rng.permutation(b.pool_pages)
    pool2 = torch.empty_like(b.kv_pool)
    pool2[torch.from_numpy(sigma)] = b.kv_pool
    b.kv_pool = pool2
    b.kv_indices = sigma[b.kv_indices].astype(np.int32)
    note("page permutation: permuted")
    o2, l2, _ = run(b, workers_decode=3, min_seg_pages=2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_merge_state_two_way(dt):
    rng = np.random.default_rng(12)
    n, h, d = 37, 8, 128
    va = torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32)).to(dt)
    vb = torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32)).to(dt)
    sa = torch.from_numpy(rng.standard_normal((n, h), dtype=np.float32) * 3)
    sb = torch.from_numpy(rng.standard_normal((n, h), dtype=np.float32) * 3)
    sa[0, :] = -float("inf")
    sa[1, :] = -float("inf")
    sb[1, :] = -float("inf")
    eo, el = ref.merge_states(torch.stack([va, vb]), torch.stack([sa, sb]))
    dva, dvb, dsa, dsb = va.cuda(), vb.cuda(), sa.cuda(), sb.cuda()
    vo = torch.empty_like(dva)
    so = torch.empty_like(dsa)
    note(f"merge_state {dt}")
    fi.fi_merge_state(dva, dsa, dvb, dsb, vo, so)
    torch.cuda.synchronize()
    assert_close(vo.float().cpu(), so.cpu(), eo, el, "merge_state")
    # in place into the first state
    fi.fi_merge_state(dva, dsa, dvb, dsb, dva, dsa)
    torch.cuda.synchronize()
    assert_close(dva.float().cpu(), dsa.cpu(), eo, el, "merge_state in place")


def test_long_items_reload_page_ids():
    """Few workers over a long request: each wave walks more than 64 chunks,
    so the per-wave page-id vector is reloaded mid-item."""
    b = wl.make_batch(13, None, [40000, 700, 5], page_size=16, num_qo_heads=32, num_kv_heads=8,
                      head_dim=128, dtype=torch.bfloat16, decode=True)
    o_ref, l_ref = ref.attention_of(b)
    for wd in (1, 2):
        note(f"long items W={wd}")
        o, lse, _ = run(b, workers_decode=wd, min_seg_pages=1)
        assert_close(o, lse, o_ref, l_ref, f"long items W={wd}")


# Pages of 1, 2, 4 or 8 tokens (bf16): the matrix-core decode kernel looks up
# one page per token instead of one per 16-token chunk.
SMALL_PAGES = [(D, G, P) for D in (64, 128) for G in (1, 2, 4, 8) for P in (2, 4, 8)]


@pytest.mark.parametrize("D,G,P", SMALL_PAGES)
def test_decode_small_pages_sweep(D, G, P):
    seed = 500 + D + 7 * G + 13 * P
    rng = np.random.default_rng(seed)
    kv = [0, 1, P - 1, P, P + 1, 15, 16, 17, 2 * P + 3, int(rng.integers(1, 400)), int(rng.integers(1, 400))]
    Hk = 2
    cap = 0.0 if (G + P) % 2 else 20.0
    b = wl.make_batch(seed, None, kv, page_size=P, num_qo_heads=Hk * G, num_kv_heads=Hk,
                      head_dim=D, dtype=torch.bfloat16, decode=True, nan_poison=True, soft_cap=cap)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wd, ms in ((1, 8), (5, 1), (3, 64)):
        note(f"small-page decode D={D} G={G} P={P} W={wd} min_seg={ms}")
        o, lse, _ = run(b, workers_decode=wd, min_seg_pages=ms, dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"small pages D={D} G={G} P={P} W={wd}")


def test_llama8b_decode_page_size_1_full():
    """The Llama-3-8B decode batch stored one token per page (column-vector
    BSR), split and unsplit, against the oracle at full size."""
    rng = np.random.default_rng(1002)
    kv = rng.integers(512, 4096, size=64, endpoint=True)
    b = wl.make_batch(1002, None, kv, page_size=1, decode=True, nan_poison=True)
    note("llama8b decode P=1 oracle")
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    note("llama8b decode P=1 gpu default workers")
    o, lse, plan = run(b, dev=dev)
    assert plan.info.decode_slots > 0
    assert_close(o, lse, o_ref, l_ref, "llama8b P=1")
    note("llama8b decode P=1 gpu unsplit")
    o2, lse2, _ = run(b, workers_decode=64, no_split=1, dev=dev)
    assert_close(o2, lse2, o_ref, l_ref, "llama8b P=1 unsplit")


def test_page_permutation_is_bit_exact_with_one_token_pages():
    b = wl.make_batch(17, None, [70, 3, 129, 16, 1000], page_size=1, num_qo_heads=16, num_kv_heads=4,
                      head_dim=128, dtype=torch.bfloat16, decode=True)
    note("page permutation P=1: base")
    o1, l1, _ = run(b, workers_decode=3, min_seg_pages=40)
    rng = np.random.default_rng(4)
    sigma = rng.permutation(b.pool_pages)
    pool2 = torch.empty_like(b.kv_pool)
    pool2[torch.from_numpy(sigma)] = b.kv_pool
    b.kv_pool = pool2
    b.kv_indices = sigma[b.kv_indices].astype(np.int32)
    note("page permutation P=1: permuted")
    o2, l2, _ = run(b, workers_decode=3, min_seg_pages=40)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_small_pages_many_items_per_worker():
    """Many short requests on few workers: every worker runs a chain of items,
    so the page ids of each next item are fetched during the one before."""
    rng = np.random.default_rng(19)
    kv = rng.integers(1, 200, size=300)
    b = wl.make_batch(19, None, kv, page_size=1, num_qo_heads=32, num_kv_heads=8,
                      head_dim=128, dtype=torch.bfloat16, decode=True, nan_poison=True)
    o_ref, l_ref = ref.attention_of(b)
    dev = DeviceBatch(b)
    for wd, ms, ns in ((4, 8, 0), (7, 300, 0), (5, 8, 1)):
        note(f"small pages many items W={wd} min_seg={ms} no_split={ns}")
        o, lse, _ = run(b, workers_decode=wd, min_seg_pages=ms, no_split=ns, dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"many items W={wd}")
