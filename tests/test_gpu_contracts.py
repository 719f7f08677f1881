"""GPU checks of the library's own contracts (header fi.h), beyond parity
with the method: the numeric range of V on the prefill path, and the status
word that reports page ids outside the pool."""
import numpy as np
import pytest
import torch

import paged_kv_block_bsr_amd as fi
import workloads as wl
from oracle import attn as ref

from gpu_util import DeviceBatch, assert_close, note, run

pytestmark = pytest.mark.gpu


def _with_v_scaled(b, factor, clamp=None):
    """The batch with every V element times `factor` (a power of two, so bf16
    holds the products exactly); with `clamp`, V is then clamped to +-clamp
    and the pool kept in float64 (+-65504 is not a bf16 value), for the
    oracle only."""
    import copy
    c = copy.copy(b)
    if clamp is not None:
        pool = b.kv_pool.double()
        pool[:, 1] = (pool[:, 1] * factor).clamp(-clamp, clamp)
        c.kv_pool = pool
        return c
    pool = b.kv_pool.clone()
    v = pool[:, 1].float() * factor
    pool[:, 1] = v.to(pool.dtype)
    got = pool[:, 1].float()
    assert bool(((got == v) | (got.isnan() & v.isnan())).all()), "scaled V must be exact in bf16"
    c.kv_pool = pool
    return c


@pytest.mark.parametrize("P", [16, 3])
def test_prefill_carries_v_exactly_up_to_fp16_max(P):
    """V enters the prefill P.V product as fp16.  Every step applied to V is
    linear, so scaling V by 2^13 (|V| up to ~4e4 <= 65504, exact in fp16)
    must scale o by exactly 2^13 and leave lse unchanged, bit for bit, while
    the unscaled batch matches the oracle.  Scaled by 2^15, some |V| exceed
    65504 and are clamped to +-65504 (the documented range): the output then
    matches the oracle on V clamped to +-65504, within the bar scaled by 2^15
    (rows of single-query requests run in the decode kernel, which keeps bf16
    V exact: they match the oracle on the unclamped V)."""
    rng = np.random.default_rng(910 + P)
    qo = [2, 17, 70, 1, 33, 130]
    kv = [q + int(rng.integers(0, 200)) for q in qo]
    b = wl.make_batch(910 + P, qo, kv, page_size=P, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                      dtype=torch.bfloat16, causal=True, nan_poison=True)
    o_ref, l_ref = ref.attention_of(b)
    for wp, ms in ((None, 8), (5, 1)):
        note(f"prefill P={P} Wp={wp}: unit-scale V")
        o, lse, _ = run(b, workers_decode=3, workers_prefill=wp, min_seg_pages=ms)
        assert_close(o, lse, o_ref, l_ref, f"unit V, P={P}, Wp={wp}")
        big = _with_v_scaled(b, 2.0 ** 13)
        vmax = float(torch.nan_to_num(big.kv_pool[:, 1].float(), nan=0.0).abs().max())
        assert 16384 < vmax <= 65504
        note(f"prefill P={P} Wp={wp}: V x 2^13 (max |V| {vmax:.0f})")
        o13, l13, _ = run(big, workers_decode=3, workers_prefill=wp, min_seg_pages=ms)
        assert torch.equal(o13, o * 2.0 ** 13), "o must scale exactly with V"
        assert torch.equal(l13, lse), "lse must not depend on V"
        over = _with_v_scaled(b, 2.0 ** 15)
        note(f"prefill P={P} Wp={wp}: V x 2^15, some |V| > 65504")
        o15, l15, _ = run(over, workers_decode=3, workers_prefill=wp, min_seg_pages=ms)
        # prefill rows (requests with >= 2 queries) see V clamped to +-65504;
        # decode rows run in the decode kernel, whose P.V keeps bf16 V exact
        s = 2.0 ** 15
        clamped = _with_v_scaled(b, s, clamp=65504.0)
        exact = _with_v_scaled(b, s, clamp=float("inf"))
        pre = np.repeat(b.qo_lens >= 2, b.qo_lens)
        oc_ref, lc_ref = ref.attention_of(clamped)
        oe_ref, le_ref = ref.attention_of(exact)
        assert_close(o15[pre] / s, l15[pre], oc_ref[pre] / s, lc_ref[pre], f"V x 2^15, prefill rows, P={P}")
        assert_close(o15[~pre] / s, l15[~pre], oe_ref[~pre] / s, le_ref[~pre], f"V x 2^15, decode rows, P={P}")


def _with_bad_ids(b, entries):
    """A copy of the batch's page table with kv_indices[e] = id for (e, id)."""
    idx = b.kv_indices.copy()
    for e, page in entries:
        idx[e] = page
    return idx


@pytest.mark.parametrize("kind,P,dtype", [("decode", 16, torch.bfloat16), ("decode", 4, torch.bfloat16),
                                          ("decode", 3, torch.bfloat16), ("decode", 16, torch.float32),
                                          ("prefill", 16, torch.bfloat16), ("prefill", 3, torch.bfloat16)])
def test_out_of_pool_page_ids_set_the_status_word(kind, P, dtype):
    """A page id at or past pool_pages (or negative) is read as page 0 -- never
    outside the pool -- and sets FI_STATUS_BAD_PAGE in the workspace's status
    word; requests with valid page tables are unaffected, and a later call
    with clean page tables leaves the cleared word at 0."""
    rng = np.random.default_rng(930 + P)
    kv = [40, 3 * P + 5, 60, 17]
    qo = [1, 1, 1, 1] if kind == "decode" else [3, 1, 9, 2]
    D = 64 if dtype == torch.float32 else 128
    b = wl.make_batch(930 + P, None if kind == "decode" else qo, kv, page_size=P, num_qo_heads=8,
                      num_kv_heads=2, head_dim=D, dtype=dtype, causal=True, decode=kind == "decode")
    clean = DeviceBatch(b)
    dev = DeviceBatch(b)
    bad_req = 1
    e0 = int(b.kv_indptr[bad_req])
    dev.kv_indices = torch.from_numpy(_with_bad_ids(b, [(e0, b.kv_pool.shape[0] + 7), (e0 + 1, -3)])).cuda()
    ws = fi.workspace(64 << 20)
    note(f"{kind} P={P} {dtype}: two out-of-pool page ids in request {bad_req}")
    o, lse, _ = run(b, workers_decode=3, workers_prefill=2, min_seg_pages=1, dev=dev, ws=ws)
    status = fi.fi_read_status(ws, clear=True)
    assert status & fi.FI_STATUS_BAD_PAGE
    assert fi.fi_read_status(ws) == 0
    assert torch.isfinite(o).all()
    o_ref, l_ref = ref.attention_of(b)
    rows = np.ones(b.total_qo, bool)
    if kind == "decode":
        rows[bad_req] = False
    else:
        rows[b.qo_indptr[bad_req]:b.qo_indptr[bad_req + 1]] = False
    assert_close(o[rows], lse[rows], o_ref[rows], l_ref[rows], f"{kind} P={P} rows with valid pages")
    note(f"{kind} P={P}: the same batch with its page table intact")
    o, lse, _ = run(b, workers_decode=3, workers_prefill=2, min_seg_pages=1, dev=clean, ws=ws)
    assert fi.fi_read_status(ws) == 0
    assert_close(o, lse, o_ref, l_ref, f"{kind} P={P} clean")
