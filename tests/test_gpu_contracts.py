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


def _scaled_v(b, rng, big):
    """V of every page scaled to |v| ~ big, a few entries pushed to +-6e4 and
    a few to |v| < 2^-17 (below fp16's normal range), rounded to bf16; the
    oracle reads the same bf16 values."""
    v = b.kv_pool[:, 1].float()
    v = v * big
    flat = v.view(-1)
    n = flat.numel()
    hi = torch.from_numpy(rng.choice(n, n // 97, replace=False))
    flat[hi] = torch.from_numpy(rng.choice([-6.0e4, 6.0e4], hi.numel()).astype(np.float32))
    lo = torch.from_numpy(rng.choice(n, n // 89, replace=False))
    flat[lo] = torch.from_numpy((rng.standard_normal(lo.numel()) * 3e-6).astype(np.float32))
    b.kv_pool[:, 1] = v.to(b.kv_pool.dtype)
    assert b.kv_pool[:, 1].float().abs().max() <= 65504


@pytest.mark.parametrize("P", [16, 3])
def test_prefill_v_range_up_to_fp16_max(P):
    """Prefill runs P.V with V in fp16: bf16 values of V up to 65504 in
    magnitude (and tiny ones) stay within the tolerance of the oracle."""
    rng = np.random.default_rng(910 + P)
    qo = [2, 17, 70, 1, 33, 130]
    kv = [q + int(rng.integers(0, 200)) for q in qo]
    b = wl.make_batch(910 + P, qo, kv, page_size=P, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                      dtype=torch.bfloat16, causal=True)
    _scaled_v(b, rng, 1.0e4)
    o_ref, l_ref = ref.attention_of(b)
    assert np.abs(o_ref).max() > 1e3
    dev = DeviceBatch(b)
    for wp, ms in ((None, 8), (5, 1)):
        note(f"prefill with |V| up to 6e4, P={P}, Wp={wp}")
        o, lse, _ = run(b, workers_decode=3, workers_prefill=wp, min_seg_pages=ms, dev=dev)
        assert_close(o, lse, o_ref, l_ref, f"large V, P={P}, Wp={wp}")


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
