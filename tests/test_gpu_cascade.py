"""GPU parity of the cascade (shared prefix attended once per group, merged
with each request's suffix) against the flat fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attn as ref

from gpu_util import assert_close, note, run, run_cascade

pytestmark = pytest.mark.gpu


def test_shared_prefix_cascade_equals_flat():
    cb = wl.shared_prefix_cascade(nan_poison=True)
    note("cascade oracle (flat)")
    o_ref, l_ref = ref.attention_of(cb.flat)
    note("cascade gpu")
    oc, lc = run_cascade(cb)
    assert_close(oc, lc, o_ref, l_ref, "cascade vs flat oracle")
    note("flat gpu")
    of, lf, _ = run(cb.flat)
    assert_close(of, lf, o_ref, l_ref, "flat vs flat oracle")


@pytest.mark.parametrize("D,G,cap,P", [(64, 1, 0.0, 16), (128, 8, 30.0, 16), (128, 4, 0.0, 3),
                                       (64, 2, 10.0, 1)])
def test_cascade_variants(D, G, cap, P):
    prefix = 48 * P
    cb = wl.shared_prefix_cascade(num_requests=13, prefix_len=prefix, suffix_lo=0, suffix_hi=40,
                                  seed=70 + D + G, num_qo_heads=2 * G, num_kv_heads=2, head_dim=D,
                                  page_size=P, soft_cap=cap)
    o_ref, l_ref = ref.attention_of(cb.flat)
    for wd, wp, ms in ((None, None, 8), (2, 3, 1)):
        note(f"cascade D={D} G={G} cap={cap} P={P} W=({wd},{wp})")
        oc, lc = run_cascade(cb, workers_decode=wd, workers_prefill=wp, min_seg_pages=ms)
        assert_close(oc, lc, o_ref, l_ref, f"cascade D={D} G={G}")
