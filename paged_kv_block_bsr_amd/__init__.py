"""Batched attention over a paged KV cache viewed as a block-sparse-row matrix,
for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libfi.so`` (hand-written HIP kernels
plus a host-side planner); this package is its thin ctypes binding.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    FI_BF16,
    FI_F32,
    FI_KIND_DECODE,
    FI_KIND_PREFILL,
    FI_STATUS_BAD_PAGE,
    FIError,
    Plan,
    decode_plan_buffer,
    fi_append_paged_kv,
    fi_batch_decode_paged,
    fi_batch_decode_paged_noalloc,
    fi_batch_prefill_paged,
    fi_cascade,
    fi_cascade_workspace_bytes,
    fi_default_workers,
    fi_last_error,
    fi_merge_state,
    fi_plan,
    fi_plan_bounds,
    fi_read_status,
    fi_version,
    lib,
    make_params,
    tree_mask_words,
    workspace,
)
