// prefill.hip -- launches of the batch-prefill kernel (prefill_kernel.h):
// the kernels without a sliding window or rotary embedding are built here,
// the windowed ones in prefill_window.hip, the rotary ones in prefill_rope.hip.
#include "prefill_kernel.h"

namespace fi {

int launch_prefill(const RunArgs& r) {
  if (r.dtype != FI_BF16)
    return set_error(FI_ERR_UNSUPPORTED, "prefill tiles need bf16 q / kv (fp32 runs decode rows only)");
  if ((int64_t)4 * r.P * r.Hk * r.D >= ((int64_t)1 << 32))
    return set_error(FI_ERR_UNSUPPORTED, "prefill: one page of the pool must stay below 4 GiB");
  const bool pow2_16 = r.P >= 16 && (r.P & (r.P - 1)) == 0;
  if (!pow2_16 && (uint64_t)2 * (uint64_t)r.pool_pages * (uint64_t)r.P >= ((uint64_t)1 << 32))
    return set_error(FI_ERR_UNSUPPORTED,
                     "prefill: with pages that are not a power of two >= 16 tokens, the pool must hold fewer "
                     "than 2^31 tokens");
  PrefillParams p;
  p.plan = r.plan;
  p.q = static_cast<const uint8_t*>(r.q);
  p.kv = static_cast<const uint8_t*>(r.kv_pool);
  p.qo_indptr = r.qo_indptr;
  p.kv_indptr = r.kv_indptr;
  p.kv_indices = r.kv_indices;
  p.kv_last = r.kv_last_page_len;
  p.o = static_cast<uint8_t*>(r.o);
  p.lse = r.lse;
  p.ws = r.ws;
  p.status = r.status;
  p.pool_pages = r.pool_pages;
  p.Hq = r.Hq;
  p.Hk = r.Hk;
  p.P = r.P;
  p.causal = r.causal;
  p.stream_at = r.stream_at;
  p.workers = r.workers;
  p.scale = r.sm_scale;
  p.scale_log2 = r.sm_scale * kLog2e;
  p.cap = r.soft_cap;
  p.inv_cap = r.soft_cap > 0.f ? 1.f / r.soft_cap : 0.f;
  p.window = r.window;
  p.page_shift = -1;
  if (r.P >= 16 && (r.P & (r.P - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < r.P) ++sh;
    p.page_shift = sh;
  }
  {
    int sh = 0;
    while ((2ll << sh) <= r.P) ++sh;  // floor(log2 P)
    if ((r.P & (r.P - 1)) == 0) {
      p.p_magic = 0u;
      p.p_mask = 0xffffffffu;
    } else {
      p.p_magic = (uint32_t)((((uint64_t)1 << (32 + sh)) + (uint64_t)r.P - 1) / (uint64_t)r.P);
      p.p_mask = 0u;
    }
    p.p_sh = sh;
  }
  for (int i = 0; i < kRopeMaxPairs; ++i) p.rope_f[i] = r.rope_f[i];
  p.mask = r.mask;
  p.mask_indptr = r.mask_indptr;
  p.mask_last_word = r.mask_last_word;
  if (r.mask) return launch_prefill_mask(r, p);
  if (r.rope) return launch_prefill_rope(r, p);
  if (r.window >= 0) return launch_prefill_window(r, p);
  return launch_mode<false, false>(r, p);
}

}  // namespace fi
