// fi_api.cpp -- the exported C ABI: argument and plan validation, then kernel
// launches on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fi.h"
#include "fi_internal.h"
#include "plan_format.h"

namespace fi {

static thread_local char g_error[512];

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = 0; }

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_params(const fi_attn_params* p) {
  if (!p) return set_error(FI_ERR_INVALID_ARG, "null fi_attn_params");
  if (p->dtype != FI_F32 && p->dtype != FI_BF16) return set_error(FI_ERR_UNSUPPORTED, "dtype");
  if (p->out_dtype != FI_F32 && p->out_dtype != FI_BF16)
    return set_error(FI_ERR_UNSUPPORTED, "out_dtype");
  if (p->dtype == FI_F32 && p->out_dtype != FI_F32)
    return set_error(FI_ERR_UNSUPPORTED, "fp32 inputs need fp32 outputs");
  if (p->num_qo_heads < 1 || p->num_kv_heads < 1 || p->num_qo_heads % p->num_kv_heads)
    return set_error(FI_ERR_INVALID_ARG, "head counts");
  if (p->head_dim != 64 && p->head_dim != 128) return set_error(FI_ERR_UNSUPPORTED, "head_dim");
  const int G = p->num_qo_heads / p->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return set_error(FI_ERR_UNSUPPORTED, "group size");
  if (p->page_size < 1) return set_error(FI_ERR_INVALID_ARG, "page_size");
  if (!std::isfinite(p->sm_scale) || !std::isfinite(p->logits_soft_cap) || p->logits_soft_cap < 0)
    return set_error(FI_ERR_INVALID_ARG, "sm_scale / logits_soft_cap");
  if (!std::isfinite(p->rope_theta) || !std::isfinite(p->rope_scale))
    return set_error(FI_ERR_INVALID_ARG, "rope_theta / rope_scale");
  if (p->tree_mask) {
    if (!p->mask_indptr || p->mask_bits < 1 || p->mask_bits >= ((int64_t)1 << 31))
      return set_error(FI_ERR_INVALID_ARG, "tree mask: null mask_indptr or mask_bits outside [1, 2^31)");
    if (reinterpret_cast<uintptr_t>(p->tree_mask) & 3u)
      return set_error(FI_ERR_INVALID_ARG, "tree mask: words must be 4-byte aligned");
    if (p->rope_theta > 0.f)
      return set_error(FI_ERR_UNSUPPORTED, "tree mask with the rotary embedding");
  }
  return FI_OK;
}

// The host copy of the plan must be well formed and match the parameters.
int check_plan(const int32_t* ph, const fi_attn_params* p, const char* who) {
  if (!ph) return set_error(FI_ERR_INVALID_ARG, "%s: null host plan", who);
  if (ph[H_MAGIC] != kPlanMagic || ph[H_VERSION] != kPlanVersion)
    return set_error(FI_ERR_PLAN_MISMATCH, "%s: not a plan buffer", who);
  if (ph[H_HQ] != p->num_qo_heads || ph[H_HK] != p->num_kv_heads || ph[H_D] != p->head_dim ||
      ph[H_PAGE] != p->page_size)
    return set_error(FI_ERR_PLAN_MISMATCH, "%s: plan built for other heads / head_dim / page_size",
                     who);
  if (ph[H_WINDOW] < -1) return set_error(FI_ERR_PLAN_MISMATCH, "%s: corrupted window", who);
  for (int at : {(int)H_STREAM0, (int)H_STREAM1}) {
    const int32_t* sd = ph + at;
    if (sd[S_W] < 1 || sd[S_NSPLIT] > sd[S_W] - 1 || sd[S_NSLOTS] > sd[S_SLOTCAP])
      return set_error(FI_ERR_PLAN_MISMATCH, "%s: corrupted stream descriptor", who);
  }
  return FI_OK;
}

// Rotary table: for pair d < D/2 the turn per position, theta^(-2d/D) /
// scale radians, as a fraction of a revolution in 2^-32 units (whole turns
// dropped).  The kernels multiply it by the position modulo 2^32.
void rope_table(const fi_attn_params* p, RunArgs& a) {
  a.rope = p->rope_theta > 0.f;
  for (int d = 0; d < 64; ++d) a.rope_f[d] = 0;
  if (!a.rope) return;
  const double scale = p->rope_scale > 0.f ? (double)p->rope_scale : 1.0;
  const double two_pi = 6.283185307179586476925286766559;
  for (int d = 0; d < p->head_dim / 2; ++d) {
    const double rev = std::pow((double)p->rope_theta, -2.0 * d / p->head_dim) / scale / two_pi;
    const double frac = rev - std::floor(rev);
    a.rope_f[d] = (uint32_t)(uint64_t)std::llround(std::ldexp(frac, 32));  // 2^32 wraps to 0
  }
}

float resolve_scale(const fi_attn_params* p) {
  return p->sm_scale > 0.f ? p->sm_scale : 1.0f / std::sqrt((float)p->head_dim);
}

RunArgs base_args(const int32_t* plan_dev, const fi_attn_params* p, const void* q,
                  const void* kv_pool, int64_t pool_pages, const int32_t* qo_indptr,
                  const int32_t* kv_indptr, const int32_t* kv_indices,
                  const int32_t* kv_last_page_len, void* o, float* lse, void* ws,
                  fi_dtype out_dtype, const int32_t* ph, void* stream) {
  RunArgs a;
  a.plan = plan_dev;
  a.q = q;
  a.kv_pool = kv_pool;
  a.pool_pages = pool_pages;
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.kv_last_page_len = kv_last_page_len;
  a.o = o;
  a.lse = lse;
  a.ws = static_cast<float*>(ws);
  a.status = static_cast<int32_t*>(ws);  // word 0 of the workspace's control region
  a.Hq = p->num_qo_heads;
  a.Hk = p->num_kv_heads;
  a.D = p->head_dim;
  a.P = p->page_size;
  a.G = a.Hq / a.Hk;
  a.causal = ph[H_CAUSAL];
  a.window = ph[H_WINDOW];
  rope_table(p, a);
  a.mask = p->tree_mask;
  a.mask_indptr = p->mask_indptr;
  a.mask_last_word = p->tree_mask ? (int32_t)((p->mask_bits - 1) >> 5) : 0;
  a.sm_scale = resolve_scale(p);
  a.soft_cap = p->logits_soft_cap;
  a.dtype = p->dtype;
  a.out_dtype = out_dtype;
  a.hip_stream = stream;
  return a;
}

// Decode stream, prefill stream, then the merges of split rows, each with the
// fixed grid of its stream.  A kernel is launched when its stream holds rows
// (merges: split rows), as read from the host copy of the plan; with
// graph_safe, whenever the call kind and dtype can use it, so that a captured
// call launches the same kernels for every later plan.
int run_plan(RunArgs a, const int32_t* ph, bool with_prefill, bool graph_safe) {
  int rc;
  if (with_prefill && ph[H_STREAM1 + S_NROWS] != 0 && a.dtype != FI_BF16)
    return set_error(FI_ERR_UNSUPPORTED, "prefill tiles need bf16 q / kv");
  const bool dec = graph_safe || ph[H_STREAM0 + S_NROWS] != 0;
  const bool pre = with_prefill && (graph_safe ? a.dtype == FI_BF16 : ph[H_STREAM1 + S_NROWS] != 0);
  // merge grids: one block row per split row of this plan, or the bound W - 1
  // when the launch must serve every later plan (graph capture)
  a.stream_at = H_STREAM0;
  a.workers = ph[H_STREAM0 + S_W];
  a.max_tasks = graph_safe ? a.workers - 1 : ph[H_STREAM0 + S_NSPLIT];
  RunArgs b = a;
  b.stream_at = H_STREAM1;
  b.workers = ph[H_STREAM1 + S_W];
  b.max_tasks = graph_safe ? b.workers - 1 : ph[H_STREAM1 + S_NSPLIT];
  if (dec && (rc = launch_decode(a))) return rc;
  if (pre && (rc = launch_prefill(b))) return rc;
  if (dec && (graph_safe || ph[H_STREAM0 + S_NSPLIT] != 0) && (rc = launch_merge_partials(a))) return rc;
  if (pre && (graph_safe || ph[H_STREAM1 + S_NSPLIT] != 0) && (rc = launch_merge_partials(b))) return rc;
  return FI_OK;
}

// A plan in which some row sees KV pages makes the kernels read kv_indices
// and the pool: both must be there, and the pool must hold page 0, which
// stands in for an out-of-pool id.
int check_pages(const int32_t* ph, const void* kv_pool, int64_t pool_pages,
                const int32_t* kv_indices, const char* who) {
  if (pool_pages < 0) return set_error(FI_ERR_INVALID_ARG, "%s: pool_pages < 0", who);
  if (ph[H_ANY_PAGES] && (pool_pages < 1 || !kv_pool || !kv_indices))
    return set_error(FI_ERR_INVALID_ARG,
                     "%s: the plan reads KV pages, so kv_pool, kv_indices and pool_pages >= 1 are needed", who);
  return FI_OK;
}

int check_common(const int32_t* plan_host, const int32_t* plan_dev, const fi_attn_params* params,
                 const void* q, const void* kv_pool, int64_t pool_pages, const int32_t* kv_indptr,
                 const int32_t* kv_indices, const int32_t* kv_last_page_len, const void* o,
                 const void* float_ws, int64_t float_ws_bytes, const char* who,
                 bool decode_ws_only = false) {
  int rc;
  if ((rc = check_params(params))) return rc;
  if ((rc = check_plan(plan_host, params, who))) return rc;
  const int B = plan_host[H_BATCH];
  if (!plan_dev) return set_error(FI_ERR_INVALID_ARG, "%s: null device plan", who);
  if (B > 0 && (!kv_indptr || !kv_last_page_len))
    return set_error(FI_ERR_INVALID_ARG, "%s: null index array", who);
  if (plan_host[H_TOTAL_QO] > 0 && (!q || !o))
    return set_error(FI_ERR_INVALID_ARG, "%s: null q or o", who);
  if ((rc = check_pages(plan_host, kv_pool, pool_pages, kv_indices, who))) return rc;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(o))
    return set_error(FI_ERR_INVALID_ARG, "%s: q, kv_pool and o must be 16-byte aligned", who);
  const int64_t need = decode_ws_only ? decode_ws_bytes(plan_host) : (int64_t)plan_host[H_WS_FLOATS] * 4;
  if (!float_ws || float_ws_bytes < need)
    return set_error(FI_ERR_WORKSPACE_TOO_SMALL, "%s: float workspace %lld bytes, needs %lld", who,
                     (long long)float_ws_bytes, (long long)need);
  if (!aligned16(float_ws)) return set_error(FI_ERR_INVALID_ARG, "%s: float_ws alignment", who);
  return FI_OK;
}

}  // namespace

int64_t decode_ws_bytes(const int32_t* ph) {
  if (!ph || ph[H_MAGIC] != kPlanMagic) return -1;
  const int32_t* sd = ph + H_STREAM0;
  const int64_t lse_floats = ((int64_t)sd[S_SLOTCAP] * ph[H_HQ] + 63) / 64 * 64;
  return ((int64_t)sd[S_WS_LSE] + lse_floats) * 4;
}

int decode_paged(const int32_t* plan_host, const int32_t* plan_dev, const fi_attn_params* params,
                 const void* q, const void* kv_pool, int64_t pool_pages, const int32_t* kv_indptr,
                 const int32_t* kv_indices, const int32_t* kv_last_page_len, void* o, float* lse,
                 void* float_ws, int64_t float_ws_bytes, void* stream, bool decode_ws_only) {
  int rc = check_common(plan_host, plan_dev, params, q, kv_pool, pool_pages, kv_indptr, kv_indices,
                        kv_last_page_len, o, float_ws, float_ws_bytes, "fi_batch_decode_paged",
                        decode_ws_only);
  if (rc) return rc;
  if (plan_host[H_STREAM1 + S_NROWS] != 0 || plan_host[H_TOTAL_QO] != plan_host[H_BATCH])
    return set_error(FI_ERR_PLAN_MISMATCH,
                     "fi_batch_decode_paged: plan has multi-query requests; use fi_batch_prefill_paged");
  RunArgs a = base_args(plan_dev, params, q, kv_pool, pool_pages, nullptr, kv_indptr, kv_indices,
                        kv_last_page_len, o, lse, float_ws, params->out_dtype, plan_host, stream);
  return run_plan(a, plan_host, false, params->graph_safe != 0);
}

}  // namespace fi

using namespace fi;

extern "C" {

int fi_plan(const fi_plan_in* in, int32_t* plan, int64_t plan_capacity, fi_plan_info* info) {
  return build_plan(in, plan, plan_capacity, info);
}

int fi_plan_bounds(int32_t batch_size, int64_t total_qo, int32_t num_qo_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t workers_decode,
                   int32_t workers_prefill, int64_t* plan_ints, int64_t* float_ws_bytes) {
  clear_error();
  return plan_bounds(batch_size, total_qo, num_qo_heads, num_kv_heads, head_dim, workers_decode,
                     workers_prefill, plan_ints, float_ws_bytes);
}

int fi_batch_decode_paged(const int32_t* plan_host, const int32_t* plan_dev,
                          const fi_attn_params* params, const void* q, const void* kv_pool,
                          int64_t pool_pages, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_last_page_len, void* o,
                          float* lse, void* float_ws, int64_t float_ws_bytes, void* stream) {
  clear_error();
  return decode_paged(plan_host, plan_dev, params, q, kv_pool, pool_pages, kv_indptr, kv_indices,
                      kv_last_page_len, o, lse, float_ws, float_ws_bytes, stream, false);
}

int fi_batch_prefill_paged(const int32_t* plan_host, const int32_t* plan_dev,
                           const fi_attn_params* params, const void* q, const void* kv_pool,
                           int64_t pool_pages, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           const int32_t* kv_last_page_len, void* o, float* lse,
                           void* float_ws, int64_t float_ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(plan_host, plan_dev, params, q, kv_pool, pool_pages, kv_indptr, kv_indices,
                        kv_last_page_len, o, float_ws, float_ws_bytes, "fi_batch_prefill_paged");
  if (rc) return rc;
  if (plan_host[H_BATCH] > 0 && !qo_indptr)
    return set_error(FI_ERR_INVALID_ARG, "fi_batch_prefill_paged: null qo_indptr");
  if (params->tree_mask && (plan_host[H_CAUSAL] != 1 || plan_host[H_WINDOW] >= 0))
    return set_error(FI_ERR_UNSUPPORTED, "fi_batch_prefill_paged: a tree mask needs a causal plan without a window");
  RunArgs a = base_args(plan_dev, params, q, kv_pool, pool_pages, qo_indptr, kv_indptr, kv_indices,
                        kv_last_page_len, o, lse, float_ws, params->out_dtype, plan_host, stream);
  return run_plan(a, plan_host, true, params->graph_safe != 0);
}

int fi_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                   void* v_out, float* s_out, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                   fi_dtype dtype, void* stream) {
  clear_error();
  if (n_tokens < 0 || n_heads < 1 || head_dim < 1)
    return set_error(FI_ERR_INVALID_ARG, "fi_merge_state: sizes");
  if (dtype != FI_F32 && dtype != FI_BF16) return set_error(FI_ERR_UNSUPPORTED, "fi_merge_state: dtype");
  if (n_tokens > 0 && (!v_a || !s_a || !v_b || !s_b || !v_out || !s_out))
    return set_error(FI_ERR_INVALID_ARG, "fi_merge_state: null pointer");
  return launch_merge_state(v_a, s_a, v_b, s_b, v_out, s_out, n_tokens * n_heads, head_dim, dtype,
                            dtype, stream);
}

int64_t fi_cascade_workspace_bytes(const int32_t* plan0_host, const int32_t* plan1_host) {
  clear_error();
  if (!plan0_host || !plan1_host || plan0_host[H_MAGIC] != kPlanMagic ||
      plan1_host[H_MAGIC] != kPlanMagic)
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade_workspace_bytes: not plan buffers");
  auto al = [](int64_t b) { return (b + 255) / 256 * 256; };
  const int64_t rows = (int64_t)plan1_host[H_TOTAL_QO] * plan1_host[H_HQ];
  const int64_t state = al(rows * plan1_host[H_D] * 4) + al(rows * 4);
  return al((int64_t)plan0_host[H_WS_FLOATS] * 4) + al((int64_t)plan1_host[H_WS_FLOATS] * 4) +
         2 * state;
}

int fi_cascade(const int32_t* plan0_host, const int32_t* plan0_dev, const int32_t* qo_indptr0,
               const int32_t* kv_indptr0, const int32_t* kv_indices0,
               const int32_t* kv_last_page_len0, const int32_t* plan1_host,
               const int32_t* plan1_dev, const int32_t* qo_indptr1, const int32_t* kv_indptr1,
               const int32_t* kv_indices1, const int32_t* kv_last_page_len1,
               const fi_attn_params* params, const void* q, const void* kv_pool,
               int64_t pool_pages, void* o, float* lse, void* float_ws, int64_t float_ws_bytes,
               void* stream) {
  clear_error();
  int rc;
  if ((rc = check_params(params))) return rc;
  if ((rc = check_plan(plan0_host, params, "fi_cascade level 0"))) return rc;
  if ((rc = check_plan(plan1_host, params, "fi_cascade level 1"))) return rc;
  if (plan0_host[H_CAUSAL] != 0)
    return set_error(FI_ERR_PLAN_MISMATCH, "fi_cascade: level-0 plan must be non-causal");
  if (params->rope_theta > 0.f)
    return set_error(FI_ERR_UNSUPPORTED, "fi_cascade: the rotary embedding is not supported");
  if (params->tree_mask) return set_error(FI_ERR_UNSUPPORTED, "fi_cascade: tree masks are not supported");
  if (plan0_host[H_WINDOW] >= 0 || plan1_host[H_WINDOW] >= 0)
    return set_error(FI_ERR_UNSUPPORTED, "fi_cascade: plans with a sliding window are not supported");
  if (plan0_host[H_TOTAL_QO] != plan1_host[H_TOTAL_QO])
    return set_error(FI_ERR_PLAN_MISMATCH, "fi_cascade: levels cover different query rows");
  if (!plan0_dev || !plan1_dev) return set_error(FI_ERR_INVALID_ARG, "fi_cascade: null device plan");
  if (plan0_host[H_BATCH] > 0 && (!qo_indptr0 || !kv_indptr0 || !kv_last_page_len0))
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: null level-0 index array");
  // level 1 may be a decode-only plan (qo_indptr1 NULL: one query per request)
  const bool multi1 = plan1_host[H_TOTAL_QO] != plan1_host[H_BATCH] || plan1_host[H_STREAM1 + S_NROWS] != 0;
  if (plan1_host[H_BATCH] > 0 && (!kv_indptr1 || !kv_last_page_len1 || (multi1 && !qo_indptr1)))
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: null level-1 index array");
  if ((rc = check_pages(plan0_host, kv_pool, pool_pages, kv_indices0, "fi_cascade level 0"))) return rc;
  if ((rc = check_pages(plan1_host, kv_pool, pool_pages, kv_indices1, "fi_cascade level 1"))) return rc;
  const int64_t need = fi_cascade_workspace_bytes(plan0_host, plan1_host);
  if (need < 0) return (int)need;
  if (!float_ws || float_ws_bytes < need)
    return set_error(FI_ERR_WORKSPACE_TOO_SMALL, "fi_cascade: float workspace %lld bytes, needs %lld",
                     (long long)float_ws_bytes, (long long)need);
  if (!aligned16(float_ws) || !aligned16(q) || !aligned16(kv_pool) || !aligned16(o))
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: 16-byte alignment");
  const int64_t total_qo = plan1_host[H_TOTAL_QO];
  if (total_qo > 0 && (!q || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_cascade: null q or o");
  // workspace: level-0 partials | level-1 partials | state 0 (o, lse) | state 1 (o, lse)
  auto al = [](int64_t b) { return (b + 255) / 256 * 256; };
  uint8_t* base = static_cast<uint8_t*>(float_ws);
  uint8_t* ws0 = base;
  uint8_t* ws1 = ws0 + al((int64_t)plan0_host[H_WS_FLOATS] * 4);
  const int64_t rows = total_qo * params->num_qo_heads;
  uint8_t* o0 = ws1 + al((int64_t)plan1_host[H_WS_FLOATS] * 4);
  float* l0 = reinterpret_cast<float*>(o0 + al(rows * params->head_dim * 4));
  uint8_t* o1 = reinterpret_cast<uint8_t*>(l0) + al(rows * 4);
  float* l1 = reinterpret_cast<float*>(o1 + al(rows * params->head_dim * 4));

  RunArgs a0 = base_args(plan0_dev, params, q, kv_pool, pool_pages, qo_indptr0, kv_indptr0,
                         kv_indices0, kv_last_page_len0, o0, l0, ws0, FI_F32, plan0_host, stream);
  if ((rc = run_plan(a0, plan0_host, true, params->graph_safe != 0))) return rc;
  RunArgs a1 = base_args(plan1_dev, params, q, kv_pool, pool_pages, qo_indptr1, kv_indptr1,
                         kv_indices1, kv_last_page_len1, o1, l1, ws1, FI_F32, plan1_host, stream);
  a1.status = a0.status;  // one status word per cascade workspace: its first word
  if ((rc = run_plan(a1, plan1_host, true, params->graph_safe != 0))) return rc;
  float* lse_out = lse ? lse : l1;  // without a caller lse, merge it in place
  return launch_merge_state(o0, l0, o1, l1, o, lse_out, rows, params->head_dim, FI_F32,
                            params->out_dtype, stream);
}

int fi_read_status(const void* float_ws, int32_t* status, int32_t clear, void* stream) {
  clear_error();
  if (!status) return set_error(FI_ERR_INVALID_ARG, "fi_read_status: null status pointer");
  if (!float_ws && !(float_ws = noalloc_scratch())) return FI_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, float_ws, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && clear && word != 0) e = hipMemsetAsync(const_cast<void*>(float_ws), 0, sizeof(word), s);
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "fi_read_status: %s", hipGetErrorString(e));
  *status = word;
  return FI_OK;
}

const char* fi_last_error(void) { return g_error; }

int fi_version(void) { return 100; }

int fi_default_workers(int kind, int num_cus, int num_kv_heads) {
  if (num_cus < 1 || num_kv_heads < 1) return 1;
  // decode: 5 one-wave workgroups per CU (every worker resident, none
  // waiting for a slot; with the fixed cost a plan charges per decode item,
  // 5 gave the llama8b_decode step 116.0 us against 118.2 at 6, and the
  // skewed and mixed steps no slower); prefill: 2 workgroups of 4 waves per CU
  const int per_cu = kind == FI_KIND_PREFILL ? 2 : 5;
  int w = per_cu * num_cus / num_kv_heads;
  return w < 1 ? 1 : w;
}

}  // extern "C"
