// fi_internal.h -- host-side internals shared by the library's translation
// units: the thread-local error message and the kernel launch entry points.
#pragma once
#include <stdint.h>

#include <algorithm>

#include "fi.h"

namespace fi {

// Records a printf-style message for fi_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

int build_plan(const fi_plan_in* in, int32_t* buf, int64_t capacity, fi_plan_info* info);

// The decode call with its workspace given (fi_api.cpp).  decode_ws_only:
// float_ws_bytes need only cover the control region and the decode stream's
// regions, the part a decode call touches.
int decode_paged(const int32_t* plan_host, const int32_t* plan_dev, const fi_attn_params* params,
                 const void* q, const void* kv_pool, int64_t pool_pages, const int32_t* kv_indptr,
                 const int32_t* kv_indices, const int32_t* kv_last_page_len, void* o, float* lse,
                 void* float_ws, int64_t float_ws_bytes, void* stream, bool decode_ws_only);
// Bytes of the workspace a decode call of this plan touches (its control
// region and decode regions), or < 0 if the plan is malformed.
int64_t decode_ws_bytes(const int32_t* plan_host);
// The static scratch of fi_batch_decode_paged_noalloc on the current device
// (its device address, looked up once per device), or NULL with the error set.
void* noalloc_scratch();
int plan_bounds(int32_t B, int64_t total_qo, int32_t Hq, int32_t Hk, int32_t D, int32_t Wd,
                int32_t Wp, int64_t* plan_ints, int64_t* ws_bytes);

// Everything a kernel of one stream needs; built by the API layer after
// validation.  Device pointers unless noted.
struct RunArgs {
  const int32_t* plan;          // device plan
  const void* q;
  const void* kv_pool;
  int64_t pool_pages;
  const int32_t* qo_indptr;     // NULL: request i has query row i
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last_page_len;
  void* o;                      // direct outputs
  float* lse;                   // may be NULL
  float* ws;                    // float workspace base
  int32_t* status;              // status word (bit flags, OR-ed by the kernels)
  int32_t Hq, Hk, D, P, G;
  int32_t causal;
  int32_t window;               // sliding window (keys before the query's own); -1 = none
  int32_t rope;                 // rotary embedding on q and k (rope_f holds its table)
  const uint32_t* mask;         // tree mask words, or NULL (prefill kernels only)
  const int32_t* mask_indptr;   // bit offset of each request's qo x qo block
  int32_t mask_last_word;       // index of the mask's last word
  uint32_t rope_f[64];          // per pair d < D/2: turn per position, 2^-32 revolutions
  float sm_scale;
  float soft_cap;
  fi_dtype dtype, out_dtype;
  int32_t workers;              // grid.x of this stream's kernel
  int32_t max_tasks;            // merge kernel grid.x: split rows of the plan, or W - 1 (graph_safe)
  int32_t stream_at;            // H_STREAM0 or H_STREAM1
  void* hip_stream;
};

// Kernel launches; return FI_OK or FI_ERR_*.  Each validates nothing: the
// API layer has already checked shapes, dtypes and the plan.
int launch_decode(const RunArgs& a);
int launch_prefill(const RunArgs& a);
int launch_merge_partials(const RunArgs& a);
int launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                       void* vo, float* so, int64_t n_rows, int32_t head_dim, fi_dtype vdt,
                       fi_dtype odt, void* stream);

}  // namespace fi
