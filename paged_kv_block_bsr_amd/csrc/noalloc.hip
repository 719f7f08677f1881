// noalloc.hip -- the batch-decode call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation): its float workspace is a static device array of
// this library instead of a caller buffer.
//
// The array lives once per GPU for the life of the process and is zero when
// the code object is loaded; every call on a GPU shares it and keeps what the
// last call left there.  The calls need nothing of it to start at zero (the
// status word only collects flags).  Calls that overlap on one GPU race on
// it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fi.h"
#include "fi_internal.h"

namespace fi {
namespace {

constexpr int64_t kScratchBytes = FI_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) float scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // per device: the device address of `scratch`

}  // namespace

// Device address of `scratch` on the current device, looked up with that
// device current on the first call there and kept.  Host code uses only this
// address: the array's own name is a host-side stand-in.
void* noalloc_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(FI_ERR_HIP, "no-alloc scratch: hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error(FI_ERR_UNSUPPORTED, "no-alloc scratch: device %d", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error(FI_ERR_HIP, "no-alloc scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace fi

using namespace fi;

extern "C" int fi_batch_decode_paged_noalloc(const int32_t* plan_host, const int32_t* plan_dev,
                                             const fi_attn_params* params, const void* q,
                                             const void* kv_pool, int64_t pool_pages,
                                             const int32_t* kv_indptr, const int32_t* kv_indices,
                                             const int32_t* kv_last_page_len, void* o, float* lse,
                                             void* stream) {
  clear_error();
  const int64_t need = decode_ws_bytes(plan_host);
  if (need < 0) return set_error(FI_ERR_PLAN_MISMATCH, "fi_batch_decode_paged_noalloc: not a plan buffer");
  if (need > kScratchBytes)
    return set_error(FI_ERR_WORKSPACE_TOO_SMALL,
                     "fi_batch_decode_paged_noalloc: the plan needs %lld bytes of workspace, the static "
                     "scratch holds %lld (fewer decode workers need less)",
                     (long long)need, (long long)kScratchBytes);
  void* ws = noalloc_scratch();
  if (!ws) return FI_ERR_HIP;
  return decode_paged(plan_host, plan_dev, params, q, kv_pool, pool_pages, kv_indptr, kv_indices,
                      kv_last_page_len, o, lse, ws, kScratchBytes, stream, true);
}
