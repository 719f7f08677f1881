// append.hip -- paged KV append (gfx950): a step's new K/V tokens into the
// slots their page table gives them (talk page, Background, "Dynamic Problem
// Shapes": the append stage; serving-engine page, "Page-Level Attention":
// tokens fill a request's pages in order).
//
// One wave per token.  A token's K row (num_kv_heads x head_dim elements) is
// contiguous in both the input and the pool, as is its V row, so the wave
// copies them with 16-byte loads and stores; each wave's request is found
// by a binary search of append_indptr.  Bound by HBM: every byte is read
// once and written once.
#include "device_common.h"
#include "fi.h"
#include "fi_internal.h"

namespace fi {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 8192;  // grid-stride beyond 32768 tokens

struct AppendParams {
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* append_indptr;
  uint8_t* pool;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* last;
  int64_t n_tokens;
  int64_t pool_pages;
  int64_t kv_indices_len;
  int32_t B;
  int32_t P;
  int32_t row_bytes;  // num_kv_heads * head_dim * element size (multiple of 16)
};

__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int64_t tok = (int64_t)blockIdx.x * kWaves + wave; tok < a.n_tokens;
       tok += (int64_t)gridDim.x * kWaves) {
    // request i with append_indptr[i] <= tok < append_indptr[i + 1]: the
    // last entry of [0, B) that is <= tok
    int lo = 0, hi = a.B;  // answer in [lo, hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.append_indptr[mid] <= tok) lo = mid; else hi = mid;
    }
    const int i = lo;
    const int64_t t = tok - a.append_indptr[i];
    const int64_t n = (int64_t)a.append_indptr[i + 1] - a.append_indptr[i];
    const int64_t e0 = a.kv_indptr[i];
    const int64_t pages = (int64_t)a.kv_indptr[i + 1] - e0;
    const int64_t kv_len = pages <= 0 ? 0 : (pages - 1) * a.P + a.last[i];
    const int64_t pos = kv_len - n + t;
    if (pos < 0 || t < 0 || t >= n) continue;  // more new tokens than the request holds
    const int64_t e = e0 + pos / a.P;
    if (e < 0 || e >= a.kv_indices_len) continue;
    const int64_t page = a.kv_indices[e];
    if (page < 0 || page >= a.pool_pages) continue;
    const int64_t slot = pos % a.P;
    const int64_t half = (int64_t)a.P * a.row_bytes;  // bytes of one K or V half-page
    uint8_t* dk = a.pool + page * 2 * half + slot * a.row_bytes;
    uint8_t* dv = dk + half;
    const uint8_t* sk = a.k + tok * a.row_bytes;
    const uint8_t* sv = a.v + tok * a.row_bytes;
    for (int off = lane * 16; off < a.row_bytes; off += 64 * 16) {
      const u32x4_t x = load16(sk + off);
      const u32x4_t y = load16(sv + off);
      *reinterpret_cast<u32x4_t*>(dk + off) = x;
      *reinterpret_cast<u32x4_t*>(dv + off) = y;
    }
  }
}

}  // namespace
}  // namespace fi

using namespace fi;

extern "C" int fi_append_paged_kv(const void* append_k, const void* append_v, fi_dtype dtype,
                                  const int32_t* append_indptr, int32_t batch_size, int64_t n_tokens,
                                  void* kv_pool, int64_t pool_pages, int32_t page_size,
                                  int32_t num_kv_heads, int32_t head_dim, const int32_t* kv_indptr,
                                  const int32_t* kv_indices, int64_t kv_indices_len,
                                  const int32_t* kv_last_page_len, void* stream) {
  clear_error();
  if (dtype != FI_F32 && dtype != FI_BF16) return set_error(FI_ERR_UNSUPPORTED, "fi_append_paged_kv: dtype");
  if (batch_size < 0 || n_tokens < 0 || pool_pages < 0 || kv_indices_len < 0 || page_size < 1 ||
      num_kv_heads < 1 || head_dim < 1)
    return set_error(FI_ERR_INVALID_ARG, "fi_append_paged_kv: sizes");
  const int64_t row = (int64_t)num_kv_heads * head_dim * (dtype == FI_BF16 ? 2 : 4);
  if (row % 16 != 0 || row > (1 << 30))
    return set_error(FI_ERR_UNSUPPORTED, "fi_append_paged_kv: token row of %lld bytes", (long long)row);
  if (n_tokens == 0) return FI_OK;
  if (batch_size == 0)
    return set_error(FI_ERR_INVALID_ARG, "fi_append_paged_kv: tokens without requests");
  if (!append_k || !append_v || !append_indptr || !kv_pool || !kv_indptr || !kv_indices ||
      !kv_last_page_len)
    return set_error(FI_ERR_INVALID_ARG, "fi_append_paged_kv: null pointer");
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!al(append_k) || !al(append_v) || !al(kv_pool))
    return set_error(FI_ERR_INVALID_ARG, "fi_append_paged_kv: k, v and kv_pool must be 16-byte aligned");
  AppendParams p;
  p.k = static_cast<const uint8_t*>(append_k);
  p.v = static_cast<const uint8_t*>(append_v);
  p.append_indptr = append_indptr;
  p.pool = static_cast<uint8_t*>(kv_pool);
  p.kv_indptr = kv_indptr;
  p.kv_indices = kv_indices;
  p.last = kv_last_page_len;
  p.n_tokens = n_tokens;
  p.pool_pages = pool_pages;
  p.kv_indices_len = kv_indices_len;
  p.B = batch_size;
  p.P = page_size;
  p.row_bytes = (int32_t)row;
  const int64_t blocks = (n_tokens + kWaves - 1) / kWaves;
  dim3 grid((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks)), block(kThreads);
  hipLaunchKernelGGL(append_kernel, grid, block, 0, (hipStream_t)stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(FI_ERR_HIP, "append launch: %s", hipGetErrorString(err));
  return FI_OK;
}
