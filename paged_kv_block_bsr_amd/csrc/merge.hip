// merge.hip -- log-sum-exp composition of attention states (gfx950).
//
// merge_partials: for every row the plan split over k >= 2 workers, combine
// the k partial (o, lse) slots into the final output (serving-engine page,
// "FlashDecoding: Parallel KV Split", the merge step; paper page, partial
// results merged with the log-sum-exp composition).  Grid (split rows of
// the plan, KV heads, 16-row blocks): block x takes the x-th split row of
// the stream.  A call made for graph capture launches the bound, workers -
// 1, instead, and blocks past the stream's split rows exit, so the captured
// launch serves every later plan.
//
// merge_state: the two-way merge of the cascade (serving-engine page,
// "Cascade Attention for Shared Prefixes", merge_state).
#include "device_common.h"
#include "fi_internal.h"

namespace fi {
namespace {

constexpr int kThreads = 256;

struct MergeParams {
  const int32_t* plan;
  uint8_t* o;
  float* lse;
  const float* ws;
  int32_t Hq, Hk, D, G;
  int32_t stream_at;
  int32_t out_bf16;
};

constexpr int kMergeRows = 16;  // packed rows per merge block (grid z covers a 128-row tile)

// Block (task, g, z) merges rows 16 z .. 16 z + 15 of split row `task`.
// Threads take (row, 16-dim chunk) units; when there are fewer units than
// threads, the slots are also divided among thread groups.  Each thread
// folds its slots into a running (max, sum, weighted o) state as it reads
// them -- lse and o of a slot are loaded together, so a block needs one
// round trip to memory -- and the group states are composed through LDS.
// kBatch: slots a thread loads before folding them.  Decode rows of a long
// request are split into hundreds of slots, which batches of 4 fold with
// fewer waits (skewed_long_decode: merge 13.3 -> 11.0 us); prefill tiles are
// split in two or three, where the batch's registers cost more than they
// save (slice call 0.1266 -> 0.1287 ms), so their merge folds one at a time.
template <int kBatch>
__global__ __launch_bounds__(kThreads) void merge_partials_kernel(MergeParams a) {
  const int32_t* sd = a.plan + a.stream_at;
  const int task = blockIdx.x;
  const int n_split = sd[S_NSPLIT];
  if (task >= n_split) return;
  const int g = blockIdx.y;
  // the split row's record: packed rows, query base, first slot; its slots
  // end where the next record's begin (the last at the stream's slot count)
  const int32_t* rec = a.plan + sd[S_OFF_SREC] + 4 * task;
  const int rb = rec[0], re = rec[1], qbase = rec[2], s0 = rec[3];
  const int s1 = task + 1 < n_split ? rec[4 + 3] : sd[S_NSLOTS];
  const int r0 = kMergeRows * blockIdx.z;
  if (r0 >= re - rb) return;
  const int nr = min(kMergeRows, re - rb - r0);
  // partial layout [slot][Hk][stride][D]; stride = G for decode rows, 128 for tiles
  const int stride = sd[S_KIND] == 0 ? a.G : kMaxTileRows;
  const float* wo = a.ws + sd[S_WS_O];
  const float* wl = a.ws + sd[S_WS_LSE];
  const int D = a.D, G = a.G;
  const int tid = threadIdx.x;

  // A unit is one row's 16 consecutive dims (4 x 16-byte pieces): with few
  // units per row, more thread groups share a row's slots, so a row split
  // into hundreds of slots (one very long request) is folded by many groups
  // in parallel rather than by one thread walking them all.
  constexpr int NV = 4;  // 16-byte pieces per unit
  __shared__ f32x4_t red_acc[kThreads][NV];
  __shared__ float red_m[kThreads], red_l[kThreads];
  auto write_out = [&](int rr, int c, f32x4_t (&acc)[NV], float m, float l) {
    const bool empty = m == neg_inf() || !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const int packed = rb + r0 + rr;
    const int64_t orow = (int64_t)(qbase + packed / G) * a.Hq + g * G + packed % G;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const f32x4_t x = acc[v] * inv;
      const int64_t at = orow * D + 4 * (NV * c + v);
      if (a.out_bf16) {
        reinterpret_cast<uint32_t*>(a.o)[at / 2] = pack_bf16x2(x[0], x[1]);
        reinterpret_cast<uint32_t*>(a.o)[at / 2 + 1] = pack_bf16x2(x[2], x[3]);
      } else {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.o) + at) = x;
      }
    }
    if (a.lse && c == 0) a.lse[orow] = empty ? neg_inf() : m + __logf(l);
  };
  const int chunks = D / (4 * NV);
  const int U = nr * chunks;  // (row, 16-dim chunk) units
  int UP = 1;
  while (UP < U) UP <<= 1;
  const int ngroups = UP >= kThreads ? 1 : kThreads / UP;
  const int sg = UP >= kThreads ? 0 : tid / UP;
  for (int u = (UP >= kThreads ? tid : tid % UP); u < U; u += (UP >= kThreads ? kThreads : UP)) {
    const int rr = u / chunks, c = u % chunks;
    float m = neg_inf(), l = 0.f;
    f32x4_t acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Slots s, s + ngroups, ... in batches of kBatch: a batch's loads are
    // issued together (a row split over hundreds of slots would otherwise
    // wait for each slot in turn), then folded with one rescale.  Batch
    // members past the row's last slot load nothing and count as lse -inf,
    // weight 0.
    for (int s = s0 + sg; s < s1; s += kBatch * ngroups) {
      float x[kBatch];
      f32x4_t vv[kBatch][NV];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int sb = s + b * ngroups;
        x[b] = neg_inf();
#pragma unroll
        for (int v = 0; v < NV; ++v) vv[b][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (sb < s1) {
          const int64_t pr = ((int64_t)sb * a.Hk + g) * stride + r0 + rr;
          x[b] = wl[pr];
#pragma unroll
          for (int v = 0; v < NV; ++v) vv[b][v] = *reinterpret_cast<const f32x4_t*>(wo + pr * D + 4 * (NV * c + v));
        }
      }
      float mb = x[0];
#pragma unroll
      for (int b = 1; b < kBatch; ++b) mb = fmaxf(mb, x[b]);
      if (mb > m) {  // a new running max: rescale what is there (exp(-inf) = 0 on the first batch)
        const float r = __expf(m - mb);
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] *= r;
        l *= r;
        m = mb;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const float w = x[b] == neg_inf() ? 0.f : __expf(x[b] - m);
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += w * vv[b][v];
        l += w;
      }
    }
    if (ngroups > 1) {
#pragma unroll
      for (int v = 0; v < NV; ++v) red_acc[tid][v] = acc[v];
      red_m[tid] = m;
      red_l[tid] = l;
      break;  // one unit per thread when the slots are split among groups
    }
    write_out(rr, c, acc, m, l);
  }
  if (ngroups > 1) {
    __syncthreads();
    if (tid < U) {
      float M = red_m[tid];
      for (int k = 1; k < ngroups; ++k) M = fmaxf(M, red_m[tid + k * UP]);
      f32x4_t acc[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float L = 0.f;
      if (M != neg_inf()) {
        for (int k = 0; k < ngroups; ++k) {
          const float mk = red_m[tid + k * UP];
          const float w = mk == neg_inf() ? 0.f : __expf(mk - M);
#pragma unroll
          for (int v = 0; v < NV; ++v) acc[v] += w * red_acc[tid + k * UP][v];
          L += w * red_l[tid + k * UP];
        }
      }
      write_out(tid / chunks, tid % chunks, acc, M, L);
    }
  }
}

// Two-way merge; one wave per row, lane e takes elements e, e + 64, ...  Every
// lane reads both lse values in the same instruction, before any lane writes,
// so the outputs may alias the inputs.
template <typename VT, typename OT>
__global__ __launch_bounds__(kThreads) void merge_state_kernel(const uint8_t* va, const float* sa,
                                                               const uint8_t* vb, const float* sb,
                                                               uint8_t* vo, float* so,
                                                               int64_t n_rows, int32_t D) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); row < n_rows;
       row += waves) {
    const float la = sa[row], lb = sb[row];
    const float M = fmaxf(la, lb);
    const bool empty = M == neg_inf();
    const float wa = empty ? 0.f : __expf(la - M);
    const float wb = empty ? 0.f : __expf(lb - M);
    const float inv = empty ? 0.f : 1.f / (wa + wb);
    for (int e = lane; e < D; e += 64) {
      const int64_t i = row * D + e;
      float x, y;
      if constexpr (VT::kBytes == 2) {
        x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(va)[i] << 16);
        y = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(vb)[i] << 16);
      } else {
        x = reinterpret_cast<const float*>(va)[i];
        y = reinterpret_cast<const float*>(vb)[i];
      }
      const float r = empty ? 0.f : (wa * x + wb * y) * inv;
      if constexpr (OT::kBytes == 2)
        reinterpret_cast<uint16_t*>(vo)[i] = (uint16_t)pack_bf16x2(r, 0.f);
      else
        reinterpret_cast<float*>(vo)[i] = r;
    }
    if (lane == 0) so[row] = empty ? neg_inf() : M + __logf(wa + wb);
  }
}

}  // namespace

int launch_merge_partials(const RunArgs& r) {
  MergeParams p;
  p.plan = r.plan;
  p.o = static_cast<uint8_t*>(r.o);
  p.lse = r.lse;
  p.ws = r.ws;
  p.Hq = r.Hq;
  p.Hk = r.Hk;
  p.D = r.D;
  p.G = r.G;
  p.stream_at = r.stream_at;
  p.out_bf16 = r.out_dtype == FI_BF16;
  // decode rows hold G <= 8 packed rows; prefill tiles up to 128 (8 blocks of 16)
  const int z = r.stream_at == H_STREAM0 ? 1 : kMaxTileRows / kMergeRows;
  dim3 grid(std::max(1, r.max_tasks), r.Hk, z), block(kThreads);
  if (r.stream_at == H_STREAM0)
    hipLaunchKernelGGL(merge_partials_kernel<4>, grid, block, 0, (hipStream_t)r.hip_stream, p);
  else
    hipLaunchKernelGGL(merge_partials_kernel<1>, grid, block, 0, (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return FI_OK;
}

int launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb, void* vo,
                       float* so, int64_t n_rows, int32_t head_dim, fi_dtype vdt, fi_dtype odt,
                       void* stream) {
  if (n_rows == 0) return FI_OK;
  const int64_t blocks = std::min<int64_t>((n_rows + kThreads / 64 - 1) / (kThreads / 64), 65536);
  dim3 grid((unsigned)blocks), block(kThreads);
  auto* A = static_cast<const uint8_t*>(va);
  auto* Bv = static_cast<const uint8_t*>(vb);
  auto* O = static_cast<uint8_t*>(vo);
  hipStream_t s = (hipStream_t)stream;
  if (vdt == FI_BF16 && odt == FI_BF16)
    hipLaunchKernelGGL((merge_state_kernel<BF16, BF16>), grid, block, 0, s, A, sa, Bv, sb, O, so, n_rows, head_dim);
  else if (vdt == FI_F32 && odt == FI_BF16)
    hipLaunchKernelGGL((merge_state_kernel<F32, BF16>), grid, block, 0, s, A, sa, Bv, sb, O, so, n_rows, head_dim);
  else if (vdt == FI_F32 && odt == FI_F32)
    hipLaunchKernelGGL((merge_state_kernel<F32, F32>), grid, block, 0, s, A, sa, Bv, sb, O, so, n_rows, head_dim);
  else
    return set_error(FI_ERR_UNSUPPORTED, "merge_state: dtype combination");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "merge_state launch: %s", hipGetErrorString(e));
  return FI_OK;
}

}  // namespace fi
