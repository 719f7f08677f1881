// prefill.hip -- persistent ragged batch-prefill kernel over a paged KV cache
// (gfx950, bf16, MFMA).
//
// Operation (FlashInfer pages): every query token of a request attends to the
// request's KV tokens, gathered page by page through kv_indices
// (serving-engine page, "Page-Level Attention", "Ragged Batching",
// batch_prefill_with_paged_kv_cache(..., causal=True)); pages are gathered
// into on-chip memory before the matrix cores consume them (paper page, "One
// format for every KV layout"); the plan may split a tile's KV range over
// workers, whose partial (o, lse) states are merged afterwards (paper page,
// "Load balancing that survives CUDA graphs").
//
// Mapping.  grid = (workers, KV heads), 256 threads = 4 waves.  A work item
// is a tile of up to 128 packed rows (packed row r = token r / G, head r % G
// of the KV head's group) times a range of KV pages.  Wave w owns packed rows
// 32w .. 32w + 31 of the tile; lane l holds row l % 32.  Per 64-key KV tile:
//   - the workgroup gathers K (row-major, padded rows) and V (transposed,
//     V^T[dim][key] in fp16, keys permuted within each 16-key group) into LDS, double
//     buffered, with the next tile's global loads in flight during compute;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = the
//     wave's packed query rows, kept in registers), so each lane owns the
//     logits of one query row: row max and sum need one cross-half exchange;
//   - online softmax in registers (base-2 exponentials, scale folded in);
//   - O^T += V^T P^T with v_mfma_f32_32x32x16_f16; P^T comes straight from
//     the S^T registers because the V^T key order in LDS matches the order in
//     which the S^T accumulator holds keys.  P (in [0, 1]) and V run in fp16
//     here: bf16 V converts exactly in fp16's normal range (the conversion
//     saturates at +-65504), and fp16 keeps 11 bits of P where bf16 keeps 8,
//     which bounds the PV rounding error by 2^-11 max|v| even for rows that
//     see only a few keys.
#include "device_common.h"
#include "fi_internal.h"

namespace fi {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileK = 64;         // keys per KV tile
constexpr int kVStride = kTileK + 8;  // V^T row stride (elements): 144 B, conflict-free 16 B reads

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

// Two fp32 values as an fp16 pair, rounding toward zero (exact for bf16
// inputs in fp16's normal range; saturates instead of overflowing).
__device__ __forceinline__ uint32_t pack_f16_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

struct PrefillParams {
  const int32_t* plan;
  const uint8_t* q;
  const uint8_t* kv;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last;
  uint8_t* o;
  float* lse;
  float* ws;
  int64_t pool_pages;
  int32_t Hq, Hk, P;
  int32_t causal;
  int32_t stream_at;
  float scale_log2;
  float scale;
  float cap;
};

// Position of key k (0..63) of a tile inside a V^T row: bits 2 and 3 swapped,
// so that the 8 keys lane half h needs for one MFMA k-step are contiguous.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <int D>
struct PShape {
  static constexpr int KStride = D + 8;      // K row stride (elements): rows 16 B apart in bank space
  static constexpr int KPieces = D / 32;     // 16-byte K pieces per thread per tile
  static constexpr int VPieces = D / 64;     // 16-byte V pieces per key, per thread per tile
  static constexpr int KSteps = D / 16;      // MFMA k-steps of Q K^T
  static constexpr int DBlocks = D / 32;     // 32-dim output blocks
};

template <int D, int G, typename OT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillParams a) {
  using SH = PShape<D>;
  constexpr int KS = SH::KStride;
  __shared__ __align__(16) uint16_t k_lds[2][kTileK * KS];
  __shared__ __align__(16) uint16_t v_lds[2][D * kVStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int worker = blockIdx.x;
  const int g = blockIdx.y;
  const int32_t* sd = a.plan + a.stream_at;
  const int32_t* rows = a.plan + sd[S_OFF_ROWS];
  const int32_t* items = a.plan + sd[S_OFF_ITEMS];
  const int32_t* wip = a.plan + sd[S_OFF_WIP];
  float* ws_o = a.ws + sd[S_WS_O];
  float* ws_lse = a.ws + sd[S_WS_LSE];
  const int P = a.P;
  const int Hk = a.Hk;
  const int64_t tok_stride = (int64_t)Hk * D;
  const int64_t half_stride = (int64_t)P * tok_stride;
  const int64_t page_stride = 2 * half_stride;

  const int it_begin = wip[worker];
  const int it_end = wip[worker + 1];
  for (int it = it_begin; it < it_end; ++it) {
    const int row = items[4 * it + 0];
    const int pb = items[4 * it + 1];
    const int pe = items[4 * it + 2];
    const int slot = items[4 * it + 3];
    const int req = rows[4 * row + 0];
    const int rb = rows[4 * row + 1];
    const int re = rows[4 * row + 2];
    const int kvb = a.kv_indptr[req];
    const int npg = a.kv_indptr[req + 1] - kvb;
    const int kv_len = npg ? (npg - 1) * P + a.kv_last[req] : 0;
    const int qbase = a.qo_indptr[req];
    const int qo_len = a.qo_indptr[req + 1] - qbase;
    const int t0 = pb * P;
    const int t1 = min(pe * P, kv_len);
    const int ntiles = t1 > t0 ? (t1 - t0 + kTileK - 1) / kTileK : 0;

    // this lane's packed row, its token, head and key limit
    const int r = rb + 32 * wave + l32;
    const bool row_valid = r < re;
    const int rc = row_valid ? r : re - 1;
    const int tok = rc / G;
    const int head = g * G + rc % G;
    const int lim = min(a.causal ? kv_len - qo_len + tok + 1 : kv_len, t1);
    // the wave's largest limit (limits grow with the packed row)
    const int r_last = min(rb + 32 * wave + 31, re - 1);
    const bool wave_has_rows = rb + 32 * wave < re;
    const int wave_lim = min(a.causal ? kv_len - qo_len + r_last / G + 1 : kv_len, t1);

    // packed query rows as the MFMA B operand (dims 16 kk + 8 hh .. + 8)
    bf16x8_t qp[SH::KSteps];
    {
      const uint8_t* qb = a.q + ((int64_t)(qbase + tok) * a.Hq + head) * D * 2;
#pragma unroll
      for (int kk = 0; kk < SH::KSteps; ++kk)
        qp[kk] = __builtin_bit_cast(bf16x8_t, load16(qb + (16 * kk + 8 * hh) * 2));
    }
    f32x16_t oacc[SH::DBlocks];
#pragma unroll
    for (int d = 0; d < SH::DBlocks; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
    float m_run = neg_inf();
    float l_part = 0.f;

    // ---- tile staging: global -> registers -> LDS
    u32x4_t kreg[SH::KPieces];
    u32x4_t vreg[2][SH::VPieces];
    auto page_of = [&](int tok_) -> int64_t {
      int pg = a.kv_indices[kvb + tok_ / P];
      return (uint32_t)pg < (uint64_t)a.pool_pages ? (int64_t)pg : 0;  // never read outside the pool
    };
    auto load_tile = [&](int n) {
      const int ts = t0 + n * kTileK;
      {  // K: key tid / 4, pieces (tid % 4) * KPieces ..
        const int key = ts + (tid >> 2);
        const bool valid = key < t1;
        const int kc = valid ? key : t1 - 1;
        const uint8_t* src = a.kv + (page_of(kc) * page_stride + (int64_t)(kc % P) * tok_stride +
                                     (int64_t)g * D) * 2 + (tid & 3) * SH::KPieces * 16;
#pragma unroll
        for (int j = 0; j < SH::KPieces; ++j)
          kreg[j] = valid ? load16(src + j * 16) : u32x4_t{0u, 0u, 0u, 0u};
      }
      {  // V: keys 2 (tid % 32) + {0, 1}, pieces tid / 32 + 8 j
        const int kp = tid & 31;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int key = ts + 2 * kp + s;
          const bool valid = key < t1;
          const int kc = valid ? key : t1 - 1;
          const uint8_t* src = a.kv + (page_of(kc) * page_stride + half_stride +
                                       (int64_t)(kc % P) * tok_stride + (int64_t)g * D) * 2;
#pragma unroll
          for (int j = 0; j < SH::VPieces; ++j)
            vreg[s][j] = valid ? load16(src + ((tid >> 5) + 8 * j) * 16) : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_tile = [&](int buf) {
      uint16_t* kd = &k_lds[buf][(tid >> 2) * KS + (tid & 3) * SH::KPieces * 8];
#pragma unroll
      for (int j = 0; j < SH::KPieces; ++j) *reinterpret_cast<u32x4_t*>(kd + 8 * j) = kreg[j];
      const int kp = tid & 31;
      const int pos = vt_pos(2 * kp);
#pragma unroll
      for (int j = 0; j < SH::VPieces; ++j) {
        const int dim0 = ((tid >> 5) + 8 * j) * 8;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = vreg[0][j][w], y = vreg[1][j][w];
          const uint32_t lo = pack_f16_rtz(bf16_lo(x), bf16_lo(y));  // dim 2w, keys (2kp, 2kp+1)
          const uint32_t hi = pack_f16_rtz(bf16_hi(x), bf16_hi(y));  // dim 2w + 1
          *reinterpret_cast<uint32_t*>(&v_lds[buf][(dim0 + 2 * w) * kVStride + pos]) = lo;
          *reinterpret_cast<uint32_t*>(&v_lds[buf][(dim0 + 2 * w + 1) * kVStride + pos]) = hi;
        }
      }
    };

    auto compute_tile = [&](int n, int buf) {
      const int ts = t0 + n * kTileK;
      if (!wave_has_rows || ts >= wave_lim) return;  // nothing visible for this wave
      f32x16_t sacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[mb][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < SH::KSteps; ++kk) {
          const bf16x8_t ka = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(&k_lds[buf][(32 * mb + l32) * KS + 16 * kk + 8 * hh]));
          sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qp[kk], sacc[mb], 0, 0, 0);
        }
      }
      // logits: scale (and cap), mask, log2 domain
      float tmax = neg_inf();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = ts + 32 * mb + 8 * (e >> 2) + 4 * hh + (e & 3);
          float v = sacc[mb][e];
          if (a.cap > 0.f)
            v = a.cap * tanh_from_exp(v * a.scale / a.cap) * kLog2e;
          else
            v *= a.scale_log2;
          v = key < lim ? v : neg_inf();
          sacc[mb][e] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(sacc[mb][e] - m_use);
          sacc[mb][e] = p;
          psum += p;
        }
      l_part = l_part * alpha + psum;
#pragma unroll
      for (int d = 0; d < SH::DBlocks; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
      // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int mb = ks >> 1;
        const int e0 = 8 * (ks & 1);
        f16x8_t pb8;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb8[i] = (_Float16)sacc[mb][e0 + i];
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d) {
          const f16x8_t va = __builtin_bit_cast(
              f16x8_t,
              *reinterpret_cast<const u32x4_t*>(&v_lds[buf][(32 * d + l32) * kVStride + 16 * ks + 8 * hh]));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb8, oacc[d], 0, 0, 0);
        }
      }
    };

    if (ntiles > 0) {
      load_tile(0);
      store_tile(0);
    }
    __syncthreads();
    for (int n = 0; n < ntiles; ++n) {
      const int buf = n & 1;
      if (n + 1 < ntiles) load_tile(n + 1);
      compute_tile(n, buf);
      if (n + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: normalise and write this lane's row
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    const bool empty = m_run == neg_inf() || !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_nat = empty ? neg_inf() : (m_run + fast_log2(l_tot)) * kLn2;
    if (row_valid) {
      if (slot < 0) {
        const int64_t orow = (int64_t)(qbase + tok) * a.Hq + head;
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int dim = 32 * d + 8 * e4 + 4 * hh;
            const float v0 = oacc[d][4 * e4 + 0] * inv, v1 = oacc[d][4 * e4 + 1] * inv;
            const float v2 = oacc[d][4 * e4 + 2] * inv, v3 = oacc[d][4 * e4 + 3] * inv;
            if constexpr (OT::kBytes == 2) {
              u32x2_t w;
              w[0] = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
              w[1] = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
              *reinterpret_cast<u32x2_t*>(a.o + (orow * D + dim) * 2) = w;
            } else {
              *reinterpret_cast<f32x4_t*>(a.o + (orow * D + dim) * 4) = f32x4_t{v0, v1, v2, v3};
            }
          }
        if (a.lse && hh == 0) a.lse[orow] = lse_nat;
      } else {
        const int64_t prow = ((int64_t)slot * Hk + g) * kMaxTileRows + (r - rb);
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int dim = 32 * d + 8 * e4 + 4 * hh;
            *reinterpret_cast<f32x4_t*>(ws_o + prow * D + dim) =
                f32x4_t{oacc[d][4 * e4] * inv, oacc[d][4 * e4 + 1] * inv,
                        oacc[d][4 * e4 + 2] * inv, oacc[d][4 * e4 + 3] * inv};
          }
        if (hh == 0) ws_lse[prow] = lse_nat;
      }
    }
  }
}

template <int D, int G, typename OT>
int launch_t(const RunArgs& r, const PrefillParams& p) {
  dim3 grid(r.workers, r.Hk), block(kThreads);
  hipLaunchKernelGGL((prefill_kernel<D, G, OT>), grid, block, 0, (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return FI_OK;
}

template <int D, typename OT>
int launch_g(const RunArgs& r, const PrefillParams& p) {
  switch (r.G) {
    case 1: return launch_t<D, 1, OT>(r, p);
    case 2: return launch_t<D, 2, OT>(r, p);
    case 4: return launch_t<D, 4, OT>(r, p);
    case 8: return launch_t<D, 8, OT>(r, p);
  }
  return set_error(FI_ERR_UNSUPPORTED, "prefill: group size %d", r.G);
}

template <typename OT>
int launch_d(const RunArgs& r, const PrefillParams& p) {
  if (r.D == 64) return launch_g<64, OT>(r, p);
  if (r.D == 128) return launch_g<128, OT>(r, p);
  return set_error(FI_ERR_UNSUPPORTED, "prefill: head_dim %d", r.D);
}

}  // namespace

int launch_prefill(const RunArgs& r) {
  if (r.dtype != FI_BF16)
    return set_error(FI_ERR_UNSUPPORTED, "prefill tiles need bf16 q / kv (fp32 runs decode rows only)");
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
  p.pool_pages = r.pool_pages;
  p.Hq = r.Hq;
  p.Hk = r.Hk;
  p.P = r.P;
  p.causal = r.causal;
  p.stream_at = r.stream_at;
  p.scale = r.sm_scale;
  p.scale_log2 = r.sm_scale * kLog2e;
  p.cap = r.soft_cap;
  if (r.out_dtype == FI_BF16) return launch_d<BF16>(r, p);
  return launch_d<F32>(r, p);
}

}  // namespace fi
