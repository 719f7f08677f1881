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
// Mapping.  grid = workers x KV heads (1-D, XCD-major), 512 threads = 8
// waves.  A work item is a tile of up to 128 packed rows (packed row r =
// token r / G, head r % G of the KV head's group) times a range of KV pages.
// Wave w owns packed rows 16w .. 16w + 15; lane l holds row l % 16 together
// with the three other lanes l % 16 + 16 k.  Per 64-key KV tile:
//   - the workgroup gathers K (row-major, padded rows) and V (transposed,
//     V^T[dim][key] in fp16, keys permuted inside each 32-key group) into
//     LDS, double buffered, with the next tile's global loads in flight;
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = the
//     wave's packed query rows in registers): lane l holds keys
//     16 m + 4 (l / 16) + r of query l % 16, so the row max and sum need two
//     cross-lane exchanges;
//   - online softmax in registers (base-2 exponentials, scale folded in);
//   - O^T += V^T P^T with v_mfma_f32_16x16x32_f16; P^T comes straight from
//     the S^T registers because the V^T key order in LDS matches the order in
//     which the S^T accumulator holds keys.  P (in [0, 1]) and V run in fp16:
//     bf16 V converts exactly in fp16's normal range (the conversion
//     saturates at +-65504), and fp16 keeps 11 bits of P where bf16 keeps 8,
//     which bounds the PV rounding error by 2^-11 max|v| even for rows that
//     see only a few keys.
#include "device_common.h"
#include "fi_internal.h"

namespace fi {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
constexpr int kTileK = 64;            // keys per KV tile
constexpr int kVStride = kTileK + 8;  // V^T row stride (elements): 144 B
constexpr float kMaxSlack = 8.f;      // log2-domain headroom of the lazily updated running max

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
#define FI_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

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
  int32_t workers;
  int32_t page_shift;  // log2(P) when P is a power of two >= 16, else -1
  float scale_log2;
  float scale;
  float cap;
  float inv_cap;
};

// Position of key k (0..63) of a tile inside a V^T row.  With k = 32 s +
// 16 h + 4 g + j, the S^T accumulator of lane group g holds keys 4 g + j of
// both 16-key halves h of k-step s; position 32 s + 8 g + 4 h + j makes those
// 8 keys contiguous, one 16-byte read of the PV A operand.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

#define FI_LDS __attribute__((address_space(3)))

template <int D>
struct PShape {
  static constexpr int KRow = D * 2;            // bytes of one K row (no padding)
  static constexpr int KPiecesRow = D / 8;      // 16-byte pieces of one K row
  static constexpr int KDma = kTileK * D * 2 / 1024 / kWaves;  // direct-to-LDS K loads per wave
  static constexpr int KSteps = D / 32;         // MFMA k-steps of Q K^T
  static constexpr int DBlocks = D / 16;        // 16-dim output blocks
  static constexpr int VPiecesPerRow = D / 8;   // 16-byte pieces of one V row
};

template <int D, int G, bool FAST, bool CAP, typename OT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void prefill_kernel(PrefillParams a) {
  using SH = PShape<D>;
  static_assert(SH::KDma >= 1, "tile too small for the direct-to-LDS split");
  // K tile: row-major, the 16-byte piece p of key k stored at
  // p ^ (k % pieces-per-row), which stays inside the row
  __shared__ __align__(16) uint8_t k_lds[2][kTileK * SH::KRow];
  __shared__ __align__(16) uint16_t v_lds[2][D * kVStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give
  // each XCD a contiguous run of (head, worker) slots so that neighbouring
  // workers, which take neighbouring query tiles of the same request, share
  // one L2 and re-read its KV pages from there.
  int worker, g;
  {
    const int N = a.workers * a.Hk, q8 = N / 8, r8 = N % 8;
    const int x = blockIdx.x % 8, i = blockIdx.x / 8;
    const int s = x * q8 + min(x, r8) + i;
    g = s / a.workers;
    worker = s % a.workers;
  }
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
  // staging roles: direct-to-LDS K load j of wave w covers tile bytes
  // (w * KDma + j) * 1024 + 16 lane, i.e. key k_key(j), stored piece lane %
  // pieces-per-row; V keys 2 (tid % 32) + {0, 1} at piece tid / 32 (threads
  // past the row idle)
  auto k_key = [&](int j) { return ((wave * SH::KDma + j) * 1024 + 16 * lane) / SH::KRow; };
  const int k_pp = lane % SH::KPiecesRow;
  const int v_kp = tid & 31;
  const int v_piece = tid >> 5;
  const bool v_active = v_piece < SH::VPiecesPerRow;

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
    const int r = rb + kRowsPerWave * wave + l16;
    const bool row_valid = r < re;
    const int rc = row_valid ? r : re - 1;
    const int tok = rc / G;
    const int head = g * G + rc % G;
    const int causal_off = kv_len - qo_len;
    const int lim = min(a.causal ? causal_off + tok + 1 : kv_len, t1);
    const int r_first = min(rb + kRowsPerWave * wave, re - 1);
    const int wave_lim_min = min(a.causal ? causal_off + r_first / G + 1 : kv_len, t1);

    // packed query rows as the MFMA B operand (dims 32 ks + 8 g4 .. + 8)
    bf16x8_t qp[SH::KSteps];
    {
      const uint8_t* qb = a.q + ((int64_t)(qbase + tok) * a.Hq + head) * D * 2;
#pragma unroll
      for (int ks = 0; ks < SH::KSteps; ++ks)
        qp[ks] = __builtin_bit_cast(bf16x8_t, load16(qb + (32 * ks + 8 * g4) * 2));
    }
    f32x4_t oacc[SH::DBlocks];
#pragma unroll
    for (int d = 0; d < SH::DBlocks; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf();
    float l_part = 0.f;

    // ---- tile staging: K global -> LDS directly, V global -> registers ->
    // LDS (fp16, transposed); page ids fetched a tile ahead of their loads
    u32x4_t vreg[2];
    struct Pages {
      int k[SH::KDma];
      int v0, v1;
    };
    auto clamp_key = [&](int key) { return key < t1 ? key : t1 - 1; };
    auto page_idx = [&](int key) { return FAST ? key >> a.page_shift : key / P; };
    auto slot_of = [&](int key) { return FAST ? key & (P - 1) : key % P; };
    auto page_at = [&](int key) -> int {
      int pg = a.kv_indices[kvb + page_idx(key)];
      return (uint32_t)pg < (uint64_t)a.pool_pages ? pg : 0;  // never read outside the pool
    };
    auto fetch_pages = [&](int n) -> Pages {
      Pages pg;
#pragma unroll
      for (int j = 0; j < SH::KDma; ++j) pg.k[j] = 0;
      pg.v0 = pg.v1 = 0;
      if (n < ntiles) {
        const int ts = t0 + n * kTileK;
#pragma unroll
        for (int j = 0; j < SH::KDma; ++j) pg.k[j] = page_at(clamp_key(ts + k_key(j)));
        pg.v0 = page_at(clamp_key(ts + 2 * v_kp));
        pg.v1 = page_at(clamp_key(ts + 2 * v_kp + 1));
      }
      return pg;
    };
    // Keys past t1 read the clamped (valid, finite) last key: their logits
    // are masked and their P is exactly 0, so neither K nor V needs zeroing.
    auto load_tile = [&](int n, int buf, const Pages& pg) {
      const int ts = t0 + n * kTileK;
#pragma unroll
      for (int j = 0; j < SH::KDma; ++j) {
        const int key = k_key(j);
        const int kc = clamp_key(ts + key);
        const uint8_t* src = a.kv + ((int64_t)pg.k[j] * page_stride + (int64_t)slot_of(kc) * tok_stride +
                                     (int64_t)g * D) * 2 + (k_pp ^ (key & (SH::KPiecesRow - 1))) * 16;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (FI_LDS void*)(&k_lds[buf][(wave * SH::KDma + j) * 1024]), 16, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // K before V: the wait for V then covers K
      if (v_active) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int kc = clamp_key(ts + 2 * v_kp + s2);
          const uint8_t* src = a.kv + ((int64_t)(s2 ? pg.v1 : pg.v0) * page_stride + half_stride +
                                       (int64_t)slot_of(kc) * tok_stride + (int64_t)g * D) * 2;
          vreg[s2] = load16(src + v_piece * 16);
        }
      }
    };
    auto store_tile = [&](int buf) {
      if (v_active) {
        const int pos = vt_pos(2 * v_kp);
        const int dim0 = v_piece * 8;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = vreg[0][w], y = vreg[1][w];
          *reinterpret_cast<uint32_t*>(&v_lds[buf][(dim0 + 2 * w) * kVStride + pos]) =
              pack_f16_rtz(bf16_lo(x), bf16_lo(y));  // dim 2w, keys (2kp, 2kp+1)
          *reinterpret_cast<uint32_t*>(&v_lds[buf][(dim0 + 2 * w + 1) * kVStride + pos]) =
              pack_f16_rtz(bf16_hi(x), bf16_hi(y));  // dim 2w + 1
        }
      }
    };

    auto compute_tile = [&](int n, int buf) {
      const int ts = t0 + n * kTileK;
      // S^T = K Q^T: 4 blocks of 16 keys
      f32x4_t sacc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < SH::KSteps; ++ks) {
        bf16x8_t ka[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int key = 16 * mb + l16;
          const int pp = (4 * ks + g4) ^ (key & (SH::KPiecesRow - 1));
          ka[mb] = __builtin_bit_cast(bf16x8_t,
                                      *reinterpret_cast<const u32x4_t*>(&k_lds[buf][key * SH::KRow + pp * 16]));
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[mb], qp[ks], sacc[mb], 0, 0, 0);
      }
      // logits: with the cap, into the log2 domain now; without it, the
      // scale is applied inside the exponent below (order-preserving, > 0)
      if constexpr (CAP) {
        const float c_in = a.scale * a.inv_cap, c_out = a.cap * kLog2e;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[mb][e] = c_out * tanh_from_exp(sacc[mb][e] * c_in);
      }
      const float sc = CAP ? 1.f : a.scale_log2;
      if (__builtin_expect(ts + kTileK > wave_lim_min, 0)) {  // some key is hidden from some row
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[mb][e] = ts + 16 * mb + 4 * g4 + e < lim ? sacc[mb][e] : neg_inf();
      }
      float tmax = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
      tmax = fmaxf(tmax, fmaxf(fmaxf(fmaxf(sacc[2][0], sacc[2][1]), fmaxf(sacc[2][2], sacc[2][3])),
                               fmaxf(fmaxf(sacc[3][0], sacc[3][1]), fmaxf(sacc[3][2], sacc[3][3]))));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      tmax *= sc;  // into the log2 domain
      // the reference max only moves when a tile beats it by more than 2^8
      const float m_new = tmax > m_run + kMaxSlack ? tmax : m_run;
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[mb][e] = fast_exp2(fmaf(sacc[mb][e], sc, -m_use));
      const f32x4_t s01 = sacc[0] + sacc[1], s23 = sacc[2] + sacc[3];
      const f32x4_t s4 = s01 + s23;
      l_part = l_part * alpha + ((s4[0] + s4[1]) + (s4[2] + s4[3]));
      if (__builtin_expect(__any(alpha != 1.f), 0)) {  // wave-uniform; rare once the max settles
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d) oacc[d] *= alpha;
      }
      // O^T += V^T P^T over 2 k-steps of 32 keys
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f16x8_t pb8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb8[i] = (_Float16)sacc[2 * ks][i];
          pb8[4 + i] = (_Float16)sacc[2 * ks + 1][i];
        }
#pragma unroll
        for (int d0 = 0; d0 < SH::DBlocks; d0 += 4) {
          f16x8_t va[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            va[d] = __builtin_bit_cast(
                f16x8_t, *reinterpret_cast<const u32x4_t*>(
                             &v_lds[buf][(16 * (d0 + d) + l16) * kVStride + 32 * ks + 8 * g4]));
#pragma unroll
          for (int d = 0; d < 4; ++d)
            oacc[d0 + d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[d], pb8, oacc[d0 + d], 0, 0, 0);
        }
      }
    };

    // The compiler does not track direct-to-LDS loads: every thread waits
    // for all of its loads before the barrier that publishes a tile.
    Pages pg_next = fetch_pages(1);
    if (ntiles > 0) {
      load_tile(0, 0, fetch_pages(0));
      store_tile(0);
    }
    FI_WAIT_VMCNT(0);
    __syncthreads();
    for (int n = 0; n < ntiles; ++n) {
      const int buf = n & 1;
      if (n + 1 < ntiles) load_tile(n + 1, buf ^ 1, pg_next);
      pg_next = fetch_pages(n + 2);  // page ids one tile ahead of the loads
      compute_tile(n, buf);  // fully masked tiles of a wave give p = 0 and leave its state as is
      if (n + 1 < ntiles) store_tile(buf ^ 1);
      FI_WAIT_VMCNT(0);
      __syncthreads();
    }

    // ---- epilogue: normalise and write this lane's row (dims 16 d + 4 g4 + e)
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const bool empty = m_run == neg_inf() || !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_nat = empty ? neg_inf() : (m_run + fast_log2(l_tot)) * kLn2;
    if (row_valid) {
      if (slot < 0) {
        const int64_t orow = (int64_t)(qbase + tok) * a.Hq + head;
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d) {
          const int dim = 16 * d + 4 * g4;
          const float v0 = oacc[d][0] * inv, v1 = oacc[d][1] * inv;
          const float v2 = oacc[d][2] * inv, v3 = oacc[d][3] * inv;
          if constexpr (OT::kBytes == 2) {
            u32x2_t w;
            w[0] = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
            w[1] = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
            *reinterpret_cast<u32x2_t*>(a.o + (orow * D + dim) * 2) = w;
          } else {
            *reinterpret_cast<f32x4_t*>(a.o + (orow * D + dim) * 4) = f32x4_t{v0, v1, v2, v3};
          }
        }
        if (a.lse && g4 == 0) a.lse[orow] = lse_nat;
      } else {
        const int64_t prow = ((int64_t)slot * Hk + g) * kMaxTileRows + (r - rb);
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d)
          *reinterpret_cast<f32x4_t*>(ws_o + prow * D + 16 * d + 4 * g4) = oacc[d] * inv;
        if (g4 == 0) ws_lse[prow] = lse_nat;
      }
    }
  }
}

template <int D, int G, bool FAST, bool CAP, typename OT>
int launch_k(const RunArgs& r, const PrefillParams& p) {
  dim3 grid(r.workers * r.Hk), block(kThreads);
  hipLaunchKernelGGL((prefill_kernel<D, G, FAST, CAP, OT>), grid, block, 0, (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return FI_OK;
}

template <int D, int G, typename OT>
int launch_t(const RunArgs& r, const PrefillParams& p) {
  const bool fast = p.page_shift >= 0, cap = p.cap > 0.f;
  if (fast) return cap ? launch_k<D, G, true, true, OT>(r, p) : launch_k<D, G, true, false, OT>(r, p);
  return cap ? launch_k<D, G, false, true, OT>(r, p) : launch_k<D, G, false, false, OT>(r, p);
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
  p.workers = r.workers;
  p.scale = r.sm_scale;
  p.scale_log2 = r.sm_scale * kLog2e;
  p.cap = r.soft_cap;
  p.inv_cap = r.soft_cap > 0.f ? 1.f / r.soft_cap : 0.f;
  p.page_shift = -1;
  if (r.P >= 16 && (r.P & (r.P - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < r.P) ++sh;
    p.page_shift = sh;
  }
  if (r.out_dtype == FI_BF16) return launch_d<BF16>(r, p);
  return launch_d<F32>(r, p);
}

}  // namespace fi
