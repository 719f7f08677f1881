// decode.hip -- persistent batch-decode kernel over a paged KV cache (gfx950).
//
// Operation (FlashInfer pages): one query token per row attends to the KV
// tokens of its request, gathered page by page through kv_indices
// (serving-engine page, "Page-Level Attention"); the G query heads that share
// a KV head are packed into one row so each K/V byte is read once for all of
// them (talk page, "Head Group Packing"); a long request is split over
// workers by the plan and each worker emits a partial (output, log-sum-exp)
// state (serving-engine page, "FlashDecoding: Parallel KV Split"; paper
// page, fixed-grid persistent kernels).
//
// Mapping.  grid = (workers, KV heads), 256 threads = 4 waves.  A workgroup
// walks its plan items; the 4 waves of the workgroup share an item and take
// its 16-token chunks round-robin, each with its own online-softmax state,
// merged through LDS when the item ends.  Per chunk a wave:
//   - loads K as the A operand of one v_mfma_f32_16x16x32_bf16 per 32 dims
//     (lane l: token l%16, dims 8*(l/16)..+8 of the slice; 16-byte loads),
//     with the packed query heads as the B operand (zero columns past G), so
//     S[token][head] lands in 4 registers per lane;
//   - loads V in row order (lane l: token group l/NC, 16-byte piece l%NC) and
//     accumulates P.V on the vector ALU;
//   - exchanges P and the rescale factors of the chunk through a 1 KiB LDS
//     slab private to the wave.
// Loads of the next chunk are issued before the current chunk is computed.
// All exponentials are base 2 with log2(e) folded into the logit scale.
#include "device_common.h"
#include "fi_internal.h"

namespace fi {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 16;

struct DecodeParams {
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
  int32_t page_shift;  // log2(P) when P is a power of two >= 16, else -1
  int32_t stream_at;
  float scale_log2;    // sm_scale * log2(e)
  float scale;         // sm_scale
  float cap;           // soft-cap; 0 = off
};

template <typename T, int D>
struct Shape {
  static constexpr int E = 16 / T::kBytes;  // elements per 16-byte piece
  static constexpr int NC = D / E;          // pieces per K/V row
  static constexpr int TPL = 64 / NC;       // tokens per V load instruction
  static constexpr int NL = kChunk / TPL;   // V loads per lane per chunk
  static constexpr int NK = D / (4 * E);    // K loads per lane per chunk
  static_assert(NL == NK, "K and V loads per chunk differ");
};

template <typename T, int NK>
__device__ __forceinline__ f32x4_t qk_mfma(const u32x4_t (&kp)[NK], const u32x4_t (&qp)[NK]) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NK; ++p) {
    if constexpr (T::kBytes == 2) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kp[p]),
                                                  __builtin_bit_cast(bf16x8_t, qp[p]), s, 0, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kp[p][e]),
                                                 __uint_as_float(qp[p][e]), s, 0, 0, 0);
    }
  }
  return s;
}

template <typename OT>
__device__ __forceinline__ void store_out(uint8_t* base, int64_t idx, float v) {
  if constexpr (OT::kBytes == 2)
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(base)[idx] = v;
}

template <typename T, int D, int G, bool FAST, typename OT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams a) {
  using SH = Shape<T, D>;
  constexpr int E = SH::E, NC = SH::NC, NL = SH::NL, NK = SH::NK;
  constexpr int TB = T::kBytes;

  __shared__ __align__(16) float p_lds[kWaves][G][kChunk];
  __shared__ float alpha_lds[kWaves][G];
  __shared__ float m_lds[kWaves][G];
  __shared__ float l_lds[kWaves][G];
  __shared__ __align__(16) float acc_lds[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  const int64_t tok_stride = (int64_t)Hk * D;       // elements between slots
  const int64_t half_stride = (int64_t)P * tok_stride;  // K block -> V block
  const int64_t page_stride = 2 * half_stride;

  const int tk = lane & 15;   // K / S lane: token within chunk, head column
  const int kq = lane >> 4;   // K / S lane: dim slice / token quad
  const int vr = lane / NC;   // V lane: token group
  const int vc = lane % NC;   // V lane: 16-byte piece of the row
  const int hS = lane & 15;

  const int it_begin = wip[worker];
  const int it_end = wip[worker + 1];
  for (int it = it_begin; it < it_end; ++it) {
    const int row = items[4 * it + 0];
    const int pb = items[4 * it + 1];
    const int pe = items[4 * it + 2];
    const int slot = items[4 * it + 3];
    const int req = rows[4 * row + 0];
    const int kvb = a.kv_indptr[req];
    const int npg = a.kv_indptr[req + 1] - kvb;
    const int kv_len = npg ? (npg - 1) * P + a.kv_last[req] : 0;
    const int t0 = pb * P;
    const int t1 = min(pe * P, kv_len);
    const int qrow = a.qo_indptr ? a.qo_indptr[req] : req;
    const int nch = t1 > t0 ? (t1 - t0 + kChunk - 1) / kChunk : 0;

    // packed query heads as MFMA B operand: column hS, dims of slice kq
    u32x4_t qp[NK];
    {
      const uint8_t* qb =
          a.q + ((int64_t)qrow * a.Hq + (int64_t)g * G + (hS < G ? hS : 0)) * D * TB;
#pragma unroll
      for (int p = 0; p < NK; ++p) {
        qp[p] = load16(qb + (int64_t)(4 * p + kq) * 16);
        if (hS >= G) qp[p] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    float m_run = neg_inf();  // S lane: running max (log2 domain) of head hS
    float l_part = 0.f;       // S lane: partial normaliser of head hS
    float acc[G][E];          // V lane: partial P.V of its tokens
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.f;

    auto page_of = [&](int tok) -> int64_t {
      int pg = a.kv_indices[kvb + (FAST ? (tok >> a.page_shift) : tok / P)];
      return (uint32_t)pg < (uint64_t)a.pool_pages ? (int64_t)pg : 0;  // never read outside the pool
    };

    // Issue the K and V loads of chunk c.
    auto load_chunk = [&](int c, u32x4_t (&kb)[NK], u32x4_t (&vb)[NL]) {
      const int cs = t0 + c * kChunk;
      if constexpr (FAST) {
        const int64_t page = page_of(cs);
        const int slot0 = cs & (P - 1);
        const uint8_t* pbase = a.kv + (page * page_stride + (int64_t)g * D) * TB;
        const int tkk = min(cs + tk, t1 - 1) - cs;
        const uint8_t* kaddr = pbase + ((int64_t)(slot0 + tkk) * tok_stride) * TB;
#pragma unroll
        for (int p = 0; p < NK; ++p) kb[p] = load16(kaddr + (4 * p + kq) * 16);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          const int tv = min(cs + vr * NL + k, t1 - 1) - cs;
          vb[k] = load16(pbase + (half_stride + (int64_t)(slot0 + tv) * tok_stride) * TB + vc * 16);
        }
      } else {
        const int tkk = min(cs + tk, t1 - 1);
        const uint8_t* kaddr =
            a.kv + (page_of(tkk) * page_stride + (int64_t)(tkk % P) * tok_stride + (int64_t)g * D) * TB;
#pragma unroll
        for (int p = 0; p < NK; ++p) kb[p] = load16(kaddr + (4 * p + kq) * 16);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          const int tv = min(cs + vr * NL + k, t1 - 1);
          vb[k] = load16(a.kv + (page_of(tv) * page_stride + half_stride +
                                 (int64_t)(tv % P) * tok_stride + (int64_t)g * D) * TB + vc * 16);
        }
      }
    };

    auto compute_chunk = [&](int c, const u32x4_t (&kb)[NK], const u32x4_t (&vb)[NL]) {
      const int cs = t0 + c * kChunk;
      f32x4_t s = qk_mfma<T, NK>(kb, qp);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = s[r];
        if (a.cap > 0.f)
          v = a.cap * tanh_from_exp(v * a.scale / a.cap) * kLog2e;
        else
          v *= a.scale_log2;
        x[r] = (cs + 4 * kq + r < t1) ? v : neg_inf();
      }
      float cm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      cm = fmaxf(cm, __shfl_xor(cm, 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      const float m_new = fmaxf(m_run, cm);
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[r] - m_use);
      l_part = l_part * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m_run = m_new;
      if (hS < G) {
        *reinterpret_cast<f32x4_t*>(&p_lds[wave][hS][4 * kq]) = f32x4_t{p[0], p[1], p[2], p[3]};
        if (kq == 0) alpha_lds[wave][hS] = alpha;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float pv[G][NL];
      float al[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        al[h] = alpha_lds[wave][h];
#pragma unroll
        for (int k = 0; k < NL; ++k) pv[h][k] = p_lds[wave][h][vr * NL + k];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= al[h];
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        // a V token past t1 was loaded from a clamped address; give it zero weight
        const bool valid = cs + vr * NL + k < t1;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float v = valid ? piece_elem<T>(vb[k], e) : 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pv[h][k], v, acc[h][e]);
        }
      }
    };

    // chunks of this wave: wave, wave + 4, ...; two register sets in flight
    {
      u32x4_t kA[NK], vA[NL], kB[NK], vB[NL];
      int c = wave;
      if (c < nch) load_chunk(c, kA, vA);
      for (; c < nch; c += 2 * kWaves) {
        if (c + kWaves < nch) load_chunk(c + kWaves, kB, vB);
        compute_chunk(c, kA, vA);
        if (c + kWaves >= nch) break;
        if (c + 2 * kWaves < nch) load_chunk(c + 2 * kWaves, kA, vA);
        compute_chunk(c + kWaves, kB, vB);
      }
    }

    // wave totals: P.V over the token groups, normaliser over the token quads
#pragma unroll
    for (int off = NC; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
    if (lane < G) {
      m_lds[wave][lane] = m_run;
      l_lds[wave][lane] = l_part;
    }
    if (vr == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc_lds[wave][h][vc * E + e] = acc[h][e];
    }
    __syncthreads();
    // merge the four wave states of this item and write it out
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int h = idx / D, d = idx % D;
      float M = neg_inf();
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, m_lds[wv][h]);
      float out = 0.f, lse2 = neg_inf();
      if (M != neg_inf()) {
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
          const float sc = fast_exp2(m_lds[wv][h] - M);
          L += l_lds[wv][h] * sc;
          O += acc_lds[wv][h][d] * sc;
        }
        out = O / L;
        lse2 = M + fast_log2(L);
      }
      const int head = g * G + h;
      if (slot < 0) {
        store_out<OT>(a.o, ((int64_t)qrow * a.Hq + head) * D + d, out);
        if (a.lse && d == 0) a.lse[(int64_t)qrow * a.Hq + head] = lse2 * kLn2;
      } else {
        const int64_t prow = ((int64_t)slot * Hk + g) * G + h;
        ws_o[prow * D + d] = out;
        if (d == 0) ws_lse[prow] = lse2 * kLn2;
      }
    }
    __syncthreads();
  }
}

template <typename T, int D, int G, bool FAST, typename OT>
int launch_t(const RunArgs& r, const DecodeParams& p) {
  dim3 grid(r.workers, r.Hk), block(kThreads);
  hipLaunchKernelGGL((decode_kernel<T, D, G, FAST, OT>), grid, block, 0,
                     (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return FI_OK;
}

template <typename T, int D, int G, typename OT>
int launch_fast(const RunArgs& r, const DecodeParams& p) {
  return p.page_shift >= 0 ? launch_t<T, D, G, true, OT>(r, p) : launch_t<T, D, G, false, OT>(r, p);
}

template <typename T, int D, typename OT>
int launch_g(const RunArgs& r, const DecodeParams& p) {
  switch (r.G) {
    case 1: return launch_fast<T, D, 1, OT>(r, p);
    case 2: return launch_fast<T, D, 2, OT>(r, p);
    case 4: return launch_fast<T, D, 4, OT>(r, p);
    case 8: return launch_fast<T, D, 8, OT>(r, p);
  }
  return set_error(FI_ERR_UNSUPPORTED, "decode: group size %d", r.G);
}

template <typename T, typename OT>
int launch_d(const RunArgs& r, const DecodeParams& p) {
  if (r.D == 64) return launch_g<T, 64, OT>(r, p);
  if (r.D == 128) return launch_g<T, 128, OT>(r, p);
  return set_error(FI_ERR_UNSUPPORTED, "decode: head_dim %d", r.D);
}

}  // namespace

int launch_decode(const RunArgs& r) {
  DecodeParams p;
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
  p.page_shift = -1;
  if (r.P >= 16 && (r.P & (r.P - 1)) == 0) {
    int s = 0;
    while ((1 << s) < r.P) ++s;
    p.page_shift = s;
  }
  p.stream_at = r.stream_at;
  p.scale = r.sm_scale;
  p.scale_log2 = r.sm_scale * kLog2e;
  p.cap = r.soft_cap;
  if (r.dtype == FI_BF16 && r.out_dtype == FI_BF16) return launch_d<BF16, BF16>(r, p);
  if (r.dtype == FI_BF16 && r.out_dtype == FI_F32) return launch_d<BF16, F32>(r, p);
  if (r.dtype == FI_F32 && r.out_dtype == FI_F32) return launch_d<F32, F32>(r, p);
  return set_error(FI_ERR_UNSUPPORTED, "decode: dtype combination");
}

}  // namespace fi
