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
// Mapping.  grid = (workers, KV heads), one wave (64 threads) per workgroup:
// each wave is a worker that walks its plan items alone, chunk after chunk
// of 16 tokens, with no barrier shared with other waves.  (The code is
// written for kWaves waves sharing an item -- chunks round-robin, states
// merged through LDS at the item's end -- and kWaves = 1 measured faster
// than 4 on batch decode: more, shorter workers end closer together.)  Per
// chunk a wave:
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

constexpr int kWaves = 1;  // waves per workgroup, sharing its items
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 16;
constexpr float kMaxSlack = 8.f;  // log2-domain headroom of the lazily updated running max

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
  int32_t* status;     // status word: kStatusBadPage when a page id is not below pool_pages
  int64_t pool_pages;
  int32_t Hq, Hk, P;
  int32_t page_shift;  // log2(P) when P is a power of two >= 16, else -1
  int32_t small_shift; // log2(P) when P is 1, 2, 4 or 8, else -1
  int32_t stream_at;
  float scale_log2;    // sm_scale * log2(e)
  float scale;         // sm_scale
  float cap;           // soft-cap; 0 = off
  float inv_cap;       // 1 / cap (0 when off)
  int32_t window;      // sliding window: keys seen before the query's own; -1 = none
  uint32_t rope_f[kRopeMaxPairs];  // rotary turn per position of pair d (2^-32 revolutions)
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

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// S = K Q^T for one chunk.  F16: the operands are fp16 (rotated q and k)
// rather than the storage type.
template <typename T, int NK, bool F16 = false>
__device__ __forceinline__ f32x4_t qk_mfma(const u32x4_t (&kp)[NK], const u32x4_t (&qp)[NK]) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NK; ++p) {
    if constexpr (T::kBytes == 2 && F16) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, kp[p]),
                                                 __builtin_bit_cast(f16x8_t, qp[p]), s, 0, 0, 0);
    } else if constexpr (T::kBytes == 2) {
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
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)pack_bf16x2(v, 0.f);
  else
    reinterpret_cast<float*>(base)[idx] = v;
}

template <typename T, int D, int G, bool FAST, typename OT, bool ROPE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams a) {
  using SH = Shape<T, D>;
  constexpr int E = SH::E, NC = SH::NC, NL = SH::NL, NK = SH::NK;
  constexpr int TB = T::kBytes;
  // rotary table in LDS (the lanes read it with their own dims)
  __shared__ uint32_t rope_tab[ROPE ? D / 2 : 1];
  if constexpr (ROPE) {
    for (int i = threadIdx.x; i < D / 2; i += kThreads) rope_tab[i] = a.rope_f[i];
    __syncthreads();
  }

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
  const int32_t* items = a.plan + sd[S_OFF_ITEMS];
  const int32_t* meta = a.plan + sd[S_OFF_META];
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

  uint32_t bad_page = 0;  // a page id outside the pool was read (page 0 was used instead)
  const int it_begin = wip[worker];
  const int it_end = wip[worker + 1];
  for (int it = it_begin; it < it_end; ++it) {
    // the item and its request's record: two independent loads
    const int pb = items[4 * it + 1];
    const int pe = items[4 * it + 2];
    const int slot = items[4 * it + 3];
    const int32_t* im = meta + kMetaInts * it;
    const int kvb = im[M_KVB];
    const int kv_len = im[M_KVLEN];
    const int t0 = pb * P;
    const int t1 = min(pe * P, kv_len);
    // first key inside the window (keys before it in the first page are masked)
    const int klo = a.window >= 0 && kv_len - 1 > a.window ? kv_len - 1 - a.window : 0;
    const int qrow = im[M_QOBASE];
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
      // rotary embedding: the query sits at position kv_len - 1; piece
      // 4 p + kq holds dims E (4 p + kq) .., its partner D / 2 further
      if constexpr (ROPE) {
#pragma unroll
        for (int p = 0; p < NK / 2; ++p)
          rope_pieces<T>(qp[p], qp[p + NK / 2], (const FI_LDS uint32_t*)rope_tab + E * (4 * p + kq), kv_len - 1);
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
      const bool ok = (uint32_t)pg < (uint64_t)a.pool_pages;
      bad_page |= !ok;
      return ok ? (int64_t)pg : 0;  // never read outside the pool
    };
    // Page ids of this wave's chunks, 64 at a time: lane j holds the page of
    // the wave's chunk 64 * batch + j, read back with readlane when its loads
    // are issued, so no page lookup sits in front of the K/V loads.
    int pid_vec = 0;
    auto load_pids = [&](int batch) {
      const int c = wave + kWaves * (64 * batch + lane);
      pid_vec = c < nch ? (int)page_of(t0 + c * kChunk) : 0;
    };

    // Issue the K and V loads of chunk c (the wave's kth-th chunk).
    auto load_chunk = [&](int c, int kth, u32x4_t (&kb)[NK], u32x4_t (&vb)[NL]) {
      const int cs = t0 + c * kChunk;
      if constexpr (FAST) {
        if ((kth & 63) == 0) load_pids(kth >> 6);
        const int64_t page = __builtin_amdgcn_readlane(pid_vec, kth & 63);
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
      f32x4_t s;
      if constexpr (ROPE) {  // the lane's key (token cs + tk) turned to its position
        u32x4_t kr[NK];
#pragma unroll
        for (int p = 0; p < NK; ++p) kr[p] = kb[p];
#pragma unroll
        for (int p = 0; p < NK / 2; ++p)
          rope_pieces<T>(kr[p], kr[p + NK / 2], (const FI_LDS uint32_t*)rope_tab + E * (4 * p + kq), cs + tk);
        s = qk_mfma<T, NK, true>(kr, qp);
      } else {
        s = qk_mfma<T, NK>(kb, qp);
      }
      float x[4];
      if (a.cap > 0.f) {
        const float c_in = a.scale * a.inv_cap, c_out = a.cap * kLog2e;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = c_out * tanh_from_exp(s[r] * c_in);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = s[r] * a.scale_log2;
      }
      if (cs + kChunk > t1) {  // tail chunk
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (cs + 4 * kq + r < t1) ? x[r] : neg_inf();
      }
      if (cs < klo) {  // chunk starts before the window
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (cs + 4 * kq + r >= klo) ? x[r] : neg_inf();
      }
      float cm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      cm = fmaxf(cm, __shfl_xor(cm, 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      // The reference max only moves when the chunk beats it by more than
      // 2^8: weights stay <= 256 (safe in fp32) and most chunks need no rescale.
      const float m_new = cm > m_run + kMaxSlack ? cm : m_run;
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
      bool rescale = false;
#pragma unroll
      for (int h = 0; h < G; ++h) rescale |= al[h] != 1.f;
      if (rescale) {  // wave-uniform: al[] is the same LDS value in every lane
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= al[h];
      }
      if (cs + kChunk <= t1) {  // whole chunk valid (wave-uniform)
#pragma unroll
        for (int k = 0; k < NL; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float v = piece_elem<T>(vb[k], e);
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pv[h][k], v, acc[h][e]);
          }
      } else {
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
      }
    };

    // chunks of this wave: wave + 4 k, k = 0, 1, ...; two register sets in flight
    {
      u32x4_t kA[NK], vA[NL], kB[NK], vB[NL];
      const int myn = nch > wave ? (nch - wave + kWaves - 1) / kWaves : 0;
      if (myn > 0) load_chunk(wave, 0, kA, vA);
      for (int k = 0; k < myn; k += 2) {
        if (k + 1 < myn) load_chunk(wave + kWaves * (k + 1), k + 1, kB, vB);
        compute_chunk(wave + kWaves * k, kA, vA);
        if (k + 1 >= myn) break;
        if (k + 2 < myn) load_chunk(wave + kWaves * (k + 2), k + 2, kA, vA);
        compute_chunk(wave + kWaves * (k + 1), kB, vB);
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
  report_status(a.status, bad_page, kStatusBadPage);
}

// ---------------------------------------------------------------------------
// bf16 decode with page_size a power of two: P.V on the matrix cores.  Pages
// of >= 16 tokens hold a whole chunk (one page id per chunk); with pages of
// 1, 2, 4 or 8 tokens (SMALLP: the column-vector sparse matrix of the talk
// page, Key Findings and "Block Sparse Matrix") a chunk spans several pages and
// each lane looks up the page of its own token.
//
// Per wave and 16-token chunk: K goes global -> VGPRs as the A operand of
// S = K Q^T (v_mfma_f32_16x16x32_bf16, as above); V goes global -> LDS by
// direct-to-LDS loads (no VGPRs held while in flight) into a two-stage ring
// private to the wave, row-major with the 16-byte pieces of token t stored at
// piece ^ (t mod pieces-per-row) to spread LDS banks; ds_read_b64_tr_b16 then
// returns, per lane, 4 consecutive tokens of one dim, which is the V^T A
// operand of v_mfma_f32_16x16x16_bf16; its B operand (tokens 4 (l/16) .. +3
// of head l % 16) is exactly how the S accumulator holds P, so P never leaves
// the lane.  P is split into bf16 hi + lo parts (two MFMAs), keeping ~16 bits.
// O^T accumulates in 4 registers per 16-dim block; lane l owns head l % 16.
// The compiler does not track direct-to-LDS loads, so the kernel waits on
// vmcnt itself before reading a stage.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
#define FI_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// 3 waves per SIMD; the rotary variant at D = 128 needs the registers of 2
template <int D, int G, typename OT, bool ROPE, bool SMALLP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ROPE && D == 128 ? 2 : 3, ROPE && D == 128 ? 2 : 3)))
void decode_mfma_kernel(DecodeParams a) {
  constexpr int RB = D * 2;              // bytes of one K / V row of one head
  constexpr int NP = RB / 16;            // 16-byte pieces per row
  constexpr int NK = D / 32;             // K loads per lane per chunk
  constexpr int NV = kChunk * RB / 1024; // direct-to-LDS V loads per wave per chunk
  constexpr int NB = D / 16;             // 16-dim output blocks
  constexpr int kStage = kChunk * RB;    // bytes of one V stage
  static_assert(NK == NV, "one K and one V load per 32 dims");
  // vector-memory operations issued per chunk: K and V loads, and with small
  // pages the page-id load of the chunk two ahead
  constexpr int kChunkOps = 2 * NK + (SMALLP ? 1 : 0);

  __shared__ __align__(16) uint8_t vring[kWaves][2][kStage];
  __shared__ float m_lds[kWaves][G];
  __shared__ float l_lds[kWaves][G];
  // rotary table in LDS (the lanes read it with their own dims)
  __shared__ uint32_t rope_tab[ROPE ? D / 2 : 1];
  if constexpr (ROPE) {
    for (int i = threadIdx.x; i < D / 2; i += kThreads) rope_tab[i] = a.rope_f[i];
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int worker = blockIdx.x;
  const int g = blockIdx.y;
  const int32_t* sd = a.plan + a.stream_at;
  const int32_t* items = a.plan + sd[S_OFF_ITEMS];
  const int32_t* meta = a.plan + sd[S_OFF_META];
  const int32_t* wip = a.plan + sd[S_OFF_WIP];
  float* ws_o = a.ws + sd[S_WS_O];
  float* ws_lse = a.ws + sd[S_WS_LSE];
  const int P = a.P;
  const int Hk = a.Hk;
  const int64_t tok_stride = (int64_t)Hk * D;
  const int64_t half_stride = (int64_t)P * tok_stride;
  const int64_t page_stride = 2 * half_stride;
  const int tk = lane & 15;   // S lane: token row of K; head column
  const int kq = lane >> 4;   // S lane: dim slice of K, token quad of S
  const int hS = lane & 15;
  // direct-to-LDS V load k of lane l covers LDS bytes k*1024 + 16 l of the stage
  // = token (k*1024 + 16 l) / RB, stored piece ((16 l) % RB) / 16
  // transposed read: source lane (group gq, j) points at token 4 gq + j/4,
  // dims 16 b + 4 (j % 4) .. + 4
  const int tr_tok = 4 * kq + (tk >> 2);
  const int tr_sub = tk & 3;

  // epilogue scratch of its own: the V ring is already loading the next item
  __shared__ __align__(16) float acc_lds[kWaves * G * D];

  uint32_t bad_page = 0;  // a page id outside the pool was read (page 0 was used instead)
  const int it_begin = wip[worker];
  const int it_end = wip[worker + 1];
  // An item's record is loaded while the previous item runs, so only the
  // first item of a worker waits for it.
  struct Rec {
    int pb, pe, slot, kvb, kv_len, qrow;
  };
  auto load_rec = [&](int it) -> Rec {
    Rec r{0, 0, -1, 0, 0, 0};
    if (it < it_end) {
      const int32_t* im = meta + kMetaInts * it;
      r = Rec{items[4 * it + 1], items[4 * it + 2], items[4 * it + 3], im[M_KVB], im[M_KVLEN], im[M_QOBASE]};
    }
    return r;
  };
  // item geometry: keys [t0, t1), chunks of kChunk keys, the request's page
  // ids at kvb, and the first key inside the window (keys before it in the
  // item's first page are masked)
  struct Ctx {
    int t0, t1, kvb, nch, klo;
  };
  auto make_ctx = [&](const Rec& r) -> Ctx {
    const int t0 = r.pb * P, t1 = min(r.pe * P, r.kv_len);
    const int klo = a.window >= 0 && r.kv_len - 1 > a.window ? r.kv_len - 1 - a.window : 0;
    return Ctx{t0, t1, r.kvb, t1 > t0 ? (t1 - t0 + kChunk - 1) / kChunk : 0, klo};
  };
  // page id of the wave's chunk 64 batch + lane, loaded raw (checked where
  // it is read, so the load is not waited for on the spot)
  auto load_pids = [&](const Ctx& x, int batch) -> int {
    const int c = wave + kWaves * (64 * batch + lane);
    return c < x.nch ? a.kv_indices[x.kvb + ((x.t0 + c * kChunk) >> a.page_shift)] : 0;
  };
  // SMALLP (pages of 1, 2, 4 or 8 tokens): a chunk spans several pages, so
  // every lane looks up the page of its own token -- token tk of the wave's
  // kth chunk, clamped to the item's last key like the loads below -- raw,
  // two chunks ahead of its use.  The load is issued even for chunks past
  // the item's end (it then reads the item's first page id), so that every
  // chunk issues the same number of memory operations, which the waits in
  // the chunk loop count on.  Needs x.nch >= 1.
  auto load_id = [&](const Ctx& x, int kth) -> int {
    const int c = wave + kWaves * kth;
    const int tok = min(x.t0 + c * kChunk + tk, x.t1 - 1);
    return a.kv_indices[x.kvb + (c < x.nch ? tok >> a.small_shift : 0)];
  };
  // K -> registers, V -> LDS stage `st` for the wave's kth chunk c
  auto issue = [&](const Ctx& x, int pid_vec, int c, int kth, int st, u32x4_t (&kb)[NK]) {
    const int cs = x.t0 + c * kChunk;
    if constexpr (SMALLP) {
      // pid_vec is this lane's own page id (token tk).  K piece 4 p + kq and
      // V piece 4 k + kq of that token: V load k of lane l lands at stage
      // bytes k 1024 + 16 l, i.e. piece 4 k + l / 16 of token l % 16.
      const bool ok = (uint32_t)pid_vec < (uint64_t)a.pool_pages;
      bad_page |= !ok;
      const int64_t page = ok ? pid_vec : 0;  // never outside the pool
      const int tok = cs + min(tk, x.t1 - 1 - cs);
      const uint8_t* kaddr = a.kv + (page * page_stride + (int64_t)(tok & (P - 1)) * tok_stride + (int64_t)g * D) * 2;
#pragma unroll
      for (int p = 0; p < NK; ++p) kb[p] = load16(kaddr + (4 * p + kq) * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NV; ++k)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kaddr + half_stride * 2 + (4 * k + kq) * 16),
                                         (FI_LDS void*)(&vring[wave][st][k * 1024]), 16, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    const int pid = __builtin_amdgcn_readlane(pid_vec, kth & 63);
    const bool ok = (uint32_t)pid < (uint64_t)a.pool_pages;
    bad_page |= !ok;
    const int64_t page = ok ? pid : 0;  // never read outside the pool
    const int slot0 = cs & (P - 1);
    const int last = x.t1 - 1 - cs;  // last valid token of the chunk (may exceed 15)
    const uint8_t* pbase = a.kv + (page * page_stride + (int64_t)g * D) * 2;
    const uint8_t* kaddr = pbase + (int64_t)(slot0 + min(tk, last)) * tok_stride * 2;
#pragma unroll
    for (int p = 0; p < NK; ++p) kb[p] = load16(kaddr + (4 * p + kq) * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int t = (k * 1024 + 16 * lane) / RB;
      const int pp = ((16 * lane) % RB) / 16;
      const int piece = pp ^ (t & (NP - 1));
      const uint8_t* src = pbase + (half_stride + (int64_t)(slot0 + min(t, last)) * tok_stride) * 2 + piece * 16;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (FI_LDS void*)(&vring[wave][st][k * 1024]), 16, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // max / sum over the 4 lanes that hold one head (l, l ^ 16, l ^ 32, l ^ 48)
  auto head_max = [](float v) {
    auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    auto pq = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(pq[0]), __uint_as_float(pq[1]));
  };
  auto head_sum = [](float v) {
    auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    auto pq = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(pq[0]) + __uint_as_float(pq[1]);
  };

  // The first chunk of the next item is issued when the current item's
  // chunks are done, before its epilogue, and that item's page ids are
  // fetched during the current one: consecutive items of a worker overlap.
  u32x4_t kA[NK], kB[NK];
  Rec nxt = load_rec(it_begin);
  bool pre_issued = false;  // chunk 0 of the coming item is in kA / stage 0
  int pid_pre = 0;          // page ids (batch 0) of the coming item, when pre_issued
  int pid_pre1 = 0;         // SMALLP: the lane's page id in chunk 1 of the coming item
  for (int it = it_begin; it < it_end; ++it) {
    const Rec cur = nxt;
    nxt = load_rec(it + 1);
    const Ctx cx = make_ctx(cur);
    const int slot = cur.slot;
    const int t0 = cx.t0, t1 = cx.t1;
    const int qrow = cur.qrow;
    const int nch = cx.nch;
    const int myn = nch > wave ? (nch - wave + kWaves - 1) / kWaves : 0;
    int pid_vec = 0;
    int idA = 0, idB = 0;  // SMALLP: the lane's page ids of the next even / odd chunk to issue
    if constexpr (SMALLP) {
      if (nch > 0) {
        idA = load_id(cx, pre_issued ? 2 : 0);
        idB = pre_issued ? pid_pre1 : load_id(cx, 1);
      }
    } else {
      pid_vec = pre_issued ? pid_pre : load_pids(cx, 0);
    }

    u32x4_t qp[NK];
    {
      const uint8_t* qb = a.q + ((int64_t)qrow * a.Hq + (int64_t)g * G + (hS < G ? hS : 0)) * RB;
#pragma unroll
      for (int p = 0; p < NK; ++p) {
        qp[p] = load16(qb + (4 * p + kq) * 16);
        if (hS >= G) qp[p] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (ROPE) {  // the query sits at position kv_len - 1
#pragma unroll
        for (int p = 0; p < NK / 2; ++p)
          rope_pieces<BF16>(qp[p], qp[p + NK / 2], (const FI_LDS uint32_t*)rope_tab + 8 * (4 * p + kq),
                            cur.kv_len - 1);
      }
    }
    float m_run = neg_inf();
    float l_part = 0.f;
    f32x4_t oacc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // st (a constant at every call) is also the parity of kth
    auto issue_k = [&](int c, int kth, int st, u32x4_t (&kb)[NK]) {
      if constexpr (SMALLP) {
        int& id = st ? idB : idA;
        issue(cx, id, c, kth, st, kb);
        id = load_id(cx, kth + 2);
      } else {
        if ((kth & 63) == 0 && kth > 0) pid_vec = load_pids(cx, kth >> 6);
        issue(cx, pid_vec, c, kth, st, kb);
      }
    };

    auto compute = [&](int c, int st, const u32x4_t (&kb)[NK]) {
      const int cs = t0 + c * kChunk;
      f32x4_t s;
      if constexpr (ROPE) {  // the lane's key (token cs + tk) turned to its position
        u32x4_t kr[NK];
#pragma unroll
        for (int p = 0; p < NK; ++p) kr[p] = kb[p];
#pragma unroll
        for (int p = 0; p < NK / 2; ++p)
          rope_pieces<BF16>(kr[p], kr[p + NK / 2], (const FI_LDS uint32_t*)rope_tab + 8 * (4 * p + kq), cs + tk);
        s = qk_mfma<BF16, NK, true>(kr, qp);
      } else {
        s = qk_mfma<BF16, NK>(kb, qp);
      }
      float x[4];
      if (a.cap > 0.f) {
        const float c_in = a.scale * a.inv_cap, c_out = a.cap * kLog2e;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = c_out * tanh_from_exp(s[r] * c_in);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = s[r] * a.scale_log2;
      }
      if (cs + kChunk > t1) {  // tail chunk
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (cs + 4 * kq + r < t1) ? x[r] : neg_inf();
      }
      if (cs < cx.klo) {  // chunk starts before the window
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (cs + 4 * kq + r >= cx.klo) ? x[r] : neg_inf();
      }
      const float cm = head_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      const float m_new = cm > m_run + kMaxSlack ? cm : m_run;
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[r] - m_use);
      l_part = l_part * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      if (__any(hS < G && alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < NB; ++b) oacc[b] *= alpha;
      }
      // P^T as bf16 hi + lo parts (lo = the rounding remainder of hi)
      const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
      const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
      const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
      const s16x4_t bhi = __builtin_bit_cast(s16x4_t, u32x2_t{h01, h23});
      const s16x4_t blo = __builtin_bit_cast(s16x4_t, u32x2_t{l01, l23});
      const FI_LDS uint8_t* stage = (const FI_LDS uint8_t*)(&vring[wave][st][0]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int dim = 16 * b + 4 * tr_sub;
        int off;
        if constexpr (SMALLP) {  // piece pc of token t at (pc / 4) 1024 + (16 (pc % 4) + t) 16
          const int pc = dim >> 3;
          off = (pc >> 2) * 1024 + (16 * (pc & 3) + tr_tok) * 16;
        } else {
          off = tr_tok * RB + ((dim >> 3) ^ (tr_tok & (NP - 1))) * 16;
        }
        FI_LDS s16x4_t* src = (FI_LDS s16x4_t*)(stage + off + (dim & 7) * 2);
        const s16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(src);
        oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, bhi, oacc[b], 0, 0, 0);
        oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, blo, oacc[b], 0, 0, 0);
      }
    };

    const bool has_next = it + 1 < it_end;
    Ctx nx{0, 0, 0, 0, 0};
    int pid_next = 0, pid_next1 = 0;
    {
      if (myn > 0 && !pre_issued) issue_k(wave, 0, 0, kA);
      for (int k = 0; k < myn; k += 2) {
        const bool n1 = k + 1 < myn;
        if (n1) issue_k(wave + kWaves * (k + 1), k + 1, 1, kB);
        if (n1) FI_WAIT_VMCNT(kChunkOps); else FI_WAIT_VMCNT(0);
        __builtin_amdgcn_sched_barrier(0);
        compute(wave + kWaves * k, 0, kA);
        __builtin_amdgcn_sched_barrier(0);
        if (k == 0 && has_next) {  // the next item's record has landed by now
          nx = make_ctx(nxt);
          if constexpr (SMALLP) {
            pid_next = nx.nch > 0 ? load_id(nx, 0) : 0;
            pid_next1 = nx.nch > 0 ? load_id(nx, 1) : 0;
          } else {
            pid_next = load_pids(nx, 0);
          }
        }
        if (!n1) break;
        const bool n2 = k + 2 < myn;
        if (n2) issue_k(wave + kWaves * (k + 2), k + 2, 0, kA);
        if (n2) FI_WAIT_VMCNT(kChunkOps); else FI_WAIT_VMCNT(0);
        __builtin_amdgcn_sched_barrier(0);
        compute(wave + kWaves * (k + 1), 1, kB);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (myn == 0 && has_next) {
        nx = make_ctx(nxt);
        if constexpr (SMALLP) {
          pid_next = nx.nch > 0 ? load_id(nx, 0) : 0;
          pid_next1 = nx.nch > 0 ? load_id(nx, 1) : 0;
        } else {
          pid_next = load_pids(nx, 0);
        }
      }
      // chunk 0 of the next item, into kA / stage 0 (this wave's last chunk
      // has been computed, so both are free)
      pre_issued = has_next && nx.nch > wave;
      if (pre_issued) {
        pid_pre = pid_next;
        pid_pre1 = pid_next1;
        issue(nx, pid_pre, wave, 0, 0, kA);
      }
    }

    // wave totals (sum over the 4 lanes of a head: l, l ^ 16, l ^ 32, l ^ 48),
    // then merge the waves through LDS -- or, with one wave, write straight
    // from the accumulator: lane l holds dims 16 b + 4 kq .. + 3 of head
    // l % 16, and its head's max and sum
    l_part = head_sum(l_part);
    if constexpr (kWaves == 1) {
      if (hS < G) {
        const bool empty = m_run == neg_inf();
        const float inv = empty ? 0.f : 1.f / l_part;
        const float lse2 = empty ? neg_inf() : m_run + fast_log2(l_part);
        if (slot < 0) {
          const int64_t orow = (int64_t)qrow * a.Hq + g * G + hS;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t x = oacc[b] * inv;
            const int64_t at = orow * D + 16 * b + 4 * kq;
            if constexpr (OT::kBytes == 2)
              *reinterpret_cast<u32x2_t*>(a.o + at * 2) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            else
              *reinterpret_cast<f32x4_t*>(a.o + at * 4) = x;
          }
          if (a.lse && kq == 0) a.lse[orow] = lse2 * kLn2;
        } else {
          const int64_t prow = ((int64_t)slot * Hk + g) * G + hS;
#pragma unroll
          for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4_t*>(ws_o + prow * D + 16 * b + 4 * kq) = oacc[b] * inv;
          if (kq == 0) ws_lse[prow] = lse2 * kLn2;
        }
      }
      continue;
    }
    if (lane < G) {
      m_lds[wave][lane] = m_run;
      l_lds[wave][lane] = l_part;
    }
    if (hS < G) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<f32x4_t*>(&acc_lds[(wave * G + hS) * D + 16 * b + 4 * kq]) = oacc[b];
    }
    __syncthreads();
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
          O += acc_lds[(wv * G + h) * D + d] * sc;
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
  report_status(a.status, bad_page, kStatusBadPage);
}

template <int D, int G, typename OT, bool ROPE, bool SMALLP>
int launch_mfma(const RunArgs& r, const DecodeParams& p) {
  dim3 grid(r.workers, r.Hk), block(kThreads);
  hipLaunchKernelGGL((decode_mfma_kernel<D, G, OT, ROPE, SMALLP>), grid, block, 0, (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return FI_OK;
}

template <typename T, int D, int G, bool FAST, typename OT, bool ROPE>
int launch_t(const RunArgs& r, const DecodeParams& p) {
  dim3 grid(r.workers, r.Hk), block(kThreads);
  hipLaunchKernelGGL((decode_kernel<T, D, G, FAST, OT, ROPE>), grid, block, 0,
                     (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return FI_OK;
}

template <typename T, int D, int G, typename OT, bool ROPE>
int launch_fast(const RunArgs& r, const DecodeParams& p) {
  if constexpr (T::kBytes == 2) {
    if (p.page_shift >= 0) return launch_mfma<D, G, OT, ROPE, false>(r, p);
    if (p.small_shift >= 0) return launch_mfma<D, G, OT, ROPE, true>(r, p);
  }
  return p.page_shift >= 0 ? launch_t<T, D, G, true, OT, ROPE>(r, p) : launch_t<T, D, G, false, OT, ROPE>(r, p);
}

template <typename T, int D, int G, typename OT>
int launch_rope(const RunArgs& r, const DecodeParams& p) {
  return r.rope ? launch_fast<T, D, G, OT, true>(r, p) : launch_fast<T, D, G, OT, false>(r, p);
}

template <typename T, int D, typename OT>
int launch_g(const RunArgs& r, const DecodeParams& p) {
  switch (r.G) {
    case 1: return launch_rope<T, D, 1, OT>(r, p);
    case 2: return launch_rope<T, D, 2, OT>(r, p);
    case 4: return launch_rope<T, D, 4, OT>(r, p);
    case 8: return launch_rope<T, D, 8, OT>(r, p);
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
  p.status = r.status;
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
  p.small_shift = -1;
  if (r.P < 16 && (r.P & (r.P - 1)) == 0) {
    int s = 0;
    while ((1 << s) < r.P) ++s;
    p.small_shift = s;
  }
  p.stream_at = r.stream_at;
  p.scale = r.sm_scale;
  p.scale_log2 = r.sm_scale * kLog2e;
  p.cap = r.soft_cap;
  p.inv_cap = r.soft_cap > 0.f ? 1.f / r.soft_cap : 0.f;
  p.window = r.window;
  for (int i = 0; i < kRopeMaxPairs; ++i) p.rope_f[i] = r.rope_f[i];
  if (r.dtype == FI_BF16 && r.out_dtype == FI_BF16) return launch_d<BF16, BF16>(r, p);
  if (r.dtype == FI_BF16 && r.out_dtype == FI_F32) return launch_d<BF16, F32>(r, p);
  if (r.dtype == FI_F32 && r.out_dtype == FI_F32) return launch_d<F32, F32>(r, p);
  return set_error(FI_ERR_UNSUPPORTED, "decode: dtype combination");
}

}  // namespace fi
