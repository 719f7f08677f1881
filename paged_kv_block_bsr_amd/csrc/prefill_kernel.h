// prefill_kernel.h -- persistent ragged batch-prefill kernel over a paged KV cache
// (gfx950, bf16, MFMA), included by prefill.hip (kernels without a sliding
// window or rotary embedding), prefill_window.hip (with a window) and
// prefill_rope.hip (with the rotary embedding, window or not): translation
// units that build in parallel.
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
// Mapping.  grid = workers x KV heads (1-D, XCD-major), 256 threads = 4
// waves.  A work item is a tile of up to 128 packed rows (packed row r =
// token r / G, head r % G of the KV head's group) times a range of KV pages.
// Wave w owns packed rows 32 w .. 32 w + 31; lane l holds row l % 32, and
// lanes l and l + 32 split each 32-key block between them.  Per 64-key tile:
//   - K goes global -> LDS directly (row-major, 16-byte pieces XOR-swizzled
//     within the row); V goes global -> registers -> LDS as fp16 V^T with
//     the keys of every 16-key group permuted to the order in which the
//     S^T accumulator holds them.  Both are double buffered; K runs two
//     tiles ahead, V one.
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = the
//     wave's packed query rows, kept in registers): each lane owns the 32
//     logits of its row that lie in its half, so max and sum are lane-local
//     plus one swap with the lane 32 apart.  The product for tile n + 1 is
//     issued in the same instruction stream as the softmax of tile n, so
//     the matrix cores and the vector unit work side by side.
//   - online softmax in registers (base-2 exponentials, scale folded in,
//     lazily moved running max); P is packed to fp16 and the row sum is
//     taken over the packed values with v_dot2, so numerator and
//     denominator see the same rounded weights.
//   - O^T += V^T P^T with v_mfma_f32_32x32x16_f16; P^T comes straight from
//     the S^T registers.  P and V run in fp16: bf16 V converts exactly in
//     fp16's normal range (the conversion saturates at +-65504), and fp16
//     keeps 11 bits of P where bf16 keeps 8.
//   - with a tree mask (MASK, speculative decoding: paper page, opening
//     paragraph; the token trees of the talk page, Background and "Block
//     Sparse Matrix"), the
//     request's draft tokens are its last qo_len keys; tiles that reach the
//     draft take the masked step, where each lane tests the bits of its row
//     (two 32-bit words per 32-key block, loaded before the step's K/V
//     loads) for the draft keys of the block.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "fi_internal.h"

namespace fi {

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
  int32_t* status;     // status word: kStatusBadPage when a page id is not below pool_pages
  int64_t pool_pages;
  int32_t Hq, Hk, P;
  int32_t causal;
  int32_t stream_at;
  int32_t workers;
  int32_t page_shift;  // log2(P) when P is a power of two >= 16, else -1
  // key / P for any P as (umulhi(key, p_magic) + (key & p_mask)) >> p_sh
  // (exact for keys below 2^31): a power of two has magic 0, mask all ones;
  // any other P has sh = floor(log2 P), magic = ceil(2^(32 + sh) / P) < 2^32
  uint32_t p_magic;
  uint32_t p_mask;
  int32_t p_sh;
  float scale_log2;
  float scale;
  float cap;
  float inv_cap;
  int32_t window;      // sliding window: keys seen before the query's own (kernels built with WIN)
  // tree mask (kernels built with MASK): bit n of the bit stream is bit n % 32
  // of mask[n / 32]; request i's qo x qo block starts at bit mask_indptr[i]
  const uint32_t* mask;
  const int32_t* mask_indptr;
  int32_t mask_last_word;
  uint32_t rope_f[kRopeMaxPairs];  // rotary turn per position of pair d (kernels built with ROPE)
};

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kTileK = 64;            // keys per KV tile
constexpr int kVStride = kTileK + 8;  // V^T row stride (elements): 144 B, conflict-free 16-byte reads
constexpr float kMaxSlack = 8.f;      // log2-domain headroom of the lazily updated running max

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
#define FI_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Two fp32 values as an fp16 pair, rounding toward zero (exact for bf16
// inputs in fp16's normal range; saturates instead of overflowing).
__device__ __forceinline__ uint32_t pack_f16_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// max of three floats as one v_maximum3_f32 (NaN-propagating maximum, which
// needs no quietening of its inputs as fmaxf does; the logits it is applied
// to are finite or -inf, never NaN).  It stays a compiler builtin, not inline
// asm: its inputs come straight from matrix-core results, and only for code
// it can see does the compiler insert the wait states that must separate an
// MFMA from a VALU read of its result.  (An asm form read the accumulators
// too early, a timing-dependent stale max.)
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// v_permlane32_swap on (x, x) leaves x of lane l % 32 in one result and x of
// lane l % 32 + 32 in the other, in every lane: combining the two gives the
// pair's max / sum in both halves.
__device__ __forceinline__ float half_max(float x) {
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}


// Position of key k (0..63) of a tile inside a V^T row: bits 2 and 3
// swapped.  The S^T accumulator of lane half h holds keys 8 i + 4 h + j
// (i = 0..3, j = 0..3) of a 32-key block; with the swap, the 8 keys half h
// feeds to one 16-key k-step of the PV product are contiguous.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }


template <int D>
struct PShape {
  static constexpr int KRow = D * 2;                           // bytes of one K row (no padding)
  static constexpr int KPiecesRow = D / 8;                     // 16-byte pieces of one K row
  static constexpr int KDma = kTileK * D * 2 / 1024 / kWaves;  // direct-to-LDS K loads per wave
  static constexpr int KeysPerWave = kTileK / kWaves;          // keys of the tile one wave's K loads cover
  static constexpr int KSteps = D / 16;                        // MFMA k-steps of K Q^T
  static constexpr int DBlocks = D / 32;                       // 32-dim blocks of O^T
  static constexpr int VPiecesRow = D / 8;                     // 16-byte pieces of one V row
  static constexpr int VThreads = 16 * VPiecesRow;             // threads staging V: 4 keys x 1 piece each
};

template <int D, int G, bool FAST, bool CAP, bool WIN, bool ROPE, bool MASK, typename OT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams a) {
  using SH = PShape<D>;
  static_assert(SH::KDma >= 1 && SH::VThreads <= kThreads, "tile shape");
  // two buffers each, as separate arrays: the buffer a step uses is a
  // compile-time choice, so the compiler can tell the direct-to-LDS writes of
  // one buffer from the reads of the other and need not wait for them
  __shared__ __align__(16) uint8_t k_lds0[kTileK * SH::KRow];
  __shared__ __align__(16) uint8_t k_lds1[kTileK * SH::KRow];
  __shared__ __align__(16) uint16_t v_lds0[D * kVStride];
  __shared__ __align__(16) uint16_t v_lds1[D * kVStride];
  __shared__ uint32_t rope_tab[ROPE ? D / 2 : 1];  // rotary table, read with the lanes' own dims
  if constexpr (ROPE) {
    for (int i = threadIdx.x; i < D / 2; i += kThreads) rope_tab[i] = a.rope_f[i];
    __syncthreads();
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
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
  const int32_t* items = a.plan + sd[S_OFF_ITEMS];
  const int32_t* meta = a.plan + sd[S_OFF_META];
  const int32_t* wip = a.plan + sd[S_OFF_WIP];
  float* ws_o = a.ws + sd[S_WS_O];
  float* ws_lse = a.ws + sd[S_WS_LSE];
  const int P = a.P;
  const int Hk = a.Hk;
  const int tok_bytes = Hk * D * 2;
  const int64_t half_bytes = (int64_t)P * tok_bytes;
  const int64_t page_bytes = 2 * half_bytes;
  const uint32_t page_bytes_u = (uint32_t)page_bytes;  // < 2^32: checked on the host
  const uint8_t* kv_head = a.kv + (int64_t)g * D * 2;
  // staging roles.  K: load j of wave w fills tile bytes (w KDma + j) 1024 +
  // 16 lane, i.e. key k_key(j) (the wave's keys are 16 consecutive ones),
  // LDS piece lane % pieces-per-row.  V: thread t < VThreads stages keys
  // 4 (t % 16) .. + 3 at piece t / 16.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto k_key = [&](int j) { return ((wave * SH::KDma + j) * 1024 + 16 * lane) / SH::KRow; };
  const int k_pp = lane % SH::KPiecesRow;
  // per-lane part of the K source offset of load j when the wave's 16 keys
  // sit in one page (tile-independent: key % pieces-per-row depends on the
  // key's place among the 16 only)
  uint32_t k_off[SH::KDma];
#pragma unroll
  for (int j = 0; j < SH::KDma; ++j) {
    const int kk = (j * 1024 + 16 * lane) / SH::KRow;
    k_off[j] = kk * tok_bytes + (k_pp ^ (kk & (SH::KPiecesRow - 1))) * 16;
  }
  const int v_kg = tid & 15;
  const int v_piece = tid >> 4;
  const bool v_active = SH::VThreads == kThreads || tid < SH::VThreads;
  const uint32_t pool_lim = a.pool_pages < 0x80000000ll ? (uint32_t)a.pool_pages : 0x80000000u;

  const int it_begin = wip[worker];
  const int it_end = wip[worker + 1];

  // ---- items.  An item's record and the page ids of its first tile are
  // loaded early in the item before it, its query rows and first K/V tile
  // before that item's epilogue: consecutive items of a worker overlap
  // instead of paying three dependent memory round trips each.
  struct Item {
    int pb, pe, slot, rb, re, kvb, kv_len, qbase, qo_len, req;
  };
  auto load_item = [&](int it) -> Item {
    Item x{0, 0, -1, 0, 0, 0, 0, 0, 0, 0};  // past the worker's last item: no keys
    if (it < it_end) {
      const int32_t* im = meta + kMetaInts * it;
      x = Item{items[4 * it + 1], items[4 * it + 2], items[4 * it + 3], im[M_RB], im[M_RE],
               im[M_KVB],         im[M_KVLEN],       im[M_QOBASE],      im[M_QOLEN], MASK ? im[M_REQ] : 0};
    }
    return x;
  };
  // the fields are wave-uniform: scalar registers hold them across an item
  // (converted once the loads are known to have landed, so that the
  // conversion does not wait for them)
  auto uniform = [](const Item& x) {
    auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    return Item{u(x.pb), u(x.pe), u(x.slot), u(x.rb), u(x.re), u(x.kvb), u(x.kv_len), u(x.qbase), u(x.qo_len), u(x.req)};
  };
  // an item's keys [t0, t1) in ntiles tiles, and its request's page ids
  struct Ctx {
    int t0, t1, ntiles;
    const int32_t* kvi;
  };
  auto make_ctx = [&](const Item& x) -> Ctx {
    const int t0 = x.pb * P, t1 = min(x.pe * P, x.kv_len);
    return Ctx{t0, t1, t1 > t0 ? (t1 - t0 + kTileK - 1) / kTileK : 0, a.kv_indices + x.kvb};
  };
  // this lane's packed row of an item, and that row's token and head
  auto row_of = [&](const Item& x) { return x.rb + kRowsPerWave * wave + l32; };
  auto tok_head = [&](const Item& x, int& tok, int& head) {
    const int r = row_of(x);
    const int rc = r < x.re ? r : x.re - 1;
    tok = rc / G;
    head = g * G + rc % G;
  };

  // ---- staging
  auto page_idx = [&](int key) -> int {
    if constexpr (FAST) return key >> a.page_shift;
    const uint32_t k = (uint32_t)key;
    return (int)((__umulhi(k, a.p_magic) + (k & a.p_mask)) >> a.p_sh);
  };
  auto slot_of = [&](int key) { return FAST ? key & (P - 1) : key - page_idx(key) * P; };
  auto clamp_key = [&](const Ctx& c, int key) { return key < c.t1 ? key : c.t1 - 1; };
  // page ids are loaded raw and checked where they are used, a tile
  // later, so the load is never waited for early; an id outside the pool
  // reads page 0 instead, and is reported in the status word at the end
  uint32_t bad_page = 0;
  auto checked = [&](int pg) -> uint32_t {
    const bool ok = (uint32_t)pg < pool_lim;
    bad_page |= !ok;
    return ok ? (uint32_t)pg : 0u;
  };
  auto raw_page = [&](const Ctx& c, int key) -> int { return c.kvi[(uint32_t)page_idx(key)]; };
  // With power-of-two pages of >= 16 tokens (FAST) a wave's 16 K keys sit
  // in one page (tiles start on 16-key boundaries), whose id is then
  // wave-uniform, and so do a thread's 4 V keys.  With other pages (down to
  // one token each: the column-vector BSR) lane l of every wave loads the id
  // of tile key l -- one coalesced load per tile -- and each K or V key
  // gets its pool row from that lane (key_rows below).  K keys past t1 need
  // no clamping beyond the page (their logits are masked; the page is valid)
  // with FAST pages; otherwise, and for V, keys are clamped to t1 - 1 so
  // that masked keys still read finite values (P = 0 times a NaN would not
  // vanish).
  struct KPages {
    int id[1];
  };
  struct VPages {  // FAST: the thread's V page; otherwise unused (the ids are in KPages)
    int id[1];
  };
  auto fetch_k = [&](const Ctx& c, int n) -> KPages {
    KPages pg;
    const int ts = c.t0 + n * kTileK;
    if constexpr (FAST) {
      const int pi = min(page_idx(ts + wave_u * SH::KeysPerWave), page_idx(c.t1 - 1));
      pg.id[0] = n < c.ntiles ? c.kvi[(uint32_t)pi] : 0;  // same in every lane of the wave
    } else {
      pg.id[0] = n < c.ntiles ? raw_page(c, clamp_key(c, ts + lane)) : 0;  // tile key `lane`
    }
    return pg;
  };
  auto fetch_v = [&](const Ctx& c, int n) -> VPages {
    VPages pg;
    const int ts = c.t0 + n * kTileK;
    const bool ok = n < c.ntiles && v_active;
    pg.id[0] = FAST && ok ? raw_page(c, clamp_key(c, ts + 4 * v_kg)) : 0;
    return pg;
  };
  // Other pages: lane l turns the id of tile key l into that key's K row in
  // the pool, counted in token rows (page p's K rows start at row 2 p P, its
  // V rows P later; below 2^32 rows: checked on the host), so a K or V key
  // needs only that lane's row (ds_bpermute) and one multiply-add.
  auto key_rows = [&](const Ctx& c, int n, const KPages& pg) -> uint32_t {
    const int kl = clamp_key(c, c.t0 + n * kTileK + lane);
    return 2u * checked(pg.id[0]) * (uint32_t)P + (uint32_t)slot_of(kl);
  };
  auto row_addr = [&](uint32_t row) { return kv_head + (uint64_t)row * (uint32_t)tok_bytes; };
  auto dma_k = [&](const Ctx& c, int n, uint8_t* kb, const KPages& pg) {
    if constexpr (FAST) {
      const int ts = c.t0 + n * kTileK;
      const int pid = __builtin_amdgcn_readfirstlane(pg.id[0]);
      const uint8_t* base = kv_head + (int64_t)checked(pid) * page_bytes +
                            slot_of(ts + wave_u * SH::KeysPerWave) * tok_bytes;
#pragma unroll
      for (int j = 0; j < SH::KDma; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + k_off[j]),
                                         (FI_LDS void*)(kb + (wave_u * SH::KDma + j) * 1024), 16, 0, 0);
    } else {
      const uint32_t rows = key_rows(c, n, pg);
#pragma unroll
      for (int j = 0; j < SH::KDma; ++j) {
        const int key = k_key(j);
        const uint8_t* src = row_addr(__shfl(rows, key)) + (k_pp ^ (key & (SH::KPiecesRow - 1))) * 16;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (FI_LDS void*)(kb + (wave_u * SH::KDma + j) * 1024), 16, 0, 0);
      }
    }
  };
  u32x4_t vreg[4] = {};
  auto load_v = [&](const Ctx& c, int n, const KPages& pk, const VPages& pg) {
    if constexpr (!FAST) {  // each key's V row from its lane (every lane takes part)
      const uint32_t rows = key_rows(c, n, pk) + (uint32_t)P;
      uint32_t vrow[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vrow[j] = __shfl(rows, 4 * v_kg + j);
      if (v_active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[j] = load16(row_addr(vrow[j]) + v_piece * 16);
      }
      return;
    }
    if (v_active) {
      const int ts = c.t0 + n * kTileK;
      const uint8_t* base = kv_head + half_bytes + v_piece * 16;
      if (ts + kTileK <= c.t1) {  // whole tile valid: the 4 keys are consecutive slots of one page
        const uint8_t* b0 = base + (uint64_t)checked(pg.id[0]) * page_bytes_u +
                            __umul24((uint32_t)slot_of(ts + 4 * v_kg), (uint32_t)tok_bytes);
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[j] = load16(b0 + (uint32_t)(j * tok_bytes));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kc = clamp_key(c, ts + 4 * v_kg + j);
          const uint8_t* pbase = base + (uint64_t)checked(pg.id[0]) * page_bytes_u;
          vreg[j] = load16(pbase + __umul24((uint32_t)slot_of(kc), (uint32_t)tok_bytes));
        }
      }
    }
  };
  auto store_v = [&](uint16_t* vb) {
    if (v_active) {
      uint16_t* dst = vb + (8 * v_piece) * kVStride + vt_pos(4 * v_kg);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2_t lo, hi;  // dims 2w and 2w + 1 of the piece, keys 4 kg .. + 3
        lo[0] = pack_f16_rtz(bf16_lo(vreg[0][w]), bf16_lo(vreg[1][w]));
        lo[1] = pack_f16_rtz(bf16_lo(vreg[2][w]), bf16_lo(vreg[3][w]));
        hi[0] = pack_f16_rtz(bf16_hi(vreg[0][w]), bf16_hi(vreg[1][w]));
        hi[1] = pack_f16_rtz(bf16_hi(vreg[2][w]), bf16_hi(vreg[3][w]));
        *reinterpret_cast<u32x2_t*>(dst + (2 * w) * kVStride) = lo;
        *reinterpret_cast<u32x2_t*>(dst + (2 * w + 1) * kVStride) = hi;
      }
    }
  };

  // packed query rows as the MFMA B operand (dims 16 ks + 8 hh .. + 8)
  bf16x8_t qp[SH::KSteps];
  auto load_q = [&](const Item& x) {
    int tok, head;
    tok_head(x, tok, head);
    const uint8_t* qb = a.q + ((int64_t)(x.qbase + tok) * a.Hq + head) * D * 2;
#pragma unroll
    for (int ks = 0; ks < SH::KSteps; ++ks)
      qp[ks] = __builtin_bit_cast(bf16x8_t, load16(qb + (16 * ks + 8 * hh) * 2));
  };

  // ---- rotary embedding.  Queries are turned in registers once per item
  // (lane dims 16 ks + 8 hh .. + 8; the partner of ks is ks + KSteps / 2).
  // Keys are turned once per workgroup, in LDS, after a tile has landed and
  // before it is read: thread t takes key t / 4 and D / 64 piece pairs
  // (c, c + D / 16) of its row, in place.  Both come out as fp16, and the
  // QK^T product of these kernels runs on the fp16 matrix-core instruction.
  auto rope_q = [&](int pos) {
#pragma unroll
    for (int ks = 0; ks < SH::KSteps / 2; ++ks) {
      u32x4_t lo = __builtin_bit_cast(u32x4_t, qp[ks]), hi = __builtin_bit_cast(u32x4_t, qp[ks + SH::KSteps / 2]);
      rope_pieces<BF16>(lo, hi, (const FI_LDS uint32_t*)rope_tab + 16 * ks + 8 * hh, pos);
      qp[ks] = __builtin_bit_cast(bf16x8_t, lo);
      qp[ks + SH::KSteps / 2] = __builtin_bit_cast(bf16x8_t, hi);
    }
  };
  auto rope_k = [&](uint8_t* kb, int ts) {
    constexpr int PPT = D / 64, HALF = D / 16;
    const int key = tid >> 2;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int c = (tid & 3) * PPT + j;
      uint8_t* row = kb + key * SH::KRow;
      u32x4_t* plo = reinterpret_cast<u32x4_t*>(row + ((c ^ (key & (SH::KPiecesRow - 1))) * 16));
      u32x4_t* phi = reinterpret_cast<u32x4_t*>(row + (((c + HALF) ^ (key & (SH::KPiecesRow - 1))) * 16));
      u32x4_t lo = *plo, hi = *phi;
      rope_pieces<BF16>(lo, hi, (const FI_LDS uint32_t*)rope_tab + 8 * c, ts + key);
      *plo = lo;
      *phi = hi;
    }
  };

  // the worker's first item: query rows, tile 0 and the page ids of tile 1
  Item item = uniform(load_item(it_begin));
  KPages pk{};
  VPages pv_ids{};
  if (it_begin < it_end) {
    const Ctx c = make_ctx(item);
    load_q(item);
    pk = fetch_k(c, 0);
    pv_ids = fetch_v(c, 0);
    if (c.ntiles > 0) {
      dma_k(c, 0, k_lds0, pk);
      load_v(c, 0, pk, pv_ids);
    }
    pk = fetch_k(c, 1);
    pv_ids = fetch_v(c, 1);
  }

  for (int it = it_begin; it < it_end; ++it) {
    const Item nxt_raw = load_item(it + 1);
    const Ctx cx = make_ctx(item);
    const int t0 = cx.t0, ntiles = cx.ntiles;
    const int slot = item.slot, rb = item.rb, re = item.re, qbase = item.qbase;

    // this lane's packed row, its token, head and key limit
    const int r = row_of(item);
    const bool row_valid = r < re;
    int tok, head;
    tok_head(item, tok, head);
    const int causal_off = item.kv_len - item.qo_len;
    const int lim = min(a.causal ? causal_off + tok + 1 : item.kv_len, cx.t1);
    const int r_first = min(rb + kRowsPerWave * wave, re - 1);
    const int wave_lim_min = min(a.causal ? causal_off + r_first / G + 1 : item.kv_len, cx.t1);
    // Sliding window: the first key the lane's query sees, and the largest
    // such key over the wave's rows (tiles that start before it are masked).
    // lo is not clamped at 0 (keys are never negative) but at the item's end
    // t1, so that the lane's visible span below is never negative; a window
    // of kv_len keys or more hides nothing, so w is clamped at kv_len (with
    // kv_len + qo_len < 2^30, checked by the planner, every bound here stays
    // well inside int32).  The lane holds lo instead of lim: a causal row's
    // key limit is lo + w + 1 (unless lo was clamped, and then it sees no key
    // of the item), a non-causal one's is the item's end.
    // Tree mask: the first bit of this lane's row (draft token tok of a
    // request whose draft starts at key causal_off); read in masked steps,
    // where the compiler waits for it.
    int mrow = 0;
    if constexpr (MASK) mrow = a.mask_indptr[item.req] + tok * item.qo_len;
    int lo = 0, wave_lo_max = 0, w = 0;
    if constexpr (WIN) {
      w = min(a.window, item.kv_len);
      lo = min(causal_off + tok - w, cx.t1);
      wave_lo_max = causal_off + min(rb + kRowsPerWave * wave_u + kRowsPerWave - 1, re - 1) / G - w;
    }

    f32x16_t oacc[SH::DBlocks];
#pragma unroll
    for (int d = 0; d < SH::DBlocks; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
    float m_run = neg_inf();
    float l_part = 0.f;

    // ---- compute pieces, per 32-key block b of a tile
    // K operands of block b: key 32 b + l32, dims 16 ks + 8 hh .. + 8
    auto kread = [&](const uint8_t* kb, int b, u32x4_t (&kop)[SH::KSteps]) {
      const int key = 32 * b + l32;
      const uint8_t* krow = kb + key * SH::KRow;
#pragma unroll
      for (int ks = 0; ks < SH::KSteps; ++ks) {
        const int pp = (2 * ks + hh) ^ (key & (SH::KPiecesRow - 1));
        kop[ks] = *reinterpret_cast<const u32x4_t*>(krow + pp * 16);
      }
    };
    // S^T block: keys 32 b + 8 i + 4 hh + j of the tile in s[4 i + j]
    auto qk = [&](const u32x4_t (&kop)[SH::KSteps], f32x16_t& s) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < SH::KSteps; ++ks) {
        if constexpr (ROPE)  // rotated q and k are fp16
          s = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, kop[ks]),
                                                     __builtin_bit_cast(f16x8_t, qp[ks]), s, 0, 0, 0);
        else
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kop[ks]), qp[ks], s, 0, 0, 0);
      }
    };
    // V^T operands of block b: dims 32 d + l32, k-steps k of 16 keys
    auto vread = [&](const uint16_t* vb, int b, u32x4_t (&vop)[2][SH::DBlocks]) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d)
          vop[k][d] = *reinterpret_cast<const u32x4_t*>(vb + (32 * d + l32) * kVStride + 32 * b + 16 * k + 8 * hh);
    };
    auto pv = [&](const u32x4_t (&vop)[2][SH::DBlocks], const f16x8_t (&pb)[2]) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d)
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, vop[k][d]), pb[k], oacc[d], 0, 0, 0);
    };
    const float sc = CAP ? 1.f : a.scale_log2;
    // logits -> log2 domain (cap) and the mask, at mask level M: 0 none; 1 the
    // key limit (tiles that reach past the wave's smallest limit); 2 the
    // limit and the window start (tiles that start before the wave's largest
    // window start)
    auto prepare = [&](int n, int b, f32x16_t& s, auto mask_tag, uint64_t mwin) {
      constexpr int M = decltype(mask_tag)::value;
      const int bs = t0 + n * kTileK + 32 * b;
      if constexpr (CAP) {
        const float c_in = a.scale * a.inv_cap, c_out = a.cap * kLog2e;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = c_out * tanh_from_exp(s[e] * c_in);
      }
      if constexpr (M >= 1) {
        // key 8 i + j of this half is visible iff it is < rel (and >= rlo:
        // as one unsigned compare, kk - rlo < rel - rlo, where rel >= rlo)
        int rel, rlo = 0;
        if constexpr (WIN) {
          // from the lane's first visible key (the empty asm keeps the
          // compiler from computing rel ahead of the loop, where it would
          // hold a second register per lane through it)
          rlo = lo - bs - 4 * hh;
          asm volatile("" : "+v"(rlo));
          rel = a.causal ? min(rlo + w + 1, cx.t1 - bs - 4 * hh) : cx.t1 - bs - 4 * hh;
        } else {
          rel = lim - bs - 4 * hh;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = 8 * (e >> 2) + (e & 3);
          if constexpr (M == 1) s[e] = kk < rel ? s[e] : neg_inf();
          else s[e] = (uint32_t)(kk - rlo) < (uint32_t)(rel - rlo) ? s[e] : neg_inf();
        }
        if constexpr (MASK) {
          // draft key u = key - causal_off (u < 0: a key before the draft,
          // visible; u == tok: the row's own key, visible): bit mrow + u,
          // at bit mrow + u - 32 w0 of the block's 64-bit window
          const int ub = bs + 4 * hh - causal_off;  // u of the lane's first key in the block
          const int w0 = (mrow + max(ub, 0)) >> 5;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int u = ub + 8 * (e >> 2) + (e & 3);
            const bool vis = u < 0 || u == tok || ((mwin >> ((mrow + u - 32 * w0) & 63)) & 1ull);
            s[e] = vis ? s[e] : neg_inf();
          }
        }
      }
    };
    // the two words of a block's mask window (see prepare); word indices are
    // clamped into [0, the stream's last word], so a malformed mask_indptr
    // reads wrong bits but never outside the mask
    auto mask_window = [&](int n, int b) -> uint64_t {
      const int ub = t0 + n * kTileK + 32 * b + 4 * hh - causal_off;
      const int w0 = (mrow + max(ub, 0)) >> 5;
      const uint32_t lo_w = a.mask[min(max(w0, 0), a.mask_last_word)];
      const uint32_t hi_w = a.mask[min(max(w0 + 1, 0), a.mask_last_word)];
      return (uint64_t)lo_w | ((uint64_t)hi_w << 32);
    };
    // Online softmax of a prepared block, in two parts.  update_max: the
    // block's row max; the running max moves only when a block beats it by
    // more than 2^8, and then (rarely, wave-uniform branch) the accumulator
    // and the row sum are rescaled.  exps: P^T (fp16) for the block's 2 PV
    // k-steps, its row sum (over the packed values) added into l_part.
    float m_use = 0.f;  // m_run, or 0 while it is -inf
    auto update_max = [&](f32x16_t& s) {
      float tm = max3(s[0], s[1], s[2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) tm = max3(tm, s[e], s[e + 1]);
      tm = fmaxf(tm, s[15]);
      const float tmax = half_max(tm) * sc;
      const bool move = tmax > m_run + kMaxSlack;
      if (__builtin_expect(__any(move), 0)) {
        const float m_new = move ? tmax : m_run;
        const float m_new_use = m_new == neg_inf() ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_new_use);  // 1 where the max stays, 0 from -inf
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d) oacc[d] *= alpha;
        l_part *= alpha;
        m_run = m_new;
        m_use = m_new_use;
      }
    };
    auto exps = [&](const f32x16_t& s, f16x8_t (&pb)[2]) {
      const f16x2_t ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = fast_exp2(fmaf(s[8 * k + 2 * i], sc, -m_use));
          const float p1 = fast_exp2(fmaf(s[8 * k + 2 * i + 1], sc, -m_use));
          const f16x2_t pp = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
          pb[k][2 * i] = pp[0];
          pb[k][2 * i + 1] = pp[1];
          l_part = __builtin_amdgcn_fdot2(pp, ones, l_part, false);
        }
      }
    };

    // ---- pipeline.  Per tile n (buffers chosen at compile time):
    //   K(b0) reads | QK(b0) with the K(b1) reads and the issue of tile
    //   n + 1's loads | QK(b1) with softmax(b0) and the V(b0) reads |
    //   PV(b0) with softmax(b1) and the V(b1) reads | PV(b1) with the fp16
    //   conversion of V(n + 1) | one barrier.
    // The compiler does not track direct-to-LDS loads: every thread waits
    // for all of its loads before the barrier.
    // Tile 0 (K in k_lds0, V in registers), the query rows and the page ids
    // of tile 1 were issued before the previous item's epilogue (or above).
    if (ntiles > 0) store_v(v_lds0);
    FI_WAIT_VMCNT(0);
    __syncthreads();
    if constexpr (ROPE) {  // the query rows and key tile 0 have landed: turn them
      rope_q(causal_off + tok);
      if (ntiles > 0) {
        rope_k(k_lds0, t0);
        __syncthreads();
      }
    }
    // the next item's record has landed: the page ids of its first tile
    // (with other pages than FAST ones fetched after the loop instead:
    // holding them through it spills)
    const Item nxt = uniform(nxt_raw);
    const Ctx nc = make_ctx(nxt);
    KPages npk{};
    VPages npv{};
    if constexpr (FAST) {
      npk = fetch_k(nc, 0);
      npv = fetch_v(nc, 0);
    }

    // Loads for tile n + 1 are issued even past the last tile (page ids of
    // tiles past the end read as 0, a valid page): nothing reads that data,
    // and the body stays free of branches.
    auto step = [&](int n, auto cur, auto mask_tag) {
      constexpr bool B1 = decltype(cur)::value;
      uint8_t* kb = B1 ? k_lds1 : k_lds0;
      uint8_t* kb_next = B1 ? k_lds0 : k_lds1;
      uint16_t* vb = B1 ? v_lds1 : v_lds0;
      uint16_t* vb_next = B1 ? v_lds0 : v_lds1;
      u32x4_t kop0[SH::KSteps], kop1[SH::KSteps];
      u32x4_t vop0[2][SH::DBlocks], vop1[2][SH::DBlocks];
      f32x16_t s0, s1;
      f16x8_t p0[2], p1[2];
      uint64_t mw0 = 0, mw1 = 0;
      if constexpr (MASK && decltype(mask_tag)::value >= 1) {  // before the tile loads, so that their use waits for these alone
        mw0 = mask_window(n, 0);
        mw1 = mask_window(n, 1);
      }
      kread(kb, 0, kop0);
      kread(kb, 1, kop1);
      dma_k(cx, n + 1, kb_next, pk);
      load_v(cx, n + 1, pk, pv_ids);
      pk = fetch_k(cx, n + 2);
      pv_ids = fetch_v(cx, n + 2);
      // The products and the softmax run at a raised wave priority, the V
      // conversion and the wait for the next tile at the normal one: while
      // this workgroup's waves wait, the other workgroup's waves on the same
      // SIMDs win the issue slots (slice call 0.1382 ms against 0.1427).
      __builtin_amdgcn_s_setprio(3);
      qk(kop0, s0);
      prepare(n, 0, s0, mask_tag, mw0);
      // QK(b1) + softmax(b0) + V(b0) reads
      qk(kop1, s1);
      update_max(s0);
      vread(vb, 0, vop0);
      exps(s0, p0);
      prepare(n, 1, s1, mask_tag, mw1);
      // PV(b0) + softmax(b1) + V(b1) reads
      pv(vop0, p0);
      update_max(s1);
      vread(vb, 1, vop1);
      exps(s1, p1);
      // PV(b1) + the conversion of the next V tile
      pv(vop1, p1);
      __builtin_amdgcn_s_setprio(0);
      store_v(vb_next);
      FI_WAIT_VMCNT(0);
      __syncthreads();
      if constexpr (ROPE) {  // key tile n + 1 has landed in kb_next: turn it before it is read
        if (n + 1 < ntiles) {
          rope_k(kb_next, t0 + (n + 1) * kTileK);
          __syncthreads();
        }
      }
    };
    auto step_any = [&](int n, auto cur) {
      const int ts = t0 + n * kTileK;
      if (ts + kTileK > wave_lim_min || (WIN && ts < wave_lo_max) || (MASK && ts + kTileK > causal_off))
        step(n, cur, std::integral_constant<int, WIN ? 2 : 1>{});
      else step(n, cur, std::integral_constant<int, 0>{});
    };
    // A wave whose 32 rows all lie past the tile's end (tiles of fewer than
    // 128 rows) has nothing to compute: per tile it does only its share of
    // the staging -- its quarter of the K loads and its V pieces -- and the
    // barrier, so the busy waves of the tile and the other workgroup on the
    // CU get its issue slots.  (The rotary kernels turn K in LDS with every
    // thread and keep the full step.)
    auto stage_only = [&](int n, auto cur) {
      constexpr bool B1 = decltype(cur)::value;
      dma_k(cx, n + 1, B1 ? k_lds0 : k_lds1, pk);
      load_v(cx, n + 1, pk, pv_ids);
      pk = fetch_k(cx, n + 2);
      pv_ids = fetch_v(cx, n + 2);
      store_v(B1 ? v_lds0 : v_lds1);
      FI_WAIT_VMCNT(0);
      __syncthreads();
    };
    if (!ROPE && rb + kRowsPerWave * wave_u >= re) {
      for (int n = 0; n < ntiles; n += 2) {
        stage_only(n, std::false_type{});
        if (n + 1 < ntiles) stage_only(n + 1, std::true_type{});
      }
    } else {
      for (int n = 0; n < ntiles; n += 2) {
        step_any(n, std::false_type{});
        if (n + 1 < ntiles) step_any(n + 1, std::true_type{});
      }
    }


    // The next item's first tile, query rows and tile-1 page ids: every
    // buffer is free after the last step's barrier (or the one above), and
    // the epilogue below uses registers only.
    if (it + 1 < it_end) {
      load_q(nxt);
      if constexpr (!FAST) {
        npk = fetch_k(nc, 0);
        npv = fetch_v(nc, 0);
      }
      if (nc.ntiles > 0) {
        dma_k(nc, 0, k_lds0, npk);
        load_v(nc, 0, npk, npv);
      }
      pk = fetch_k(nc, 1);
      pv_ids = fetch_v(nc, 1);
    }

    // ---- epilogue: normalise and write this lane's row (dims 32 d + 8 i + 4 hh + j)
    const float l_tot = half_sum(l_part);
    const bool empty = m_run == neg_inf() || !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_nat = empty ? neg_inf() : (m_run + fast_log2(l_tot)) * kLn2;
    if (row_valid) {
      if (slot < 0) {
        const int64_t orow = (int64_t)(qbase + tok) * a.Hq + head;
#pragma unroll
        for (int d = 0; d < SH::DBlocks; ++d)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int dim = 32 * d + 8 * i + 4 * hh;
            const float v0 = oacc[d][4 * i] * inv, v1 = oacc[d][4 * i + 1] * inv;
            const float v2 = oacc[d][4 * i + 2] * inv, v3 = oacc[d][4 * i + 3] * inv;
            if constexpr (OT::kBytes == 2) {
              u32x2_t w;
              w[0] = pack_bf16x2(v0, v1);
              w[1] = pack_bf16x2(v2, v3);
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
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4_t*>(ws_o + prow * D + 32 * d + 8 * i + 4 * hh) =
                f32x4_t{oacc[d][4 * i] * inv, oacc[d][4 * i + 1] * inv, oacc[d][4 * i + 2] * inv,
                        oacc[d][4 * i + 3] * inv};
        if (hh == 0) ws_lse[prow] = lse_nat;
      }
    }
    item = nxt;
  }
  report_status(a.status, bad_page, kStatusBadPage);
}

template <int D, int G, bool FAST, bool CAP, bool WIN, bool ROPE, bool MASK, typename OT>
int launch_k(const RunArgs& r, const PrefillParams& p) {
  dim3 grid(r.workers * r.Hk), block(kThreads);
  hipLaunchKernelGGL((prefill_kernel<D, G, FAST, CAP, WIN, ROPE, MASK, OT>), grid, block, 0, (hipStream_t)r.hip_stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FI_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return FI_OK;
}

template <int D, int G, bool WIN, bool ROPE, bool MASK, typename OT>
int launch_t(const RunArgs& r, const PrefillParams& p) {
  const bool fast = p.page_shift >= 0, cap = p.cap > 0.f;
  if (fast) return cap ? launch_k<D, G, true, true, WIN, ROPE, MASK, OT>(r, p) : launch_k<D, G, true, false, WIN, ROPE, MASK, OT>(r, p);
  return cap ? launch_k<D, G, false, true, WIN, ROPE, MASK, OT>(r, p) : launch_k<D, G, false, false, WIN, ROPE, MASK, OT>(r, p);
}

template <int D, bool WIN, bool ROPE, bool MASK, typename OT>
int launch_g(const RunArgs& r, const PrefillParams& p) {
  switch (r.G) {
    case 1: return launch_t<D, 1, WIN, ROPE, MASK, OT>(r, p);
    case 2: return launch_t<D, 2, WIN, ROPE, MASK, OT>(r, p);
    case 4: return launch_t<D, 4, WIN, ROPE, MASK, OT>(r, p);
    case 8: return launch_t<D, 8, WIN, ROPE, MASK, OT>(r, p);
  }
  return set_error(FI_ERR_UNSUPPORTED, "prefill: group size %d", r.G);
}

template <bool WIN, bool ROPE, bool MASK, typename OT>
int launch_d(const RunArgs& r, const PrefillParams& p) {
  if (r.D == 64) return launch_g<64, WIN, ROPE, MASK, OT>(r, p);
  if (r.D == 128) return launch_g<128, WIN, ROPE, MASK, OT>(r, p);
  return set_error(FI_ERR_UNSUPPORTED, "prefill: head_dim %d", r.D);
}

// The kernels of one window / rotary mode, for the output type of the call.
template <bool WIN, bool ROPE, bool MASK = false>
int launch_mode(const RunArgs& r, const PrefillParams& p) {
  if (r.out_dtype == FI_BF16) return launch_d<WIN, ROPE, MASK, BF16>(r, p);
  return launch_d<WIN, ROPE, MASK, F32>(r, p);
}

}  // namespace

// defined in prefill_window.hip, prefill_rope.hip and prefill_mask.hip
int launch_prefill_window(const RunArgs& r, const PrefillParams& p);
int launch_prefill_rope(const RunArgs& r, const PrefillParams& p);
int launch_prefill_mask(const RunArgs& r, const PrefillParams& p);

}  // namespace fi
