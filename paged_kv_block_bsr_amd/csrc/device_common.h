// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_format.h"

namespace fi {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage type tags: the kernels read and write raw bits.
struct BF16 {
  static constexpr int kBytes = 2;
};
struct F32 {
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 values as a bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// tanh from its definition, tanh(y) = 1 - 2 / (e^{2y} + 1), with the
// hardware reciprocal; saturates to +-1 (e -> inf gives 1, e -> 0 gives -1).
__device__ __forceinline__ float tanh_from_exp(float y) {
  float e = fast_exp2(2.0f * kLog2e * y);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Element i of a 16-byte piece holding elements of storage type T, as float.
template <typename T>
__device__ __forceinline__ float piece_elem(const u32x4_t& v, int i);

template <>
__device__ __forceinline__ float piece_elem<BF16>(const u32x4_t& v, int i) {
  uint32_t w = v[i >> 1];
  return (i & 1) ? bf16_hi(w) : bf16_lo(w);
}

template <>
__device__ __forceinline__ float piece_elem<F32>(const u32x4_t& v, int i) {
  return __uint_as_float(v[i]);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

#define FI_LDS __attribute__((address_space(3)))

// Sets `bits` in the status word when `bad` is nonzero in some lane of the
// wave: the lowest such lane does one vector-memory atomic OR.
__device__ __forceinline__ void report_status(int32_t* status, uint32_t bad, int32_t bits) {
  const uint64_t m = __ballot(bad != 0);
  if (m != 0 && (uint32_t)__lane_id() == (uint32_t)(__ffsll((unsigned long long)m) - 1))
    __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- rotary embedding (rotate-half form: the pair (x[d], x[d + D/2]) turns
// by pos / scale * theta^(-2d/D)).  The host supplies, per pair d, the turn
// per position as a 32-bit fixed-point fraction of a revolution; the angle of
// a position is that times pos modulo 2^32 (exact integer arithmetic, whole
// turns drop out), and v_sin / v_cos take it in revolutions.  Tables are read
// from LDS through address-space-3 pointers only: a flat load would also count
// in the vector-memory counter the kernels wait on by hand.
constexpr int kRopeMaxPairs = 64;

__device__ __forceinline__ void rope_cos_sin(uint32_t f, int pos, float& c, float& s) {
  const float rev = (float)(int32_t)((uint32_t)pos * f) * 0x1p-32f;  // in [-0.5, 0.5)
  c = __builtin_amdgcn_cosf(rev);
  s = __builtin_amdgcn_sinf(rev);
}

// Two fp32 values as an fp16 pair (lo in bits 0..15), round to nearest even,
// saturating at +-65504 instead of overflowing.
__device__ __forceinline__ uint32_t pack_f16x2_sat(float lo, float hi) {
  lo = __builtin_amdgcn_fmed3f(lo, -65504.f, 65504.f);
  hi = __builtin_amdgcn_fmed3f(hi, -65504.f, 65504.f);
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Rotate the pairs held by two 16-byte pieces of storage type T: `lo` has
// dims d0 .. d0 + n - 1, `hi` the same dims + D/2 (n = 16 / sizeof(T)); f is
// the table at d0.  bf16 pieces come back as fp16 (11-bit significand, round
// to nearest even, saturating): the rotated values feed fp16 matrix-core
// products, whose rounding keeps the logits within the attention tolerance
// where bf16's 8 bits would not.  fp32 pieces stay fp32.
template <typename T>
__device__ __forceinline__ void rope_pieces(u32x4_t& lo, u32x4_t& hi, const FI_LDS uint32_t* f,
                                            int pos) {
  if constexpr (T::kBytes == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float c0, s0, c1, s1;
      rope_cos_sin(f[2 * w], pos, c0, s0);
      rope_cos_sin(f[2 * w + 1], pos, c1, s1);
      const float a0 = bf16_lo(lo[w]), a1 = bf16_hi(lo[w]);
      const float b0 = bf16_lo(hi[w]), b1 = bf16_hi(hi[w]);
      lo[w] = pack_f16x2_sat(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
      hi[w] = pack_f16x2_sat(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float c, s;
      rope_cos_sin(f[w], pos, c, s);
      const float a = __uint_as_float(lo[w]), b = __uint_as_float(hi[w]);
      lo[w] = __float_as_uint(a * c - b * s);
      hi[w] = __float_as_uint(b * c + a * s);
    }
  }
}

}  // namespace fi
