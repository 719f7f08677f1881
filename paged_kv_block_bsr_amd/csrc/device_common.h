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

}  // namespace fi
