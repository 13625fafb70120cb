// Device-side helpers shared by the AcceptMoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace amoe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;

// error bits (same values as ACCEPTMOE_ERR_* in the public header)
constexpr int kErrBadTree = 1;
constexpr int kErrDepth = 2;
constexpr int kErrNonFinite = 4;
constexpr int kErrCommit = 8;

constexpr uint32_t kFlagNatural = 1u;
constexpr uint32_t kFlagNoRenorm = 2u;
constexpr uint32_t kFlagLogitsIn = 4u;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u)
    return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_act(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ------------------------------------------------------- top-k keys -------
// A 64-bit key that orders (logit descending, expert index ascending) as an
// unsigned integer: high word = logit bits mapped to an order-preserving
// unsigned (with -0 folded onto +0), low word = ~index.  Key 0 is below every
// real key and marks an empty / excluded slot.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}
__device__ __forceinline__ int key_expert(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}

// ----------------------------------------------------- wave reductions ----
// xor butterflies: every lane ends with the same, bitwise identical result
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, kWave);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

}  // namespace amoe
