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
typedef __attribute__((ext_vector_type(2))) double f64x2_t;

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;

// error bits (same values as ACCEPTMOE_ERR_* in the public header)
constexpr int kErrBadTree = 1;
constexpr int kErrDepth = 2;
constexpr int kErrNonFinite = 4;
constexpr int kErrCommit = 8;
constexpr int kErrWorkspace = 16;  // an arrival counter was not zero at the start of a call

constexpr uint32_t kFlagNatural = 1u;
constexpr uint32_t kFlagNoRenorm = 2u;
constexpr uint32_t kFlagLogitsIn = 4u;
constexpr uint32_t kFlagDemandFull = 8u;   // demand over every expert's score
constexpr uint32_t kFlagNoAnchor = 16u;    // no root anchor
constexpr uint32_t kFlagUnitCommit = 32u;  // every draft position weighs 1
constexpr uint32_t kFlagsKnown = 63u;

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

// SiLU of the SwiGLU experts [MoE-SD blog, MoE layer]: z * sigmoid(z)
// (the hardware reciprocal, not a correctly rounded divide: every expert
// kernel takes this same function, so all paths give the same bits)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

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
// Reductions over the 64 lanes with DPP moves inside each 16-lane row (xor 1,
// xor 2, half-row mirror, row mirror) and one readlane per row.  Partner
// values are combined commutatively, so every lane holds the same bits at
// every step, and the four row results are combined in a fixed order: the
// result is identical in all lanes and from run to run.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele steps inside each
// 16-lane row with DPP row shifts (lanes shifted in from outside the row
// read 0), then the totals of the rows below added from three readlanes.
// Integer adds: exact, so the order does not matter.
template <int SHR>
__device__ __forceinline__ uint32_t row_shr_zero(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x110 + SHR, 0xf, 0xf, true));
}
__device__ __forceinline__ uint32_t wave_inclusive_sum_u32(uint32_t v) {
  v += row_shr_zero<1>(v);
  v += row_shr_zero<2>(v);
  v += row_shr_zero<4>(v);
  v += row_shr_zero<8>(v);
  const uint32_t r0 = readlane_u32(v, 15), r1 = readlane_u32(v, 31), r2 = readlane_u32(v, 47);
  const int row = (static_cast<int>(threadIdx.x) & (kWave - 1)) >> 4;
  return v + (row == 0 ? 0u : (row == 1 ? r0 : (row == 2 ? r0 + r1 : r0 + r1 + r2)));
}

template <int CTRL>
__device__ __forceinline__ void max_step_u64(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = dpp_mov<CTRL>(hi), ol = dpp_mov<CTRL>(lo);
  const bool t = oh > hi || (oh == hi && ol > lo);
  hi = t ? oh : hi;
  lo = t ? ol : lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint32_t hi = static_cast<uint32_t>(v >> 32), lo = static_cast<uint32_t>(v);
  max_step_u64<kDppXor1>(hi, lo);
  max_step_u64<kDppXor2>(hi, lo);
  max_step_u64<kDppHalfMirror>(hi, lo);
  max_step_u64<kDppMirror>(hi, lo);
  uint64_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint64_t o = (static_cast<uint64_t>(readlane_u32(hi, 16 * row)) << 32) |
                       readlane_u32(lo, 16 * row);
    r = o > r ? o : r;
  }
  return r;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o = dpp_mov<kDppXor1>(v);
  v = o > v ? o : v;
  o = dpp_mov<kDppXor2>(v);
  v = o > v ? o : v;
  o = dpp_mov<kDppHalfMirror>(v);
  v = o > v ? o : v;
  o = dpp_mov<kDppMirror>(v);
  v = o > v ? o : v;
  uint32_t r = readlane_u32(v, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const uint32_t x = readlane_u32(v, 16 * row);
    r = x > r ? x : r;
  }
  return r;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_mov<CTRL>(__float_as_uint(v)));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  float r = __uint_as_float(readlane_u32(__float_as_uint(v), 0));
#pragma unroll
  for (int row = 1; row < 4; ++row) r = fmaxf(r, __uint_as_float(readlane_u32(__float_as_uint(v), 16 * row)));
  return r;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t o = (static_cast<uint64_t>(dpp_mov<CTRL>(static_cast<uint32_t>(u >> 32))) << 32) |
                     dpp_mov<CTRL>(static_cast<uint32_t>(u));
  return __builtin_bit_cast(double, o);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t o = (static_cast<uint64_t>(readlane_u32(static_cast<uint32_t>(u >> 32), lane)) << 32) |
                     readlane_u32(static_cast<uint32_t>(u), lane);
  return __builtin_bit_cast(double, o);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = v + dpp_f64<kDppXor1>(v);
  v = v + dpp_f64<kDppXor2>(v);
  v = v + dpp_f64<kDppHalfMirror>(v);
  v = v + dpp_f64<kDppMirror>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// Wait until this wave's outstanding global stores have been acknowledged by
// the L2 of its XCD (s_waitcnt vmcnt(0); expcnt and lgkmcnt left alone).  A
// work-group barrier alone does not wait for them.
__device__ __forceinline__ void wait_global_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Device-scope (agent) stores and loads: they bypass the caches that are
// not coherent across XCDs (the per-XCD L2 and the CU's L1), so data that
// work-groups of one kernel hand to each other through them needs no cache
// write-back or invalidation -- whole-cache operations that stall the other
// waves of the XCD.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last-arriver election for data written with store_dev and read with
// load_dev.  Every thread of the work-group calls it after its store_dev
// writes; it returns true in exactly one of the nblocks work-groups counting
// on the same counter, the last to arrive, which may then load_dev what the
// others wrote.  Each wave waits until its device-scope stores are complete
// before the barrier; one thread then counts the arrival with an atomic
// whose returned value decides.  The counter must be zero before the first
// arrival; the last arriver resets it.  A count outside [0, nblocks) means
// the counter did not start at zero (a workspace that was not zero-filled,
// or shared by calls that overlap): kErrWorkspace is then OR-ed into
// *misuse, and the caller's kernels still only read and write in range.
__device__ __forceinline__ bool last_arrival_dev(int* counter, int nblocks, int* misuse) {
  __shared__ int s_last_dev;
  wait_global_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == nblocks - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev < 0 || prev >= nblocks)
      __hip_atomic_fetch_or(misuse, kErrWorkspace, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last_dev = last ? 1 : 0;
  }
  __syncthreads();
  return s_last_dev != 0;
}

}  // namespace amoe
