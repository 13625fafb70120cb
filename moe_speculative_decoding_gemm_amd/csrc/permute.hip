// Standalone permute / group-by-expert kernel (one 1024-thread work-group,
// see amoe_permute.h), the shared-expert identity grouping, and the
// unpermute + gate-weighted combine [MoE-SD blog, MoE layer].

#include "amoe_common.h"
#include "amoe_launch.h"
#include "amoe_permute.h"

namespace amoe {

namespace {

__global__ __launch_bounds__(1024) void permute_kernel(int N, int k, int E,
                                                       const int32_t* __restrict__ topk_idx,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_assign,
                                                       int32_t* __restrict__ inv_pos,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ n_active,
                                                       const uint8_t* __restrict__ resident,
                                                       StatsDev* __restrict__ stats) {
  __shared__ PermuteSmem<1024> sm;
  permute_block<1024>(N, k, E, topk_idx, counts, offsets, sorted_assign, inv_pos, active,
                      n_active, resident, stats, sm);
}

__global__ void shared_grouping_kernel(int N, int32_t* offsets, int32_t* sorted_assign,
                                       int32_t* active, int32_t* n_active) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < N) sorted_assign[t] = t;
  if (t == 0) {
    offsets[0] = 0;
    offsets[1] = N;
    active[0] = 0;
    n_active[0] = 1;
  }
}

// y[i, h..h+3] = sum_j g[i][j] * y_perm[inv_pos[i*k+j]][h..h+3] (+ y_shared),
// summed in slot order j = 0..k-1; all loads of a thread are issued up front.
// kTok: the rows are already in token-major order (row i*k + j), so the
// loads need no inv_pos round trip first; the arithmetic is the same.
// KK > 0: k is KK (the loops have no bounds to test at run time); 0: k as
// given.
template <bool kBf16, bool kTok, int KK>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c) {
  const int N = c.N, k = KK > 0 ? KK : c.k, H = c.H;
  constexpr int KM = KK > 0 ? KK : kMaxK;
  const int h4 = H >> 2;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(N) * h4) return;
  const int i = static_cast<int>(idx / h4);
  const int h = static_cast<int>(idx - static_cast<size_t>(i) * h4) * 4;
  const float* src[KM];
  float g[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      const int row = kTok ? i * k + j : c.inv_pos[static_cast<size_t>(i) * k + j];
      src[j] = c.y_perm + static_cast<size_t>(row) * H;
      g[j] = c.gate[static_cast<size_t>(i) * k + j];
    }
  }
  f32x4_t v[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) v[j] = *reinterpret_cast<const f32x4_t*>(src[j] + h);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(g[j], v[j][q], acc[q]);
    }
  if (c.y_shared)
    acc += *reinterpret_cast<const f32x4_t*>(c.y_shared + static_cast<size_t>(i) * H + h);
  if (kBf16) {
    u32x2_t o;
    o[0] = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o[1] = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(c.y) + static_cast<size_t>(i) * H + h) = o;
  } else {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(c.y) + static_cast<size_t>(i) * H + h) = acc;
  }
}

template <bool kBf16, int KK>
void launch_combine_k(const CombineArgs& c, unsigned blocks, hipStream_t stream) {
  if (c.inv_pos)
    combine_kernel<kBf16, false, KK><<<blocks, 256, 0, stream>>>(c);
  else
    combine_kernel<kBf16, true, KK><<<blocks, 256, 0, stream>>>(c);
}
template <bool kBf16>
void launch_combine_t(const CombineArgs& c, unsigned blocks, hipStream_t stream) {
  if (c.k == 8)
    launch_combine_k<kBf16, 8>(c, blocks, stream);
  else if (c.k == 4)
    launch_combine_k<kBf16, 4>(c, blocks, stream);
  else
    launch_combine_k<kBf16, 0>(c, blocks, stream);
}

}  // namespace

hipError_t launch_permute(int N, int k, int E, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_assign, int32_t* inv_pos,
                          int32_t* active, int32_t* n_active, const uint8_t* resident,
                          void* stats, hipStream_t stream) {
  permute_kernel<<<1, 1024, 0, stream>>>(N, k, E, topk_idx, counts, offsets, sorted_assign,
                                         inv_pos, active, n_active, resident,
                                         static_cast<StatsDev*>(stats));
  return hipGetLastError();
}

hipError_t launch_shared_grouping(int N, int32_t* offsets, int32_t* sorted_assign,
                                  int32_t* active, int32_t* n_active, hipStream_t stream) {
  shared_grouping_kernel<<<(N + 255) / 256, 256, 0, stream>>>(N, offsets, sorted_assign,
                                                              active, n_active);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream) {
  const size_t n = static_cast<size_t>(c.N) * (c.H / 4);
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (c.act_bf16)
    launch_combine_t<true>(c, blocks, stream);
  else
    launch_combine_t<false>(c, blocks, stream);
  return hipGetLastError();
}

}  // namespace amoe
