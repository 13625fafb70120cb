// Permute / group-by-expert of the N*k assignments [MoE-SD blog, MoE layer],
// and the unpermute + gate-weighted combine.
//
// permute: one 1024-thread work-group.  Pass 1 is an LDS histogram (integer
// atomics: the counts do not depend on their order).  A single wave scans the
// counts into offsets and compacts the active experts.  Pass 2 scatters in
// rounds of 1024 assignments: inside a wave, lanes with the same expert find
// each other with eight ballots over the expert-id bits and take their rank
// from a popcount of the lower peers; per-wave totals are scanned across the
// 16 waves in wave order.  Ranks therefore follow assignment order and the
// sort is stable and deterministic.

#include "amoe_common.h"
#include "amoe_launch.h"

namespace amoe {

namespace {

struct StatsDev {  // mirrors acceptmoe_stats
  int32_t n_anchor, n_selfsize, n_eligible, n_pruned, n_active, n_active_nonresident,
      n_natural_union, err_flags;
  double r_eff, demand_total;
};

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// exclusive scan of v[0..n) (n <= 256) by one wave; returns the total
__device__ int wave_exclusive_scan_256(const int* v, int* out, int n) {
  const int lane = lane_id();
  int loc[4];
  int s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = lane * 4 + q;
    loc[q] = s;
    s += idx < n ? v[idx] : 0;
  }
  int inc = s;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  const int base = inc - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = lane * 4 + q;
    if (idx < n) out[idx] = base + loc[q];
  }
  return __shfl(inc, kWave - 1, kWave);
}

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
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_off[kMaxE];
  __shared__ int s_flag[kMaxE];
  __shared__ int s_apos[kMaxE];
  __shared__ int s_run[kMaxE];
  __shared__ int s_w[16][kMaxE];
  __shared__ int s_nact;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = lane_id();
  const int total = N * k;
  if (t < kMaxE) {
    s_cnt[t] = 0;
    s_run[t] = 0;
  }
  __syncthreads();
  // an out-of-range expert id (a caller error) is clamped so that no access
  // leaves its buffer; the grouping is then unspecified but memory-safe
  for (int x = t; x < total; x += 1024) atomicAdd(&s_cnt[clamp_expert(topk_idx[x], E)], 1);
  __syncthreads();
  if (t < E) s_flag[t] = s_cnt[t] > 0 ? 1 : 0;
  __syncthreads();
  if (wave == 0) {
    wave_exclusive_scan_256(s_cnt, s_off, E);
    const int na = wave_exclusive_scan_256(s_flag, s_apos, E);
    if (lane == 0) s_nact = na;
  }
  __syncthreads();
  if (t < E) {
    counts[t] = s_cnt[t];
    offsets[t] = s_off[t];
    if (s_flag[t]) active[s_apos[t]] = t;
  }
  if (t == 0) {
    offsets[E] = total;
    n_active[0] = s_nact;
  }
  if (stats && t < kWave) {
    int nr = 0;
    if (resident)
      for (int e = t; e < E; e += kWave) nr += (s_flag[e] && !resident[e]) ? 1 : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) nr += __shfl_xor(nr, m, kWave);
    if (t == 0) {
      stats->n_active = s_nact;
      stats->n_active_nonresident = nr;
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < total; base += 1024) {
    const int x = base + t;
    const bool valid = x < total;
    const int e = valid ? clamp_expert(topk_idx[x], E) : 0;
    for (int q = lane; q < E; q += kWave) s_w[wave][q] = 0;
    const uint64_t vmask = __ballot(valid);
    uint64_t peers = vmask;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t mb = __ballot(valid && bit);
      peers &= bit ? mb : ~mb;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) s_w[wave][e] = __popcll(peers);
    __syncthreads();
    if (t < E) {
      int run = s_run[t];
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int c = s_w[w][t];
        s_w[w][t] = run;
        run += c;
      }
      s_run[t] = run;
    }
    __syncthreads();
    if (valid) {
      const int pos = s_off[e] + s_w[wave][e] + rank;
      sorted_assign[pos] = x;
      inv_pos[x] = pos;
    }
    __syncthreads();
  }
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

// y[i, h..h+3] = sum_j g[i][j] * y_perm[inv_pos[i*k+j]][h..h+3] (+ y_shared)
template <bool kBf16>
__global__ __launch_bounds__(256) void combine_kernel(int N, int k, int H,
                                                      const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ y_shared,
                                                      void* __restrict__ y) {
  const int h4 = H >> 2;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(N) * h4) return;
  const int i = static_cast<int>(idx / h4);
  const int h = static_cast<int>(idx - static_cast<size_t>(i) * h4) * 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float g = gate[static_cast<size_t>(i) * k + j];
    const int row = inv_pos[static_cast<size_t>(i) * k + j];
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(y_perm + static_cast<size_t>(row) * H + h);
    acc += g * v;
  }
  if (y_shared) acc += *reinterpret_cast<const f32x4_t*>(y_shared + static_cast<size_t>(i) * H + h);
  if (kBf16) {
    u32x2_t o;
    o[0] = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o[1] = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(y) + static_cast<size_t>(i) * H + h) = o;
  } else {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + static_cast<size_t>(i) * H + h) = acc;
  }
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

hipError_t launch_combine(int N, int k, int H, int act_bf16, const float* y_perm,
                          const int32_t* inv_pos, const float* topk_gate, const float* y_shared,
                          void* y, hipStream_t stream) {
  const size_t n = static_cast<size_t>(N) * (H / 4);
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (act_bf16)
    combine_kernel<true><<<blocks, 256, 0, stream>>>(N, k, H, y_perm, inv_pos, topk_gate,
                                                     y_shared, y);
  else
    combine_kernel<false><<<blocks, 256, 0, stream>>>(N, k, H, y_perm, inv_pos, topk_gate,
                                                      y_shared, y);
  return hipGetLastError();
}

}  // namespace amoe
