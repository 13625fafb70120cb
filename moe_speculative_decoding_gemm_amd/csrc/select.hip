// AcceptMoE expert selection on gfx950: router product, per-node softmax and
// natural top-k, commitment-weighted demand, anchor, self-sizing,
// residency-aware pruning, restricted top-k and gates.
//
// Sources: [MoE-SD blog, MoE layer] for the router (softmax over all experts,
// top-k routing); [AcceptMoE news §02] and [AcceptMoE abstract] for demand,
// root anchor, self-sizing by effective rank and residency-aware pruning;
// [AcceptMoE abstract] for restricting top-k to the eligible set.
//
// Three kernels, all wave64:
//   router_partial  grid (E/64, N/64, ksplit): 64x64 logit tile over one K slice
//                   per work-group, fp32 FMA from LDS (vector ALU: the router is
//                   a few MFLOP at batch one; matrix cores are kept for the
//                   expert contractions).
//   node            one wave per node (16 per work-group): sum of the K-slice
//                   partials + bias, fp64 softmax statistics, natural top-k by
//                   64-bit (logit, ~index) keys, dense demand terms
//                   c[depth] * p for the node's top-k.  The last work-group to
//                   finish then selects the set: demand per expert (fixed
//                   summation order), entropy, set size, anchor + fill by rank
//                   counting, pruning by rank counting, statistics.
//   restricted      one wave per node: top-k over the eligible experts and the
//                   gates; the last work-group to finish groups the
//                   assignments by expert (verify_block only).
// Arrival counters are reset by the kernel before, in stream order, so no
// memset is needed.  Every reduction has a fixed order: two runs give
// identical bits.

#include "amoe_common.h"
#include "amoe_launch.h"
#include "amoe_permute.h"

namespace amoe {

namespace {

constexpr int kRT = 64;   // router tile (tokens and experts)
constexpr int kRKC = 32;  // router K chunk staged in LDS

template <typename AT>
__device__ __forceinline__ void load8(const AT* p, float* out);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* out) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

// logits partial sums over one K slice: part[ks][n][e] = sum_k x[n][k] w[e][k]
template <typename AT>
__global__ __launch_bounds__(256) void router_partial_kernel(const AT* __restrict__ x,
                                                             const AT* __restrict__ w, int N,
                                                             int E, int H, int kslice,
                                                             float* __restrict__ part,
                                                             int32_t* __restrict__ counters,
                                                             int compute) {
  __shared__ float xs[kRKC][kRT + 4];
  __shared__ float wsm[kRKC][kRT + 4];
  const int t = threadIdx.x;
  if (t == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) counters[0] = 0;
  if (!compute) return;
  const int e0 = blockIdx.x * kRT, n0 = blockIdx.y * kRT, ks = blockIdx.z;
  const int kbeg = ks * kslice;
  const int kend = min(H, kbeg + kslice);
  const int ty = t >> 4, tx = t & 15;
  const int lr = t >> 2, lk = (t & 3) * 8;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int kb = kbeg; kb < kend; kb += kRKC) {
    float v[8];
    const int n = n0 + lr;
    if (n < N) {
      load8<AT>(x + static_cast<size_t>(n) * H + kb + lk, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[lk + i][lr] = v[i];
    const int e = e0 + lr;
    if (e < E) {
      load8<AT>(w + static_cast<size_t>(e) * H + kb + lk, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) wsm[lk + i][lr] = v[i];
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kRKC; ++kk) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&xs[kk][ty * 4]);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&wsm[kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + ty * 4 + i;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) part[(static_cast<size_t>(ks) * N + n) * E + e] = acc[i][j];
    }
  }
}

// set selection by one 1024-thread work-group (the last node work-group)
__device__ void select_set(const SelectArgs& a);

// one wave per node, 16 nodes per work-group
__global__ __launch_bounds__(1024) void node_kernel(SelectArgs a) {
  const int lane = lane_id();
  const int i = blockIdx.x * 16 + static_cast<int>(threadIdx.x >> 6);
  if (threadIdx.x == 0 && blockIdx.x == 0) a.counters[1] = 0;
  if (i < a.N) {
    const int E = a.E, k = a.k;
    const bool logits_in = (a.flags & kFlagLogitsIn) != 0;
    float l[4];
    bool valid[4];
    bool nonfinite = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + kWave * q;
      valid[q] = e < E;
      float v = 0.f;
      if (valid[q]) {
        if (logits_in) {
          v = a.logits_in[static_cast<size_t>(i) * E + e];
        } else {
          // partial sums in K-slice order; loads issued eight at a time
          const float* p = a.part + static_cast<size_t>(i) * E + e;
          const size_t stride = static_cast<size_t>(a.N) * E;
          float s = 0.f;
          int ks = 0;
          for (; ks + 8 <= a.ksplit; ks += 8) {
            float t8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) t8[u] = p[(ks + u) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += t8[u];
          }
          for (; ks < a.ksplit; ++ks) s += p[ks * stride];
          v = s + (a.b_router ? a.b_router[e] : 0.f);
        }
        a.logits[static_cast<size_t>(i) * E + e] = v;
        if (a.logits_out) a.logits_out[static_cast<size_t>(i) * E + e] = v;
        if (!isfinite(v)) nonfinite = true;
      }
      l[q] = v;
    }
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (valid[q]) m = fmaxf(m, l[q]);
    m = wave_max_f32(m);
    double zs = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (valid[q]) zs += exp(static_cast<double>(l[q]) - static_cast<double>(m));
    const double z = wave_sum_f64(zs);

    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) key[q] = valid[q] ? topk_key(l[q], lane + kWave * q) : 0ull;
    int my_nat = 0;       // lane j keeps the j-th natural expert
    uint32_t in_nat = 0;  // bit q: slot q is in the natural top-k
    for (int j = 0; j < k; ++j) {
      uint64_t b = key[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) b = key[q] > b ? key[q] : b;
      b = wave_max_u64(b);
      const int ew = b ? key_expert(b) : 0;
      if ((ew & (kWave - 1)) == lane) {
        const int q = ew >> 6;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (qq == q) {
            key[qq] = 0ull;
            in_nat |= 1u << qq;
          }
      }
      if (lane == j) my_nat = ew;
    }
    if (lane < k) a.nat[static_cast<size_t>(i) * k + lane] = my_nat;

    const int d = a.depth[i];
    const int dc = d < 0 ? 0 : (d >= a.n_depth ? a.n_depth - 1 : d);
    const double c = static_cast<double>(a.commit[dc]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!valid[q]) continue;
      const int e = lane + kWave * q;
      double t = 0.0;
      if (in_nat & (1u << q)) t = c * (exp(static_cast<double>(l[q]) - static_cast<double>(m)) / z);
      a.contrib[static_cast<size_t>(i) * E + e] = t;
    }
    const bool any_nf = __ballot(nonfinite) != 0ull;
    if (lane == 0) {
      int err = any_nf ? kErrNonFinite : 0;
      const int p = a.parent[i];
      if (d < 0 || d >= a.n_depth) err |= kErrDepth;
      if (p == -1) {
        if (d != 0) err |= kErrBadTree;
      } else if (p < 0 || p >= i) {
        err |= kErrBadTree;
      } else if (d != a.depth[p] + 1) {
        err |= kErrBadTree;
      }
      a.node_err[i] = err;
      a.node_m[i] = m;
      a.node_z[i] = z;
    }
  }
  if (last_block_done(&a.counters[0], gridDim.x)) select_set(a);
}

__device__ void select_set(const SelectArgs& a) {
  __shared__ double s_part[1024];
  __shared__ double s_d[kMaxE];
  __shared__ int s_anchor[kMaxE], s_natused[kMaxE], s_rank[kMaxE], s_elig[kMaxE];
  __shared__ int s_err, s_na, s_nnat, s_nsel, s_ncand;
  __shared__ double s_tot, s_h;
  const int t = threadIdx.x;
  const int N = a.N, E = a.E, k = a.k;
  const bool natural = (a.flags & kFlagNatural) != 0;
  if (t < kMaxE) {
    s_anchor[t] = 0;
    s_natused[t] = 0;
    s_rank[t] = 0;
  }
  if (t == 0) {
    s_err = 0;
    s_na = 0;
    s_nnat = 0;
    s_nsel = 0;
    s_ncand = 0;
  }
  __syncthreads();
  for (int i = t; i < N; i += 1024) {
    const int e = a.node_err[i];
    if (e) atomicOr(&s_err, e);
  }
  for (int d = t; d < a.n_depth; d += 1024) {
    const float c = a.commit[d];
    if (!(c >= 0.f) || isinf(c)) atomicOr(&s_err, kErrCommit);
  }
  for (int x = t; x < N * k; x += 1024) {
    const int e = a.nat[x];
    s_natused[e] = 1;
    if (a.parent[x / k] == -1) s_anchor[e] = 1;
  }
  // demand: G groups of consecutive nodes, summed in group order
  const int G = 1024 / E;
  {
    const int g = t / E, e = t - g * E;
    double s = 0.0;
    if (g < G) {
      const int chunk = (N + G - 1) / G;
      const int lo = g * chunk, hi = min(N, lo + chunk);
      for (int i = lo; i < hi; ++i) s += a.contrib[static_cast<size_t>(i) * E + e];
    }
    s_part[t] = s;
  }
  __syncthreads();
  if (t < E) {
    double d = 0.0;
    for (int g = 0; g < G; ++g) d += s_part[g * E + t];
    s_d[t] = d;
    if (s_anchor[t]) atomicAdd(&s_na, 1);
    if (s_natused[t]) atomicAdd(&s_nnat, 1);
  }
  __syncthreads();
  if (t < kWave) {  // wave 0: total demand and entropy, fixed order
    double s = 0.0;
    for (int e = t; e < E; e += kWave) s += s_d[e];
    const double tot = wave_sum_f64(s);
    double h = 0.0;
    if (tot > 0.0) {
      for (int e = t; e < E; e += kWave) {
        const double d = s_d[e];
        if (d > 0.0) {
          const double q = d / tot;
          h -= q * log(q);
        }
      }
    }
    h = wave_sum_f64(h);
    if (t == 0) {
      s_tot = tot;
      s_h = h;
    }
  }
  __syncthreads();
  const double tot = s_tot;
  const double r_eff = tot > 0.0 ? exp(s_h) : 0.0;
  const int n_anchor = s_na;
  const int n_min = max(k, a.min_set);
  const int n_raw = a.fixed_budget > 0 ? a.fixed_budget : static_cast<int>(floor(r_eff + 0.5));
  const int n = min(E, max(max(n_raw, n_anchor), n_min));
  const int take = n - n_anchor;
  // fill: rank of each non-anchor expert under (demand desc, index asc)
  {
    const int g = t / E, e = t - g * E;
    if (g < G && !s_anchor[e]) {
      const int chunk = (E + G - 1) / G;
      const int lo = g * chunk, hi = min(E, lo + chunk);
      const double de = s_d[e];
      int r = 0;
      for (int f = lo; f < hi; ++f)
        if (!s_anchor[f] && (s_d[f] > de || (s_d[f] == de && f < e))) ++r;
      if (r) atomicAdd(&s_rank[e], r);
    }
  }
  __syncthreads();
  if (t < E) {
    const int el = natural ? 1 : (s_anchor[t] || s_rank[t] < take) ? 1 : 0;
    s_elig[t] = el;
    if (el) atomicAdd(&s_nsel, 1);
  }
  __syncthreads();
  const int n_selfsize = s_nsel;
  int n_remove = 0;
  if (!natural && a.resident) {
    if (t < E) {
      s_rank[t] = 0;
      const int cand = s_elig[t] && !s_anchor[t] && !a.resident[t];
      if (cand) atomicAdd(&s_ncand, 1);
    }
    __syncthreads();
    n_remove = max(0, min(a.reroute_budget, min(n_selfsize - n_min, s_ncand)));
    // rank among candidates under (demand asc, index desc)
    const int g = t / E, e = t - g * E;
    const bool ce = (t < 1024) && g < G && s_elig[e] && !s_anchor[e] && !a.resident[e];
    if (ce) {
      const int chunk = (E + G - 1) / G;
      const int lo = g * chunk, hi = min(E, lo + chunk);
      const double de = s_d[e];
      int r = 0;
      for (int f = lo; f < hi; ++f) {
        const bool cf = s_elig[f] && !s_anchor[f] && !a.resident[f];
        if (cf && (s_d[f] < de || (s_d[f] == de && f > e))) ++r;
      }
      if (r) atomicAdd(&s_rank[e], r);
    }
    __syncthreads();
    if (t < E) {
      const bool c = s_elig[t] && !s_anchor[t] && !a.resident[t];
      if (c && s_rank[t] < n_remove) s_elig[t] = 0;
    }
    __syncthreads();
  }
  if (t < E) a.eligible[t] = static_cast<uint8_t>(s_elig[t]);
  if (t == 0) {
    StatsDev* st = reinterpret_cast<StatsDev*>(a.stats);
    st->n_anchor = n_anchor;
    st->n_selfsize = natural ? E : n_selfsize;
    st->n_eligible = natural ? E : n_selfsize - n_remove;
    st->n_pruned = n_remove;
    st->n_active = 0;
    st->n_active_nonresident = 0;
    st->n_natural_union = s_nnat;
    st->err_flags = s_err;
    st->r_eff = r_eff;
    st->demand_total = tot;
  }
}

// one wave per node, 16 nodes per work-group
__global__ __launch_bounds__(1024) void restricted_kernel(SelectArgs a) {
  const int lane = lane_id();
  const int i = blockIdx.x * 16 + static_cast<int>(threadIdx.x >> 6);
  if (i < a.N) {
    const int E = a.E, k = a.k;
    const float* row = a.logits + static_cast<size_t>(i) * E;
    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + kWave * q;
      key[q] = (e < E && a.eligible[e]) ? topk_key(row[e], e) : 0ull;
    }
    int my_sel = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t b = key[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) b = key[q] > b ? key[q] : b;
      b = wave_max_u64(b);
      const int ew = b ? key_expert(b) : 0;
      if ((ew & (kWave - 1)) == lane) {
        const int q = ew >> 6;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (qq == q) key[qq] = 0ull;
      }
      if (lane == j) my_sel = ew;
    }
    const double m = static_cast<double>(a.node_m[i]);
    const double z = a.node_z[i];
    double p = 0.0;
    if (lane < k) p = exp(static_cast<double>(row[my_sel]) - m) / z;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += __shfl(p, j, kWave);
    if (lane < k) {
      const double g = (a.flags & kFlagNoRenorm) ? p : p / s;
      a.topk_idx[static_cast<size_t>(i) * k + lane] = my_sel;
      a.topk_gate[static_cast<size_t>(i) * k + lane] = static_cast<float>(g);
    }
  }
  if (a.counts) {
    if (last_block_done(&a.counters[1], gridDim.x))
      permute_block(a.N, a.k, a.E, a.topk_idx, a.counts, a.offsets, a.sorted_assign, a.inv_pos,
                    a.active, a.n_active, a.resident, static_cast<StatsDev*>(a.stats));
  }
}

}  // namespace

void select_plan(int N, int H, int E, int /*num_cu*/, int* ksplit, int* kslice) {
  const int tiles = ((E + kRT - 1) / kRT) * ((N + kRT - 1) / kRT);
  int ks = 512 / tiles;
  if (ks < 1) ks = 1;
  if (ks > H / 64) ks = H / 64;
  int sl = (H + ks - 1) / ks;
  sl = (sl + 63) / 64 * 64;
  *kslice = sl;
  *ksplit = (H + sl - 1) / sl;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  // with given logits the router only resets the arrival counter
  const bool lin = (a.flags & kFlagLogitsIn) != 0;
  const dim3 grid = lin ? dim3(1, 1, 1) : dim3((a.E + kRT - 1) / kRT, (a.N + kRT - 1) / kRT, a.ksplit);
  if (a.act_bf16)
    router_partial_kernel<uint16_t><<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.w_router), a.N, a.E,
        a.H, a.kslice, a.part, a.counters, !lin);
  else
    router_partial_kernel<float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(a.x), static_cast<const float*>(a.w_router), a.N, a.E, a.H,
        a.kslice, a.part, a.counters, !lin);
  const int nb = (a.N + 15) / 16;
  node_kernel<<<nb, 1024, 0, stream>>>(a);
  restricted_kernel<<<nb, 1024, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace amoe
