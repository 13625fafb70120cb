// AcceptMoE expert selection on gfx950: router product, per-node softmax and
// natural top-k, commitment-weighted demand, anchor, self-sizing,
// residency-aware pruning, restricted top-k, gates and the grouping of the
// assignments by expert.
//
// Sources: [MoE-SD blog, MoE layer] for the router (softmax over all experts,
// top-k routing) and the grouping; [AcceptMoE news §02] and [AcceptMoE
// abstract] for demand, root anchor, self-sizing by effective rank and
// residency-aware pruning; [AcceptMoE abstract] for restricting top-k to the
// eligible set.
//
// front_kernel (wave64, 256 threads) over a grid of (node groups of 4) x
// (K slices of the router product):
//   router   each work-group: the 4 nodes' partial logits over its K slice for
//            all experts on MFMA (16x16x32 bf16; fp32 inputs as eight
//            16x16x4 steps), rows 0..3 of each 16x16 tile being the nodes.
//            The partials are stored and read back at device scope, so the
//            hand-over to the group's last work-group needs no cache
//            write-back or invalidation (whole-L2 operations).
//   node     the last K-slice work-group of a group to finish: one wave per
//            node sums the slice partials (+ bias), takes fp64 softmax
//            statistics and the natural top-k (k rounds of a wave max over
//            32-bit order keys, ties to the lower index), and adds the demand
//            terms c[depth] * p of the node's top-k into one partial row per
//            group (stored expert-major).
// tail_kernel (one work-group of 1024 threads): demand per expert (group
// partials summed in group order), entropy, set size, anchor + fill and
// pruning by rank counting; then (N <= kFusedMaxN) every node's restricted
// top-k, the gates and the grouping by expert.  A node whose natural top-k
// lies inside the set keeps it (the k largest keys of all experts are the k
// largest of any superset of them); the others rank their set members' keys
// by counting.
// For N > kFusedMaxN a third kernel (restricted_kernel, one wave per node)
// takes the restricted top-k and gates, and a fourth (group_kernel, one
// work-group of 1024 threads) groups the assignments.
// Every reduction has a fixed order: two runs give identical bits.  Arrival
// counters are left at zero by the last arriver, so a zero-filled workspace
// stays valid across calls.

#include "amoe_common.h"
#include "amoe_launch.h"

#include <type_traits>
#include "amoe_permute.h"

namespace amoe {

namespace {

constexpr int kMaxKSplit = 16;   // router K slices (partial sums per logit)
constexpr int kNodesPerWG = 4;   // nodes per group up to kFusedMaxN nodes (one wave each)
constexpr int kNodesPerWGBig = 16;  // nodes per group above (all 16 MFMA rows, 4 per wave)
constexpr int kMaxSlice = 2048;  // K elements per router slice
constexpr int kFusedMaxN = 256;  // largest N whose restricted top-k runs in the tail
constexpr int kKeyCap = 4096;    // (node, member) keys per rank-counting pass
constexpr int kLgCap = 8192;     // logits the tail holds in LDS (N * E up to this)
constexpr int kTail = 1024;      // threads of the tail kernel (one work-group)
constexpr int kRankCountMax = 64;  // largest (padded) set whose restricted top-k counts ranks

// nodes per group of the front kernel: 4 for blocks up to 128 nodes (64 for
// layers of more than 128 experts), 16 above (a quarter of the router weight
// re-reads and of the demand rows the tail sums; 8 waves, two nodes each in
// the node phase).  Measured: DeepSeek-V3.1-shaped block (256 nodes, 256
// experts) front + tail 111 -> 90 us; 128-expert layers at 256 nodes 216.5 ->
// 213.3 us, at 128 nodes equal, at 64 nodes 4-node groups are faster
// (135.7 -> 141.8 us).
__host__ __device__ __forceinline__ int nodes_per_group(int N, int E) {
  return (N > 128 || (N > 64 && E > 128)) ? kNodesPerWGBig : kNodesPerWG;
}
// demand / flag partial rows are stored expert-major, one row of group
// partials per expert, padded so that a row starts 16-byte aligned
// waves of a front work-group: one per node of a 4-node group; 8 for a
// 16-node group (2 nodes each in the node phase, 1 or 2 expert tiles each in
// the router product)
template <int NPW>
constexpr int front_waves() { return NPW > kNodesPerWG ? 8 : 4; }
__host__ __device__ __forceinline__ int node_groups(int N, int E) {
  return (N + nodes_per_group(N, E) - 1) / nodes_per_group(N, E);
}
__host__ __device__ __forceinline__ int dpart_stride(int N, int E) { return (node_groups(N, E) + 1) & ~1; }
__host__ __device__ __forceinline__ int fpart_stride(int N, int E) { return (node_groups(N, E) + 15) & ~15; }

// MFMA operand fragment: 8 consecutive K elements of one row (x or W_r).
// v_mfma_f32_16x16x32_bf16: A[m][kk] in lane m + 16g for kk in [8g, 8g+8),
// B[kk][n] likewise in lane n + 16g, D[m][n] in lane n + 16g for m in
// [4g, 4g+4).  fp32 inputs take eight v_mfma_f32_16x16x4_f32, MFMA i over the
// elements 8g + i of each lane: together the same 16x16x32 product.
template <typename AT>
struct RFrag;
template <>
struct RFrag<uint16_t> {
  bf16x8_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const bf16x8_t*>(p); }
  __device__ __forceinline__ void zero() { v = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u}); }
};
template <>
struct RFrag<float> {
  f32x4_t lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const f32x4_t*>(p);
    hi = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ void zero() {
    lo = f32x4_t{0.f, 0.f, 0.f, 0.f};
    hi = lo;
  }
};
__device__ __forceinline__ f32x4_t rmma(const RFrag<uint16_t>& a, const RFrag<uint16_t>& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t rmma(const RFrag<float>& a, const RFrag<float>& b, f32x4_t c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[i], b.lo[i], c, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[i], b.hi[i], c, 0, 0, 0);
  return c;
}
// K steps (32 wide) whose loads are issued together (a 256-long slice at
// once for bf16): up to 128 VGPRs of W_r
template <typename AT>
struct RouterSteps {
  static constexpr int n = sizeof(AT) == 2 ? 8 : 4;
};

// ------------------------------------------------------------------ LDS ----
template <int NPW>
struct NodeSmem {
  double c[NPW][kMaxE];  // demand terms per node
  float lg[NPW > kNodesPerWG ? NPW : 1][kMaxE];  // logits, when one work-group takes all of K
  int flags[kMaxE];      // bit 0: a root routes here, bit 1: some node does
  int err;
};
struct SetSmem {
  double d[kMaxE];
  double dl[kMaxE];  // d ln d (0 for d = 0)
  double key[kMaxE];
  int anchor[kMaxE], rank[kMaxE], elig[kMaxE];
  int part[kTail];  // split_rank partial counts
  int err, na, nnat, nsel, ncand, take;
  double tot, r_eff;
};
struct TailSmem {
  SetSmem set;
  int member[kMaxE];  // eligible experts, ascending
  int nmem;
  int needy[kFusedMaxN];  // nodes whose natural top-k leaves the set
  int nneedy;
  int bad[kFusedMaxN];  // 1: the node's natural top-k leaves the set
  float m[kFusedMaxN];
  double z[kFusedMaxN];
  float lg[kLgCap];                 // [node][expert] logits when N * E <= kLgCap
  int top_e[kFusedMaxN * kMaxK];    // [node][slot] expert
  float top_l[kFusedMaxN * kMaxK];  // [node][slot] logit
  union {
    uint64_t keys[kKeyCap];           // rank counting
    double p[kFusedMaxN * kMaxK];     // gate numerators
    PermuteSmem<kTail> perm;
  } u;
};

// 32-bit order key of a logit: unsigned order = float order (-0 folded onto
// +0), at least 1 so that 0 can mark an empty slot.  The 64-bit topk_key is
// this key (unclamped) over ~index.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return o > 1u ? o : 1u;
}
// an order key (or the high word of a topk_key) back to its logit
__device__ __forceinline__ float order_logit(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  return order_logit(static_cast<uint32_t>(key >> 32));
}

// ---------------------------------------------------------- node phase ----
// Node i on one wave: logits from the K-slice partials (+ bias), from the
// work-group's own product in LDS (lrow, when one work-group took all of K)
// or from logits_in, fp64 softmax statistics, natural top-k (written in slot
// order), demand terms into sm.c[slot], anchor / natural-use flags, error
// bits.  d, p, dp, cf: depth, parent, parent's depth and commit[depth] of
// node i.
// KSM: K-slice partials loaded per logit (a bound on ksplit: 8 or kMaxKSplit)
template <int Q, int NPW, int KSM>
__device__ __forceinline__ void node_phase(const SelectArgs& a, int i, int slot,
                                           NodeSmem<NPW>& sm, int d, int p, int dp, float cf,
                                           const float* bias, const float* lrow) {
  const int lane = lane_id();
  const int E = a.E, k = a.k;
  const bool logits_in = (a.flags & kFlagLogitsIn) != 0;
  float l[Q];
  bool valid[Q];
  bool nonfinite = false;
  if (logits_in) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      valid[q] = e < E;
      l[q] = valid[q] ? a.logits_in[static_cast<size_t>(i) * E + e] : 0.f;
    }
  } else if (lrow) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      valid[q] = e < E;
      l[q] = valid[q] ? lrow[e] + bias[q] : 0.f;
    }
  } else {
    // K-slice partial sums: every load issued first, then summed in slice
    // order.  The loads are unconditional, from clamped addresses (slices
    // past ksplit read the last one again, lanes past E the last expert;
    // neither is summed): guarded loads cost a branch each and kept them
    // from going out together (node phase of 16-node groups 37.0 -> 32.4 us
    // for the front kernel of the DeepSeek-V3.1-shaped block).
    const size_t stride = static_cast<size_t>(a.N) * E;
    const int ksl = a.ksplit - 1;
    float pv[Q][KSM];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      valid[q] = e < E;
      const float* pp = a.part + static_cast<size_t>(i) * E + min(e, E - 1);
#pragma unroll
      for (int s = 0; s < KSM; ++s) pv[q][s] = load_dev(pp + min(s, ksl) * stride);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      float sum = 0.f;
#pragma unroll
      for (int s = 0; s < KSM; ++s)
        if (valid[q] && s < a.ksplit) sum += pv[q][s];
      l[q] = valid[q] ? sum + bias[q] : 0.f;
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (valid[q]) {
      const int e = lane + kWave * q;
      a.logits[static_cast<size_t>(i) * E + e] = l[q];
      if (a.logits_out) a.logits_out[static_cast<size_t>(i) * E + e] = l[q];
      if (!isfinite(l[q])) nonfinite = true;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (valid[q]) m = fmaxf(m, l[q]);
  m = wave_max_f32(m);
  double zs = 0.0;
  double ex[Q];  // exp(l - m), kept for the demand terms
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    ex[q] = valid[q] ? exp(static_cast<double>(l[q]) - static_cast<double>(m)) : 0.0;
    if (valid[q]) zs += ex[q];
  }
  const double z = wave_sum_f64(zs);

  // natural top-k: k rounds of a wave max over 32-bit order keys; among equal
  // keys the lowest expert index (slot q, then lane) wins
  uint32_t key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) key[q] = valid[q] ? order_key(l[q]) : 0u;
  uint32_t in_nat = 0;  // bit q: slot q is in the natural top-k
  int my_e = 0;         // lane j: expert of rank j
  uint32_t my_o = 0;    //         and its key
  for (int j = 0; j < k; ++j) {
    uint32_t b = key[0];
#pragma unroll
    for (int q = 1; q < Q; ++q) b = key[q] > b ? key[q] : b;
    b = wave_max_u32(b);
    // the lowest slot q holding the maximum, then its lowest lane
    int qw = Q - 1;
    uint64_t mw = __ballot(key[Q - 1] == b);
#pragma unroll
    for (int q = Q - 2; q >= 0; --q) {
      const uint64_t mq = __ballot(key[q] == b);
      if (mq) {
        qw = q;
        mw = mq;
      }
    }
    const int lw = static_cast<int>(__builtin_ctzll(mw));
    if (lane == lw) {
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (q == qw) {
          key[q] = 0u;
          in_nat |= 1u << q;
        }
    }
    if (lane == j) {
      my_e = kWave * qw + lw;
      my_o = b;
    }
  }
  if (lane < k) {
    a.nat_idx[static_cast<size_t>(i) * k + lane] = my_e;
    a.nat_logit[static_cast<size_t>(i) * k + lane] = order_logit(my_o);
  }
  // demand terms: the node's weight times its score of every natural top-k
  // expert (of every expert under kFlagDemandFull); the weight is the
  // commitment probability of its depth (1 under kFlagUnitCommit).  Flag bit
  // 1: natural top-k (for the union statistic); bit 0: anchor (a root's
  // natural top-k, unless kFlagNoAnchor).
  const bool full = (a.flags & kFlagDemandFull) != 0;
  const double c = (a.flags & kFlagUnitCommit) ? 1.0 : static_cast<double>(cf);
  const int fl = (p == -1 && !(a.flags & kFlagNoAnchor)) ? 3 : 2;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const bool nat_q = (in_nat & (1u << q)) != 0;
    const int e = lane + kWave * q;
    if (full ? valid[q] : nat_q)
      sm.c[slot][e] = c * (ex[q] / z);
    if (nat_q) atomicOr(&sm.flags[e], fl);
  }
  const bool any_nf = __ballot(nonfinite) != 0ull;
  if (lane == 0) {
    int err = any_nf ? kErrNonFinite : 0;
    if (d < 0 || d >= a.n_depth) err |= kErrDepth;
    if (p == -1) {
      if (d != 0) err |= kErrBadTree;
    } else if (p < 0 || p >= i) {
      err |= kErrBadTree;
    } else if (d != dp + 1) {
      err |= kErrBadTree;
    }
    if (err) atomicOr(&sm.err, err);
    a.node_m[i] = m;
    a.node_z[i] = z;
  }
}

// ------------------------------------------------------- set selection ----
// Every arrival counter of the workspace must be zero between kernels of a
// call: the front kernel's elections leave its group counters at zero and
// note any count outside its range in counters[0].  A nonzero counter here
// means the workspace was not zero-filled before its first use, or was
// shared by calls that overlap: the call's outputs are then flagged
// (kErrWorkspace), and the counters are set back to zero so that later
// calls elect correctly (counters[1] counts the grouping's arrivals for
// N > kFusedMaxN, after this kernel).  The tail
// kernel's threads load the nwg + 2 counters (counters[0..1], then the node
// groups' gcount) with the kernel's other first loads; select_set checks and
// repairs them.
struct CounterCheck {
  int* ptr[2];  // this thread's counters (at most two), or null
  int val[2];
};
__device__ __forceinline__ CounterCheck load_counters(const SelectArgs& a, int nwg) {
  CounterCheck c;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int g = static_cast<int>(threadIdx.x) + r * kTail;
    c.ptr[r] = nullptr;
    c.val[r] = 0;
    if (g < nwg + 2) {
      c.ptr[r] = g < 2 ? &a.counters[g] : &a.gcount[g - 2];
      c.val[r] = __hip_atomic_load(c.ptr[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return c;
}

// Rank of expert t among the experts by counting over key[0..EP), where key
// holds the demand of the experts that take part and a sentinel for the rest
// (below or above every demand, so it never counts).  desc: order (key desc,
// index asc); else (key asc, index desc).  The E x EP comparisons are split
// over the kTail threads: thread (e, part) counts over one part of the keys
// and the parts are added in LDS.  Call with the whole work-group; returns
// the rank in threads t < E with take[t] set.
// The caller must pass a work-group barrier before it writes key or scratch
// again.
__device__ __forceinline__ int split_rank(const double* key, int* scratch, int E, bool desc,
                                          const int* take) {
  const int t = threadIdx.x;
  const int EP = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
  const int tpe = kTail / EP, e = t % EP, part = t / EP;
  const int span = EP / tpe;  // a multiple of 4
  int r = 0;
  if (e < E && take[e]) {
    const double de = key[e];
    const int f0 = part * span;
    for (int f = f0; f < f0 + span; f += 4) {
      // four keys read first, then compared without branches
      double df[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) df[u] = key[f + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int strict = desc ? (df[u] > de) : (df[u] < de);
        const int tie = (df[u] == de) & (desc ? (f + u < e) : (f + u > e));
        r += strict | tie;
      }
    }
  }
  scratch[part * EP + e] = r;
  __syncthreads();
  int rank = 0;
  if (t < E)
    for (int pp = 0; pp < tpe; ++pp) rank += scratch[pp * EP + t];
  // no barrier here: both callers pass a barrier before scratch or key is
  // written again
  return rank;
}

// One kTail-thread work-group.  nwg partial rows (per expert, expert-major)
// of demand / flags, nwg error words; cc: this thread's arrival counter as
// loaded at the start of the kernel (checked and set back to zero here).  Leaves the eligible flags in
// sm.elig (and in a.eligible), statistics in a.stats (n_active and
// n_active_nonresident follow once the restricted top-k is known).
__device__ void select_set(const SelectArgs& a, int nwg, SetSmem& sm, CounterCheck cc) {
  static_assert(kMaxE == 256 && kTail >= kMaxE, "select_set keeps one thread per expert slot");
  const int t = threadIdx.x;
  const int E = a.E, k = a.k;
  const bool natural = (a.flags & kFlagNatural) != 0;
  if (t == 0) {
    sm.err = 0;
    sm.na = 0;
    sm.nnat = 0;
    sm.nsel = 0;
    sm.ncand = 0;
  }
  // error words and the commit table, loaded together with the demand rows;
  // the loads go out before the barrier that publishes the counters above
  const int err0 = t < nwg ? a.e_part[t] : 0;
  const float com0 = t < a.n_depth ? a.commit[t] : 0.f;
  // demand per expert: its row of group partials summed in group order
  // (16-byte loads: two partials, sixteen flag bytes)
  int f = 0;
  double dsum = 0.0;
  if (t < E) {
    const int ds = dpart_stride(a.N, a.E), fs = fpart_stride(a.N, a.E);
    const double* drow = a.d_part + static_cast<size_t>(t) * ds;
    const uint8_t* frow = a.f_part + static_cast<size_t>(t) * fs;
    constexpr int B = 8;  // 16-byte loads in flight per batch: 16 partials
    // (unconditional loads from clamped addresses, as in the node phase:
    // pairs past the row read its last pair again and are not summed)
    const int wl = (nwg - 1) & ~1;
    for (int w0 = 0; w0 < nwg; w0 += 2 * B) {
      f64x2_t dv[B];
#pragma unroll
      for (int u = 0; u < B; ++u)
        dv[u] = *reinterpret_cast<const f64x2_t*>(drow + min(w0 + 2 * u, wl));
      const u32x4_t fv = *reinterpret_cast<const u32x4_t*>(frow + w0);
#pragma unroll
      for (int u = 0; u < B; ++u) {
        if (w0 + 2 * u < nwg) dsum += dv[u][0];
        if (w0 + 2 * u + 1 < nwg) dsum += dv[u][1];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (w0 + u < nwg) f |= static_cast<int>((fv[u >> 2] >> (8 * (u & 3))) & 0xffu);
    }
  }
  __syncthreads();
  if (t < E) {
    if (f & 1) atomicAdd(&sm.na, 1);
    if (f & 2) atomicAdd(&sm.nnat, 1);
  }
  if (t < kMaxE) {
    const bool in_fill = t < E && !(f & 1);  // experts that take part in the fill
    sm.d[t] = dsum;
    sm.dl[t] = dsum > 0.0 ? dsum * log(dsum) : 0.0;
    sm.anchor[t] = f & 1;
    // fill order: (demand desc, index asc) over the non-anchor experts;
    // anchors and padding carry demand -1, below every real demand
    sm.key[t] = in_fill ? dsum : -1.0;
    sm.elig[t] = in_fill;
  }
  if (err0) atomicOr(&sm.err, err0);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (cc.val[r] != 0) {
      atomicOr(&sm.err, kErrWorkspace);
      __hip_atomic_store(cc.ptr[r], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  for (int w = t + kTail; w < nwg; w += kTail) {
    const int e = a.e_part[w];
    if (e) atomicOr(&sm.err, e);
  }
  if (t < a.n_depth && (!(com0 >= 0.f) || isinf(com0))) atomicOr(&sm.err, kErrCommit);
  for (int dd = t + kTail; dd < a.n_depth; dd += kTail) {
    const float c = a.commit[dd];
    if (!(c >= 0.f) || isinf(c)) atomicOr(&sm.err, kErrCommit);
  }
  __syncthreads();
  if (t < kWave) {  // wave 0: total demand, entropy and the set size
    // H = -sum q ln q with q = d / tot equals ln tot - (sum d ln d) / tot;
    // each expert's d ln d was taken with its demand sum
    double sd = 0.0, sl = 0.0;
    for (int e = t; e < E; e += kWave) {
      sd += sm.d[e];
      sl += sm.dl[e];
    }
    const double tot = wave_sum_f64(sd);
    const double sdl = wave_sum_f64(sl);
    if (t == 0) {
      const double h = tot > 0.0 ? log(tot) - sdl / tot : 0.0;
      const double r_eff = tot > 0.0 ? exp(h) : 0.0;
      const int n_min = max(k, a.min_set);
      const int n_raw = a.fixed_budget > 0 ? a.fixed_budget : static_cast<int>(floor(r_eff + 0.5));
      const int n = min(E, max(max(n_raw, sm.na), n_min));
      sm.tot = tot;
      sm.r_eff = r_eff;
      sm.take = n - sm.na;
    }
  }
  // the fill ranks do not depend on the set size: counted while wave 0 sizes
  // the set (split_rank's barrier publishes both)
  const int fill_rank = split_rank(sm.key, sm.part, E, true, sm.elig);
  const double tot = sm.tot;
  const double r_eff = sm.r_eff;
  const int n_anchor = sm.na;
  const int n_min = max(k, a.min_set);
  const int take = sm.take;
  int el = 0;
  if (t < E) {
    el = natural ? 1 : (sm.anchor[t] || fill_rank < take) ? 1 : 0;
    if (el) atomicAdd(&sm.nsel, 1);
  }
  if (t < kMaxE) sm.elig[t] = el;
  __syncthreads();
  const int n_selfsize = sm.nsel;
  int n_remove = 0;
  if (!natural && a.resident) {
    const bool cand = t < E && sm.elig[t] && !sm.anchor[t] && !a.resident[t];
    if (cand) atomicAdd(&sm.ncand, 1);
    // pruning order among candidates: demand ascending, index descending;
    // non-candidates carry +infinity (never below a candidate's demand)
    if (t < kMaxE) {
      sm.key[t] = cand ? sm.d[t] : INFINITY;
      sm.anchor[t] = cand;  // the anchor flags are no longer needed: candidates
    }
    __syncthreads();
    n_remove = max(0, min(a.reroute_budget, min(n_selfsize - n_min, sm.ncand)));
    const int prune_rank = split_rank(sm.key, sm.part, E, false, sm.anchor);
    if (cand && prune_rank < n_remove) sm.elig[t] = 0;
    __syncthreads();
  }
  if (t < E) a.eligible[t] = static_cast<uint8_t>(sm.elig[t]);
  if (t == 0) {
    StatsDev* st = reinterpret_cast<StatsDev*>(a.stats);
    st->n_anchor = n_anchor;
    st->n_selfsize = natural ? E : n_selfsize;
    st->n_eligible = natural ? E : n_selfsize - n_remove;
    st->n_pruned = n_remove;
    st->n_active = 0;
    st->n_active_nonresident = 0;
    st->n_natural_union = sm.nnat;
    st->err_flags = sm.err;
    st->r_eff = r_eff;
    st->demand_total = tot;
  }
}

// U (unique experts of the restricted top-k) and how many of them are not
// resident, from the N*k chosen experts (LDS or global), by the whole
// work-group when no grouping follows; flag: kMaxE ints of scratch.  The
// grouping (permute_block) writes the same two statistics itself.
template <int NTHR>
__device__ __forceinline__ void active_stats(int NK, int E, const int32_t* sel,
                                             const uint8_t* resident, StatsDev* st, int* flag) {
  const int t = threadIdx.x;
  if (t < kMaxE) flag[t] = 0;
  __syncthreads();
  for (int x = t; x < NK; x += NTHR) flag[clamp_expert(sel[x], E)] = 1;
  __syncthreads();
  if (t < kWave) {
    int na = 0, nr = 0;
    for (int e = t; e < E; e += kWave) {
      na += flag[e];
      nr += (flag[e] && resident && !resident[e]) ? 1 : 0;
    }
    na = static_cast<int>(readlane_u32(wave_inclusive_sum_u32(static_cast<uint32_t>(na)), kWave - 1));
    nr = static_cast<int>(readlane_u32(wave_inclusive_sum_u32(static_cast<uint32_t>(nr)), kWave - 1));
    if (t == 0) {
      st->n_active = na;
      st->n_active_nonresident = nr;
    }
  }
}

// ------------------------------------------------- restricted top-k tail ----
// After select_set, by the same kTail-thread work-group, for N <= kFusedMaxN,
// with sm.top_e / top_l / m / z already holding the node phase's natural
// top-k and softmax statistics: every node's top-k over the eligible set, the
// gates, and (when a.counts is set) the grouping of the assignments by expert.
// lg_lds: sm.lg holds the logits (else they are read from a.logits).
// SPLIT: the grouping's split mode (a.split_rows >= 0) is on
template <bool SPLIT>
__device__ void restricted_tail(const SelectArgs& a, TailSmem& sm, bool lg_lds) {
  const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
  const int N = a.N, E = a.E, k = a.k;
  const int NK = N * k;
  for (int i = t; i < N; i += kTail) sm.bad[i] = 0;
  if (wave == 0) {  // eligible experts in ascending order
    const int nm = wave_exclusive_scan_256(sm.set.elig, sm.set.rank, kMaxE);
    if (lane == 0) {
      sm.nmem = nm;
      sm.nneedy = 0;
    }
  }
  __syncthreads();
  if (t < E && sm.set.elig[t]) sm.member[sm.set.rank[t]] = t;
  // nodes whose natural top-k leaves the set
  for (int x = t; x < NK; x += kTail)
    if (!sm.set.elig[sm.top_e[x]]) sm.bad[x / k] = 1;
  __syncthreads();
  for (int i = t; i < N; i += kTail)
    if (sm.bad[i]) sm.needy[atomicAdd(&sm.nneedy, 1)] = i;
  __syncthreads();
  const int nm = sm.nmem, nneedy = sm.nneedy;
  // Small sets: rank counting over (needy node, member) keys, rows padded to
  // a multiple of 4 with key 0 (below every key), as many nodes per pass as
  // fit.  Large sets (more than kRankCountMax members; the counting costs
  // members^2 per node): one wave per needy node keeps the node's natural
  // top-k members of the set and takes the remaining places by rounds of a
  // wave max over the set's other experts.  Both give each node's top-k keys
  // in key order (value, then lower index).
  const int nmp = (nm + 3) & ~3;
  if (nmp > kRankCountMax) {
    constexpr int NWV = kTail / kWave;
    // a node's logits (from memory when they do not fit in LDS) are loaded
    // one node ahead, so their latency hides behind the previous node's rounds
    float lv[4];
    auto load_logits = [&](int c, float (&v)[4]) {
      const int i = sm.needy[c < nneedy ? c : 0];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ec = min(lane + kWave * q, E - 1);
        v[q] = lg_lds ? sm.lg[i * E + ec] : a.logits[static_cast<size_t>(i) * E + ec];
      }
    };
    if (wave < nneedy) load_logits(wave, lv);
    for (int c = wave; c < nneedy; c += NWV) {
      const int i = sm.needy[c];
      float cur[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) cur[q] = lv[q];
      if (c + NWV < nneedy) load_logits(c + NWV, lv);
      // The node's natural top-k members of the set hold the set's largest
      // keys (the natural top-k are the largest of all experts), so they keep
      // their places, in order; only the k - kept places after them take
      // rounds of a wave max, over the set's other experts.
      int my_e = 0;
      float my_l = 0.f;
      if (lane < k) {
        my_e = sm.top_e[i * k + lane];
        my_l = sm.top_l[i * k + lane];
      }
      const bool keep = lane < k && sm.set.elig[my_e] != 0;
      const uint64_t km = __ballot(keep);
      const int kept = __popcll(km);
      uint64_t key[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + kWave * q;
        const int ec = e < E ? e : E - 1;
        key[q] = (e < E && sm.set.elig[ec]) ? topk_key(cur[q], ec) : 0ull;
      }
      for (int j = 0; j < k; ++j) {  // natural top-k experts are not candidates
        const int ej = __builtin_amdgcn_readlane(my_e, j);
        if ((ej & (kWave - 1)) == lane) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == (ej >> 6)) key[q] = 0ull;
        }
      }
      if (keep) {
        const int pos = __popcll(km & ((1ull << lane) - 1ull));
        sm.top_e[i * k + pos] = my_e;
        sm.top_l[i * k + pos] = my_l;
      }
      for (int j = kept; j < k; ++j) {
        uint64_t b = key[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) b = key[q] > b ? key[q] : b;
        b = wave_max_u64(b);
        const int ew = key_expert(b);
        if ((ew & (kWave - 1)) == lane) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == (ew >> 6)) key[q] = 0ull;
        }
        if (lane == 0 && b != 0ull) {
          sm.top_e[i * k + j] = ew;
          sm.top_l[i * k + j] = key_logit(b);
        }
      }
    }
    __syncthreads();
  }
  const int per = max(1, kKeyCap / max(nmp, 4));
  const float inv = 1.0f / static_cast<float>(max(nmp, 1));
  for (int c0 = 0; nmp <= kRankCountMax && c0 < nneedy; c0 += per) {
    const int cn = min(per, nneedy - c0);
    const int total = cn * nmp;
    for (int x = t; x < total; x += kTail) {
      int r = static_cast<int>(static_cast<float>(x) * inv);
      if (r * nmp > x) --r;
      if ((r + 1) * nmp <= x) ++r;
      const int mm = x - r * nmp;
      uint64_t key = 0ull;
      if (mm < nm) {
        const int i = sm.needy[c0 + r], e = sm.member[mm];
        const float v = lg_lds ? sm.lg[i * E + e] : a.logits[static_cast<size_t>(i) * E + e];
        key = topk_key(v, e);
      }
      sm.u.keys[x] = key;
    }
    __syncthreads();
    for (int x = t; x < total; x += kTail) {
      int r = static_cast<int>(static_cast<float>(x) * inv);
      if (r * nmp > x) --r;
      if ((r + 1) * nmp <= x) ++r;
      const uint64_t mine = sm.u.keys[x];
      const uint64_t* row = &sm.u.keys[r * nmp];
      int rank = 0;
      int f = 0;
      for (; f + 8 <= nmp; f += 8) {
        uint64_t rf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) rf[u] = row[f + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += static_cast<int>(rf[u] > mine);
      }
      if (f < nmp) {
        uint64_t rf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) rf[u] = row[f + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += static_cast<int>(rf[u] > mine);
      }
      if (mine != 0ull && rank < k) {
        const int i = sm.needy[c0 + r];
        sm.top_e[i * k + rank] = key_expert(mine);
        sm.top_l[i * k + rank] = key_logit(mine);
      }
    }
    __syncthreads();
  }
  // gates: fp64 softmax scores of the chosen experts, renormalised over the
  // node's k slots in slot order
  for (int x = t; x < NK; x += kTail) {
    const int i = x / k;
    sm.u.p[x] = exp(static_cast<double>(sm.top_l[x]) - static_cast<double>(sm.m[i])) / sm.z[i];
  }
  __syncthreads();
  const bool renorm = (a.flags & kFlagNoRenorm) == 0;
  for (int x = t; x < NK; x += kTail) {
    const int i = x / k;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += sm.u.p[i * k + j];
    const double g = renorm ? sm.u.p[x] / s : sm.u.p[x];
    a.topk_idx[x] = sm.top_e[x];
    a.topk_gate[x] = static_cast<float>(g);
  }
  __syncthreads();
  if (a.counts)
    permute_block<kTail>(N, k, E, sm.top_e, a.counts, a.offsets, a.sorted_assign, a.inv_pos,
                       a.active, a.n_active, a.resident, static_cast<StatsDev*>(a.stats),
                       sm.u.perm, a.max_rows, a.groups, a.active_w, a.group_shift,
                       SPLIT ? a.split_rows : -1, SPLIT ? a.n_work : nullptr);
  else
    active_stats<kTail>(NK, E, sm.top_e, a.resident, static_cast<StatsDev*>(a.stats),
                        sm.set.rank);
}

// commit[depth] and the parent's depth of node `node` (of any wave: clamped
// addresses, no branches; dp is 0 when p is not an earlier node)
__device__ __forceinline__ void node_deps(const SelectArgs& a, int node, int d, int p, float& cf,
                                          int& dp) {
  const int dc = d < 0 ? 0 : (d >= a.n_depth ? a.n_depth - 1 : d);
  const bool pin = p >= 0 && p < node;
  cf = a.commit[dc];
  const int pd = a.depth[pin ? p : 0];
  dp = pin ? pd : 0;
}

// ------------------------------------------------------------ router ----
// Partial logits of group g's 4 nodes over K slice ks, for all experts, into
// a.part[ks][node][expert].  Wave w takes the 16-expert tiles w, w + 4, ...
// (TPW of them); MFMA rows 0..3 are the nodes (rows 4..15 are zeros), columns
// the tile's experts; rows 4..15 repeat rows 0..3 and are discarded.  Every
// load is issued unconditionally from a clamped address (rows past E or N
// repeat the last one and are discarded), so that all of them are in flight
// together.  The node's dependent inputs (commit of
// its depth, its parent's depth) are loaded once the product's loads are
// out, so that they share the round trip.
template <typename AT, int TPW, int NPW>
__device__ __forceinline__ void router_partials(const SelectArgs& a, int g, int ks, int wave,
                                                int lane, int node, int d, int p, float& cf,
                                                int& dp, float (*lds)[kMaxE]) {
  constexpr int S = RouterSteps<AT>::n;
  const int N = a.N, E = a.E, H = a.H;
  const int n0 = g * NPW;
  const int kbeg = ks * a.kslice;
  const int nsteps = min(H - kbeg, a.kslice) >> 5;
  const int mrow = lane & 15, kq = (lane >> 4) * 8;
  // NPW = 4: MFMA rows 4..15 repeat rows 0..3 (their D rows are never
  // stored); NPW = 16: every row is a node
  const AT* xrow = static_cast<const AT*>(a.x) +
                   static_cast<size_t>(min(n0 + (mrow & (NPW - 1)), N - 1)) * H + kbeg + kq;
  const AT* wrow[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int e = min((wave + front_waves<NPW>() * tt) * 16 + mrow, E - 1);
    wrow[tt] = static_cast<const AT*>(a.w_router) + static_cast<size_t>(e) * H + kbeg + kq;
  }
  f32x4_t acc[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (NPW > kNodesPerWG && nsteps > S) {
    // 16-node groups (8 waves, long K slices): two batches of S steps in
    // flight, the loads of batch b + 1 issued before batch b's MFMAs.  Loads
    // past the slice inside a batch read its last step again (never used),
    // so the memory counter waits only for the batch it needs.
    RFrag<AT> bf[2][TPW][S];
    RFrag<AT> af[2][S];
    auto load_batch = [&](auto bc, int s0) {
      constexpr int b = decltype(bc)::value;
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int s = 0; s < S; ++s) bf[b][tt][s].load(wrow[tt] + 32 * min(s0 + s, nsteps - 1));
#pragma unroll
      for (int s = 0; s < S; ++s) af[b][s].load(xrow + 32 * min(s0 + s, nsteps - 1));
    };
    auto compute_batch = [&](auto bc, int s0) {
      constexpr int b = decltype(bc)::value;
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (s0 + s < nsteps) {
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) acc[tt] = rmma(af[b][s], bf[b][tt][s], acc[tt]);
        }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    load_batch(B0{}, 0);
    int s0 = 0;
    for (; s0 + 2 * S < nsteps; s0 += 2 * S) {
      load_batch(B1{}, s0 + S);
      compute_batch(B0{}, s0);
      load_batch(B0{}, s0 + 2 * S);
      compute_batch(B1{}, s0 + S);
    }
    // the last one or two batches, without loads past them
    if (s0 + S < nsteps) {
      load_batch(B1{}, s0 + S);
      compute_batch(B0{}, s0);
      compute_batch(B1{}, s0 + S);
    } else {
      compute_batch(B0{}, s0);
    }
  } else
  for (int s0 = 0; s0 < nsteps; s0 += S) {
    RFrag<AT> bf[TPW][S];
    RFrag<AT> af[S];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int s = 0; s < S; ++s) bf[tt][s].load(wrow[tt] + 32 * min(s0 + s, nsteps - 1));
#pragma unroll
    for (int s = 0; s < S; ++s) af[s].load(xrow + 32 * min(s0 + s, nsteps - 1));
    if (NPW == kNodesPerWG && s0 == 0) {
      asm volatile("" ::: "memory");
      node_deps(a, node, d, p, cf, dp);
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s0 + s < nsteps) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) acc[tt] = rmma(af[s], bf[tt][s], acc[tt]);
      }
  }
  // D rows 4gq..4gq+3 sit in lanes 16gq..16gq+15, one expert column each
  // (NPW = 4: only rows 0..3, lanes 0..15, are nodes); into LDS when this
  // work-group takes all of K, else to the partials at device scope
  const int gq = lane >> 4;
  if (NPW > kNodesPerWG || gq == 0) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int e = (wave + front_waves<NPW>() * tt) * 16 + (lane & 15);
      if (e < E) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * gq + j;
          if (lds)
            lds[r][e] = acc[tt][j];
          else if (n0 + r < N)
            store_dev(a.part + (static_cast<size_t>(ks) * N + n0 + r) * E + e, acc[tt][j]);
        }
      }
    }
  }
}

// ------------------------------------------------------------- kernel ----
// Q: 64-expert slots per lane, ceil(E / 64); NPW nodes per group (wave w of
// NW takes nodes n0 + w, n0 + w + NW, ... in the node phase)
template <typename AT, int Q, int NPW, int KSM>
__global__ __launch_bounds__(64 * front_waves<NPW>()) void front_kernel(SelectArgs a) {
  constexpr int NW = front_waves<NPW>();
  constexpr int NTHR = 64 * NW;
  constexpr int PER_WAVE = NPW / NW;
  __shared__ NodeSmem<NPW> sm;
  const int t = threadIdx.x, wave = t >> 6, lane = lane_id();
  const int g = blockIdx.x, ks = blockIdx.y;
  const int N = a.N, E = a.E;
  const int n0 = g * NPW;
  const bool logits_in = (a.flags & kFlagLogitsIn) != 0;
  // one work-group takes all of K (NPW > 4 only): the logits stay in LDS
  const bool whole_k = NPW > kNodesPerWG && gridDim.y == 1;

  // node-phase inputs that do not depend on the logits, loaded up front (from
  // clamped addresses, without branches) so that their latency hides under
  // the router phase; the dependent ones follow once the product's loads are
  // out
  int d[PER_WAVE], p[PER_WAVE], dp[PER_WAVE];
  float cf[PER_WAVE];
#pragma unroll
  for (int s = 0; s < PER_WAVE; ++s) {
    const int nd = min(n0 + wave + NW * s, N - 1);
    d[s] = a.depth[nd];
    p[s] = a.parent[nd];
  }
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.b_router) {
#pragma unroll
    for (int q = 0; q < Q; ++q) bias[q] = a.b_router[min(lane + kWave * q, E - 1)];
  }
  if (!logits_in) {
    // ---- partial logits of the group's nodes over K slice ks
    const int tpw = ((E + 15) / 16 + NW - 1) / NW;  // 16-expert tiles per wave
    float (*lds)[kMaxE] = whole_k ? sm.lg : nullptr;
    const int node = n0 + wave;
    // (8 waves: at most 2 tiles each for kMaxE experts)
    static_assert(kMaxE <= 16 * 2 * 8, "8-wave router groups take at most 2 tiles a wave");
    if (tpw == 1)
      router_partials<AT, 1, NPW>(a, g, ks, wave, lane, node, d[0], p[0], cf[0], dp[0], lds);
    else if (NW == 8 || tpw == 2)
      router_partials<AT, 2, NPW>(a, g, ks, wave, lane, node, d[0], p[0], cf[0], dp[0], lds);
    else if constexpr (NW == 4) {
      if (tpw == 3)
        router_partials<AT, 3, NPW>(a, g, ks, wave, lane, node, d[0], p[0], cf[0], dp[0], lds);
      else
        router_partials<AT, 4, NPW>(a, g, ks, wave, lane, node, d[0], p[0], cf[0], dp[0], lds);
    }
    // partials travel at device scope: no cache write-back or invalidation
    if (!whole_k && !last_arrival_dev(&a.gcount[g], gridDim.y, &a.counters[0])) return;
  }
  if (logits_in || NPW > kNodesPerWG) {
#pragma unroll
    for (int s = 0; s < PER_WAVE; ++s) node_deps(a, n0 + wave + NW * s, d[s], p[s], cf[s], dp[s]);
  }

  // ---- node phase (the group's last K-slice work-group)
  for (int x = t; x < kMaxE; x += NTHR) {
    sm.flags[x] = 0;
#pragma unroll
    for (int w = 0; w < NPW; ++w) sm.c[w][x] = 0.0;
  }
  if (t == 0) sm.err = 0;
  __syncthreads();
#pragma unroll
  for (int s = 0; s < PER_WAVE; ++s) {
    const int slot = wave + NW * s;
    if (n0 + slot < N)
      node_phase<Q, NPW, KSM>(a, n0 + slot, slot, sm, d[s], p[s], dp[s], cf[s], bias,
                         whole_k && !logits_in ? sm.lg[slot] : nullptr);
  }
  __syncthreads();
  const int ds = dpart_stride(N, E), fs = fpart_stride(N, E);
  for (int x = t; x < E; x += NTHR) {
    double dsum = 0.0;
#pragma unroll
    for (int w = 0; w < NPW; ++w) dsum += sm.c[w][x];  // node order
    a.d_part[static_cast<size_t>(x) * ds + g] = dsum;
    a.f_part[static_cast<size_t>(x) * fs + g] = static_cast<uint8_t>(sm.flags[x]);
  }
  if (t == 0) a.e_part[g] = sm.err;
}

// The set selection and, for N <= kFusedMaxN, every node's restricted top-k,
// the gates and the grouping: one work-group of kTail threads, after the
// front kernel.  The node phase's outputs are loaded first, all together.
template <bool SPLIT>
__global__ __launch_bounds__(kTail) void tail_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) TailSmem sm;
  const int t = threadIdx.x;
  const int N = a.N, E = a.E;
  const int nwg = node_groups(N, E);
  const bool fused = N <= kFusedMaxN;
  const CounterCheck cc = load_counters(a, nwg);
  if (!fused) {
    select_set(a, nwg, sm.set, cc);
    return;
  }
  // natural top-k, its logits, max / sum of exp per node, and (when they
  // fit) all logits, in 16-byte loads issued before the demand rows
  const int NK = N * a.k;
  const int NE = N * E;
  const bool lg_lds = NE <= kLgCap;
  constexpr int RL = kLgCap / kTail;  // 8 logits per thread
  const int x4 = 4 * t;               // 4 top-k slots per thread (NK <= 4096)
  u32x4_t pe, pl;
  f32x4_t plg[RL / 4];
  if (x4 < NK) {
    pe = *reinterpret_cast<const u32x4_t*>(a.nat_idx + x4);
    pl = *reinterpret_cast<const u32x4_t*>(a.nat_logit + x4);
  }
  if (lg_lds) {
#pragma unroll
    for (int r = 0; r < RL / 4; ++r) {
      const int x = (t * (RL / 4) + r) * 4;
      if (x < NE) plg[r] = *reinterpret_cast<const f32x4_t*>(a.logits + x);
    }
  }
  float pm = 0.f;
  double pz = 1.0;
  if (t < N) {
    pm = a.node_m[t];
    pz = a.node_z[t];
  }
  select_set(a, nwg, sm.set, cc);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (x4 + j < NK) {
      sm.top_e[x4 + j] = clamp_expert(static_cast<int>(pe[j]), E);
      sm.top_l[x4 + j] = __uint_as_float(pl[j]);
    }
  }
  if (t < N) {
    sm.m[t] = pm;
    sm.z[t] = pz;
  }
  if (lg_lds) {
#pragma unroll
    for (int r = 0; r < RL / 4; ++r) {
      const int x = (t * (RL / 4) + r) * 4;
      if (x < NE) *reinterpret_cast<f32x4_t*>(&sm.lg[x]) = plg[r];
    }
  }
  __syncthreads();
  restricted_tail<SPLIT>(a, sm, lg_lds);
}

// one wave per node, 4 nodes per work-group (N > kFusedMaxN)
__global__ __launch_bounds__(256) void restricted_kernel(SelectArgs a) {
  const int lane = lane_id();
  const int i = blockIdx.x * kNodesPerWG + static_cast<int>(threadIdx.x >> 6);
  if (i < a.N) {
    const int E = a.E, k = a.k;
    const float* row = a.logits + static_cast<size_t>(i) * E;
    // the node's natural top-k members of the set keep their places, in
    // order (they hold the set's largest keys); the remaining places take
    // rounds of a wave max over the set's other experts
    int nat_e = 0;
    if (lane < k) nat_e = clamp_expert(a.nat_idx[static_cast<size_t>(i) * k + lane], E);
    const bool keep = lane < k && a.eligible[nat_e] != 0;
    const uint64_t km = __ballot(keep);
    const int kept = __popcll(km);
    int my_sel = 0;
    for (int j = 0, pos = 0; j < k; ++j) {  // slot pos < kept: the pos-th kept natural expert
      if ((km >> j) & 1ull) {
        const int ej = __builtin_amdgcn_readlane(nat_e, j);
        if (lane == pos) my_sel = ej;
        ++pos;
      }
    }
    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + kWave * q;
      key[q] = (e < E && a.eligible[e]) ? topk_key(row[e], e) : 0ull;
    }
    for (int j = 0; j < k; ++j) {  // natural top-k experts are not candidates
      const int ej = __builtin_amdgcn_readlane(nat_e, j);
      if ((ej & (kWave - 1)) == lane) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q == (ej >> 6)) key[q] = 0ull;
      }
    }
    for (int j = kept; j < k; ++j) {
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
    for (int j = 0; j < k; ++j) s += readlane_f64(p, j);  // slot order
    if (lane < k) {
      const double g = (a.flags & kFlagNoRenorm) ? p : p / s;
      a.topk_idx[static_cast<size_t>(i) * k + lane] = my_sel;
      a.topk_gate[static_cast<size_t>(i) * k + lane] = static_cast<float>(g);
    }
  }
}

// After restricted_kernel (N > kFusedMaxN), without the grouping: one
// work-group counts the active experts for the statistics.
__global__ __launch_bounds__(kTail) void group_kernel(SelectArgs a) {
  __shared__ PermuteSmem<kTail> perm;
  active_stats<kTail>(a.N * a.k, a.E, a.topk_idx, a.resident, static_cast<StatsDev*>(a.stats),
                      perm.cnt);
}

// After restricted_kernel (N > kFusedMaxN), with the grouping: the N*k
// assignments in chunks of kGroupChunk, one work-group each.  Pass 1
// (group_count_kernel): each chunk's expert counts go to ghist; the last
// chunk to finish (elected on counters[1]) replaces them by each chunk's
// first rank per expert (the counts of the chunks before it), and builds the
// tables from the totals.  Pass 2 (group_scatter_kernel): each chunk places
// its assignments from those ranks on.  Ranks follow assignment order, so
// the grouping is the same stable sort as the one-work-group version.
constexpr int kGroupChunk = kTail;

__global__ __launch_bounds__(kTail) void group_count_kernel(SelectArgs a) {
  __shared__ PermuteSmem<kTail> sm;
  const int t = threadIdx.x, E = a.E, total = a.N * a.k;
  const int C = static_cast<int>(gridDim.x);
  const int x0 = static_cast<int>(blockIdx.x) * kGroupChunk;
  const int x1 = min(total, x0 + kGroupChunk);
  StatsDev* st = static_cast<StatsDev*>(a.stats);
  if (t < kMaxE) sm.cnt[t] = 0;
  __syncthreads();
  for (int x = x0 + t; x < x1; x += kTail) atomicAdd(&sm.cnt[clamp_expert(a.topk_idx[x], E)], 1);
  __syncthreads();
  if (t < E) store_dev(&a.ghist[static_cast<size_t>(blockIdx.x) * E + t], sm.cnt[t]);
  // an arrival count out of range (a workspace that was not zero-filled or
  // is shared by overlapping calls) is flagged in this call's statistics
  if (!last_arrival_dev(&a.counters[1], C, &st->err_flags)) return;
  // the chunks' counts, a batch of chunks at a time, loaded by every thread
  // into LDS (sm.w is free here), then scanned over the chunks per expert
  int* stage = &sm.w[0][0];
  const int cb = static_cast<int>(sizeof(sm.w) / sizeof(int)) / E;  // chunks per batch
  int run = 0;
  for (int c0 = 0; c0 < C; c0 += cb) {
    const int nc = min(cb, C - c0);
    for (int i = t; i < nc * E; i += kTail)
      stage[i] = load_dev(&a.ghist[static_cast<size_t>(c0) * E + i]);
    __syncthreads();
    if (t < E)
      for (int c = 0; c < nc; ++c) {
        const int n = stage[c * E + t];
        a.ghist[static_cast<size_t>(c0 + c) * E + t] = run;
        run += n;
      }
    __syncthreads();
  }
  if (t < E) sm.cnt[t] = run;
  __syncthreads();
  permute_tables<kTail>(a.N, a.k, E, a.counts, a.offsets, a.active, a.n_active, a.resident, st, sm,
                        a.max_rows, a.groups, a.active_w, a.group_shift, a.split_rows, a.n_work);
}

__global__ __launch_bounds__(kTail) void group_scatter_kernel(SelectArgs a) {
  __shared__ PermuteSmem<kTail> sm;
  const int t = threadIdx.x, E = a.E, total = a.N * a.k;
  const int x0 = static_cast<int>(blockIdx.x) * kGroupChunk;
  const int x1 = min(total, x0 + kGroupChunk);
  if (t < E) {
    sm.off[t] = a.offsets[t];
    sm.run[t] = a.ghist[static_cast<size_t>(blockIdx.x) * E + t];
  }
  __syncthreads();
  permute_scatter<kTail>(x0, x1, E, a.topk_idx, a.sorted_assign, a.inv_pos, sm);
}

}  // namespace

void select_plan(int N, int H, int E, int /*num_cu*/, int* ksplit, int* kslice) {
  // about 128 work-groups (groups x K slices) -- 256 for layers of more than
  // 128 experts, whose router rows are long enough to fill the chip
  // (DeepSeek-V3.1-shaped block: front 59 -> 52 us), and above 512 nodes
  // (128-expert layer at 1024 nodes: 348 -> 341 us; at 256 and 512 nodes
  // 128 are as fast or faster) -- at most kMaxKSplit slices of at most
  // kMaxSlice elements each, multiples of 64
  const int groups = node_groups(N, E);
  const int target = (E > 128 || N > 512) ? 256 : 128;
  int ks = (target + groups - 1) / groups;
  if (ks > kMaxKSplit) ks = kMaxKSplit;
  const int min_ks = (H + kMaxSlice - 1) / kMaxSlice;
  if (ks < min_ks) ks = min_ks;
  if (ks > H / 64) ks = H / 64;
  int sl = (H + ks - 1) / ks;
  sl = (sl + 63) / 64 * 64;
  *kslice = sl;
  *ksplit = (H + sl - 1) / sl;
}

int node_workgroups(int N, int E) { return node_groups(N, E); }
int group_chunks(int N, int k) { return (N * k + kGroupChunk - 1) / kGroupChunk; }
size_t dpart_elems(int N, int E) { return static_cast<size_t>(dpart_stride(N, E)) * E; }
size_t fpart_bytes(int N, int E) { return static_cast<size_t>(fpart_stride(N, E)) * E; }

template <typename AT, int NPW>
void launch_front(const SelectArgs& a, dim3 grid, int q, hipStream_t stream) {
  const int nthr = 64 * front_waves<NPW>();
  if (a.ksplit <= 8) {
    if (q == 1)
      front_kernel<AT, 1, NPW, 8><<<grid, nthr, 0, stream>>>(a);
    else if (q == 2)
      front_kernel<AT, 2, NPW, 8><<<grid, nthr, 0, stream>>>(a);
    else if (q == 3)
      front_kernel<AT, 3, NPW, 8><<<grid, nthr, 0, stream>>>(a);
    else
      front_kernel<AT, 4, NPW, 8><<<grid, nthr, 0, stream>>>(a);
  } else {
    if (q == 1)
      front_kernel<AT, 1, NPW, kMaxKSplit><<<grid, nthr, 0, stream>>>(a);
    else if (q == 2)
      front_kernel<AT, 2, NPW, kMaxKSplit><<<grid, nthr, 0, stream>>>(a);
    else if (q == 3)
      front_kernel<AT, 3, NPW, kMaxKSplit><<<grid, nthr, 0, stream>>>(a);
    else
      front_kernel<AT, 4, NPW, kMaxKSplit><<<grid, nthr, 0, stream>>>(a);
  }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  const bool lin = (a.flags & kFlagLogitsIn) != 0;
  const dim3 grid(node_groups(a.N, a.E), lin ? 1 : a.ksplit, 1);
  const int q = (a.E + kWave - 1) / kWave;
  const bool big = nodes_per_group(a.N, a.E) == kNodesPerWGBig;
  if (a.act_bf16) {
    if (big)
      launch_front<uint16_t, kNodesPerWGBig>(a, grid, q, stream);
    else
      launch_front<uint16_t, kNodesPerWG>(a, grid, q, stream);
  } else {
    if (big)
      launch_front<float, kNodesPerWGBig>(a, grid, q, stream);
    else
      launch_front<float, kNodesPerWG>(a, grid, q, stream);
  }
  if (a.split_rows >= 0)
    tail_kernel<true><<<1, kTail, 0, stream>>>(a);
  else
    tail_kernel<false><<<1, kTail, 0, stream>>>(a);
  if (a.N > kFusedMaxN) {
    restricted_kernel<<<(a.N + kNodesPerWG - 1) / kNodesPerWG, 256, 0, stream>>>(a);
    if (a.counts) {
      const int chunks = group_chunks(a.N, a.k);
      group_count_kernel<<<chunks, kTail, 0, stream>>>(a);
      group_scatter_kernel<<<chunks, kTail, 0, stream>>>(a);
    } else {
      group_kernel<<<1, kTail, 0, stream>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace amoe
