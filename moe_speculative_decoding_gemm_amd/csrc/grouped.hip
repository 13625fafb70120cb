// Grouped SwiGLU over the unique active experts on gfx950 matrix cores.
//
// [MoE-SD blog, MoE layer]: after grouping, each active expert runs once on
// the tokens routed to it.  [EcoSpec, Fig. 1]: verification time grows
// linearly with the number of active experts because each one's weight block
// has to be streamed from HBM; here each active expert's w13 and w2 are read
// once per group of up to 64 routed rows (once in practice: a 64-node tree
// routes at most 64 rows to an expert).
//
// Work decomposition (both phases): a work item is one 16-column MFMA tile of
// one active expert over the full reduction length, owned by one wave.  Items
// are numbered expert-major and dealt round-robin over the waves of a
// persistent grid sized from the CU count; the number of active experts is
// read on the device, so no host round trip is needed.
//
//   phase 1 (gate/up + SwiGLU): tile columns = 8 gate rows i0..i0+7 followed
//     by the 8 up rows of the same i, so a lane holding gate(i) and the lane
//     8 above holding up(i) meet with one shuffle; h = silu(gate) * up is
//     written to h_perm[row][i] (bf16; fp32 for fp32 weights).
//   phase 2 (down): tile columns = 16 rows of w2; y_perm[row][h] in fp32.
//
// MFMA lane layout (v_mfma_f32_16x16x32_bf16; the fp32 path issues eight
// v_mfma_f32_16x16x4_f32 that together cover the same 16x16x32 block):
//   A[m][kk]  lane m + 16g holds kk in [8g, 8g+8)     (m: routed row)
//   B[kk][n]  lane n + 16g holds kk in [8g, 8g+8)     (n: weight row)
//   D[m][n]   lane n + 16g holds m  in [4g, 4g+4)
// Weights are the B operand, loaded straight from HBM into registers (16 B per
// lane per MFMA for bf16, 8 B for fp8); the A rows (x or h_perm, a few hundred
// KB that stay in L2) are gathered through sorted_assign.  FP8 E4M3FN weights
// are widened to bf16 exactly (scale 1) and the per-128x128-block scale is
// applied to each 128-long partial sum.

#include <type_traits>
#include <utility>

#include "amoe_common.h"
#include "amoe_launch.h"

namespace amoe {

namespace {

constexpr int kMT = 4;  // M tiles (16 rows each) per pass over the weights
constexpr int kUnitTab = 64;  // work units whose parameters one table holds
constexpr int kPackChunk = 128;  // reduction elements per packed chunk
constexpr int kFragElems = 512;  // elements of one packed MFMA B fragment

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- operand fragments --------------------------------------------------
// 8 consecutive reduction elements of one row, as the MFMA wants them
struct FragBF16 {
  bf16x8_t v;
};
struct FragF32 {
  float v[8];
};

template <int WK>
struct Frag;
template <>
struct Frag<0> {
  using T = FragF32;
};
template <>
struct Frag<1> {
  using T = FragBF16;
};
template <>
struct Frag<2> {
  using T = FragBF16;
};

__device__ __forceinline__ FragBF16 load_bf16x8(const uint16_t* p) {
  FragBF16 f;
  const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  f.v = __builtin_bit_cast(bf16x8_t, u);
  return f;
}
__device__ __forceinline__ FragBF16 load_bf16x8_cached(const uint16_t* p) {
  FragBF16 f;
  const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
  f.v = __builtin_bit_cast(bf16x8_t, u);
  return f;
}
__device__ __forceinline__ FragF32 load_f32x8(const float* p, bool streaming) {
  FragF32 f;
  f32x4_t a, b;
  if (streaming) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
  } else {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[i] = a[i];
    f.v[4 + i] = b[i];
  }
  return f;
}
// 8 fp8 E4M3FN codes -> 8 bf16 (exact: every E4M3FN value is a bf16 value)
__device__ __forceinline__ FragBF16 load_fp8x8(const uint8_t* p) {
  const u32x2_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  bf16x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[0], 1.0f, false);
  bf16x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[0], 1.0f, true);
  bf16x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[1], 1.0f, false);
  bf16x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[1], 1.0f, true);
  FragBF16 f;
  f.v[0] = q0[0];
  f.v[1] = q0[1];
  f.v[2] = q1[0];
  f.v[3] = q1[1];
  f.v[4] = q2[0];
  f.v[5] = q2[1];
  f.v[6] = q3[0];
  f.v[7] = q3[1];
  return f;
}

template <int WK>
struct WeightT;
template <>
struct WeightT<0> {
  using T = float;
};
template <>
struct WeightT<1> {
  using T = uint16_t;
};
template <>
struct WeightT<2> {
  using T = uint8_t;
};

template <int WK>
__device__ __forceinline__ typename Frag<WK>::T load_w(const typename WeightT<WK>::T* p);
template <>
__device__ __forceinline__ FragF32 load_w<0>(const float* p) {
  return load_f32x8(p, true);
}
template <>
__device__ __forceinline__ FragBF16 load_w<1>(const uint16_t* p) {
  return load_bf16x8(p);
}
template <>
__device__ __forceinline__ FragBF16 load_w<2>(const uint8_t* p) {
  return load_fp8x8(p);
}

// activation operand: fp32 rows for the fp32 path, bf16 rows otherwise
template <int WK>
struct ActT {
  using T = uint16_t;
};
template <>
struct ActT<0> {
  using T = float;
};

template <int WK>
__device__ __forceinline__ typename Frag<WK>::T load_a(const typename ActT<WK>::T* p, bool ok);
template <>
__device__ __forceinline__ FragF32 load_a<0>(const float* p, bool ok) {
  FragF32 f = load_f32x8(p, false);
  if (!ok)
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
  return f;
}
template <>
__device__ __forceinline__ FragBF16 load_a<1>(const uint16_t* p, bool ok) {
  FragBF16 f = load_bf16x8_cached(p);
  if (!ok) f.v = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
  return f;
}
template <>
__device__ __forceinline__ FragBF16 load_a<2>(const uint16_t* p, bool ok) {
  return load_a<1>(p, ok);
}

__device__ __forceinline__ f32x4_t mma(const FragBF16& a, const FragBF16& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma(const FragF32& a, const FragF32& b, f32x4_t c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
  return c;
}

// One wave: D[m][n] = sum_k A[m][k] * W[n][k] for up to kMT M tiles, over
// k in [0, K).  wrow: this lane's weight row (already offset by 8g);
// arow[mt]: this lane's A row for M tile mt (offset by 8g), aok[mt]: row exists.
// For FP8 (WK == 2) the per-block scale (scale(kb), kb = k0/128) multiplies
// each 128-long partial sum.
template <int WK, typename ScaleFn>
__device__ __forceinline__ void tile_product(const typename WeightT<WK>::T* wrow,
                                             const typename ActT<WK>::T* const* arow,
                                             const bool* aok, int mt_n, int K, f32x4_t* acc,
                                             ScaleFn scale) {
  using F = typename Frag<WK>::T;
  int k0 = 0;
  for (; k0 + 128 <= K; k0 += 128) {
    F b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = load_w<WK>(wrow + k0 + 32 * s);
    if (WK == 2) {
      const float sc = scale(k0 >> 7);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt >= mt_n) break;
        f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const F a = load_a<WK>(arow[mt] + k0 + 32 * s, aok[mt]);
          tmp = mma(a, b[s], tmp);
        }
        acc[mt] += sc * tmp;
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt >= mt_n) break;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const F a = load_a<WK>(arow[mt] + k0 + 32 * s, aok[mt]);
          acc[mt] = mma(a, b[s], acc[mt]);
        }
      }
    }
  }
  // tail in steps of 32 (K is a multiple of 64; FP8 K is a multiple of 128)
  for (; k0 < K; k0 += 32) {
    const F b = load_w<WK>(wrow + k0);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt >= mt_n) break;
      const F a = load_a<WK>(arow[mt] + k0, aok[mt]);
      acc[mt] = mma(a, b, acc[mt]);
    }
  }
}

template <int WK>
__global__ __launch_bounds__(256) void gateup_kernel(GroupedArgs a) {
  using WTp = typename WeightT<WK>::T;
  using ATp = typename ActT<WK>::T;
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, k = a.k;
  const int U = *a.n_active;
  const int tiles = I / 8;
  const int total = U * tiles;
  const int nwaves = gridDim.x * 4;
  const int wv = (threadIdx.x >> 6) * gridDim.x + blockIdx.x;  // spread items over CUs first
  const WTp* w13 = static_cast<const WTp*>(a.w13);
  const ATp* x = static_cast<const ATp*>(a.x);
  for (int item = wv; item < total; item += nwaves) {
    const int u = item / tiles;
    const int it = item - u * tiles;
    const int e = a.active[u];
    const int off = a.offsets[e];
    const int te = a.offsets[e + 1] - off;
    const int i0 = it * 8;
    const int half = r >> 3;  // 0: gate row, 1: up row
    const int irow = i0 + (r & 7);
    const WTp* wrow = w13 + (static_cast<size_t>(e * 2 + half) * I + irow) * H + 8 * g;
    const float* s13 = a.s13;
    const int ib = irow >> 7;
    const int nkb = H >> 7;
    auto scale = [&](int kb) {
      return s13[(static_cast<size_t>(e * 2 + half) * (I >> 7) + ib) * nkb + kb];
    };
    for (int mg = 0; mg < te; mg += 16 * kMT) {
      const int mt_n = min(kMT, (te - mg + 15) >> 4);
      const ATp* arow[kMT];
      bool aok[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int m = mg + 16 * mt + r;
        aok[mt] = m < te;
        const int tok = aok[mt] ? a.sorted_assign[off + m] / k : 0;
        arow[mt] = x + static_cast<size_t>(tok) * H + 8 * g;
      }
      f32x4_t acc[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tile_product<WK>(wrow, arow, aok, mt_n, H, acc, scale);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt >= mt_n) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float mine = acc[mt][j];
          const float up = __shfl_xor(mine, 8, kWave);
          const int m = mg + 16 * mt + 4 * g + j;
          if (half == 0 && m < te) {
            const float h = silu(mine) * up;
            const size_t o = static_cast<size_t>(off + m) * I + irow;
            if (WK == 0)
              static_cast<float*>(a.h_perm)[o] = h;
            else
              static_cast<uint16_t*>(a.h_perm)[o] = f32_to_bf16(h);
          }
        }
      }
    }
  }
}

template <int WK>
__global__ __launch_bounds__(256) void down_kernel(GroupedArgs a) {
  using WTp = typename WeightT<WK>::T;
  using ATp = typename ActT<WK>::T;
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I;
  const int U = *a.n_active;
  const int tiles = H / 16;
  const int total = U * tiles;
  const int nwaves = gridDim.x * 4;
  const int wv = (threadIdx.x >> 6) * gridDim.x + blockIdx.x;
  const WTp* w2 = static_cast<const WTp*>(a.w2);
  const ATp* hp = static_cast<const ATp*>(a.h_perm);
  for (int item = wv; item < total; item += nwaves) {
    const int u = item / tiles;
    const int it = item - u * tiles;
    const int e = a.active[u];
    const int off = a.offsets[e];
    const int te = a.offsets[e + 1] - off;
    const int hrow = it * 16 + r;
    const WTp* wrow = w2 + (static_cast<size_t>(e) * H + hrow) * I + 8 * g;
    const float* s2 = a.s2;
    const int hb = hrow >> 7;
    const int nkb = I >> 7;
    auto scale = [&](int kb) { return s2[(static_cast<size_t>(e) * (H >> 7) + hb) * nkb + kb]; };
    for (int mg = 0; mg < te; mg += 16 * kMT) {
      const int mt_n = min(kMT, (te - mg + 15) >> 4);
      const ATp* arow[kMT];
      bool aok[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int m = mg + 16 * mt + r;
        aok[mt] = m < te;
        arow[mt] = hp + static_cast<size_t>(off + (aok[mt] ? m : 0)) * I + 8 * g;
      }
      f32x4_t acc[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tile_product<WK>(wrow, arow, aok, mt_n, I, acc, scale);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt >= mt_n) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = mg + 16 * mt + 4 * g + j;
          if (m < te) a.y_perm[static_cast<size_t>(off + m) * H + hrow] = acc[mt][j];
        }
      }
    }
  }
}


// ------------------------------------------------------------------------
// Work-group items with the activation rows staged in LDS (bf16 / fp8
// weights with bf16 activations).
//
// One work-group (4 waves) owns 64*NT weight rows of one active expert (wave
// w: N tiles w*NT .. w*NT+NT-1 of 16 rows) over the full reduction length K,
// for up to 64 routed rows at a time.  The routed rows' activations are
// staged into LDS in chunks of KC reduction elements (double buffered, one
// barrier per chunk) and shared by the 4 waves; each wave keeps its weight
// fragments for the next chunk in flight in registers (ping-pong).  Loads are
// issued in the order they are consumed -- next activation chunk, then next
// weight chunk, then compute the current chunk -- so the in-order vmcnt
// waits never stall on a newer load.
template <int WK>
struct BRaw;
template <>
struct BRaw<1> {
  using T = u32x4_t;  // 8 bf16
};
template <>
struct BRaw<2> {
  using T = u32x2_t;  // 8 fp8
};

__device__ __forceinline__ bf16x8_t to_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t to_bf16x8(const u32x2_t& u) {
  const bf16x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[0], 1.0f, false);
  const bf16x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[0], 1.0f, true);
  const bf16x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[1], 1.0f, false);
  const bf16x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[1], 1.0f, true);
  bf16x8_t f;
  f[0] = q0[0];
  f[1] = q0[1];
  f[2] = q1[0];
  f[3] = q1[1];
  f[4] = q2[0];
  f[5] = q2[1];
  f[6] = q3[0];
  f[7] = q3[1];
  return f;
}

// FP8: two resident work-groups per CU (the register budget is cut to fit),
// except with paired items.
//
// GEMM tiling for blocks with many rows per expert (PAIRED, MTMAX = 8): a
// work-group takes two adjacent 64-row items of the packed layout (wave w:
// tile w of each, 32 weight rows per wave) against up to 128 routed rows at
// a time, so every staged activation chunk feeds twice the weight rows and
// every weight chunk twice the routed rows of the default tiling -- a
// quarter of the bytes per MFMA operation moved through the CU.  Each
// output element is accumulated by the same MFMA sequence as in the default
// tiling, so the results are the same bits.
template <int WK, bool GATEUP, int NT, int KC, bool PACKED, int MTMAX = 4, bool PAIRED = false,
          bool DENSE = false>
__global__ __launch_bounds__(256, (WK == 2 && !PAIRED) ? 2 : 1) void expert_lds_kernel(GroupedArgs a) {
  static_assert(!PACKED || KC == kPackChunk, "packed weights come in 128-long chunks");
  static_assert(!PAIRED || (PACKED && NT == 2), "paired items: packed weights, two tiles a wave");
  constexpr int MT = MTMAX;
  constexpr int ROWS = 16 * MT;
  constexpr int STEPS = KC / 32;
  constexpr int LDK = KC + 8;         // LDS row stride in bf16 elements (16 B pad)
  constexpr int TPR = KC / 8;         // threads per staged row, 16 B each
  constexpr int RPP = 256 / TPR;      // staged rows per pass
  using WTp = typename WeightT<WK>::T;
  using BR = typename BRaw<WK>::T;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][ROWS * LDK];
  __shared__ int s_row[ROWS];  // down, tok_rows: output row of each routed row

  const int H = a.H, I = a.I, k = a.k;
  const int K = GATEUP ? H : I;
  const int tiles = (GATEUP ? 2 * I : H) / (64 * NT);
  // dense mode: a.dense_n experts (a.active[0..dense_n), or expert u when
  // a.active is null) over every one of the N rows: expert u's rows are
  // u*N .. u*N+N-1 of h_perm / y_perm, row m being node m's x (DENSE: the
  // launcher picks it when a.dense_n > 0)
  constexpr bool dense = DENSE;
  const int n_items = (dense ? a.dense_n : *a.n_active) * tiles;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, r = lane & 15, g = lane >> 4;
  const int nchunks = (K + KC - 1) / KC;
  // packed weights are zero-padded to whole chunks: every step is computed
  const int nsteps = PACKED ? nchunks * STEPS : (K >> 5);
  const WTp* w13 = static_cast<const WTp*>(a.w13);
  const WTp* w2 = static_cast<const WTp*>(a.w2);
  const uint16_t* src_base = static_cast<const uint16_t*>(GATEUP ? a.x : a.h_perm);
  const int src_ld = GATEUP ? H : I;

  const int R = a.row_groups > 1 ? a.row_groups : 1;
  // Units: (item, row groups g0, g0 + R, ...), or, once some expert has more
  // than 64 routed rows, (64-row group, tile) pairs from the groups table
  // (group-major, so the groups of one tile are `tiles` units apart and read
  // its weights at about the same time).
  const bool by_group =
      !dense && a.groups != nullptr && a.max_rows != nullptr && *a.max_rows > ROWS;
  const int n_units = by_group ? a.groups[0] * tiles : n_items * R;
  // snake: the active list comes heaviest first and the grid is whole rounds
  // of one work-group per CU (work-group b, b + C, b + 2C, .. share CU b % C
  // under the in-order dispatch), so the first round takes ranks 0..C-1 in
  // order and every later round runs backwards: the CU with the heaviest
  // first item gets the lightest items of the later rounds
  const int C = a.num_cu;
  const bool snake = a.snake && !by_group && C > 0 && gridDim.x % C == 0;
  // A unit's parameters: group entry -> active expert -> offsets -> weight
  // slot, a chain of dependent loads.
  auto decode = [&](int unit, bool first, int& tile, int& g0, int& rstep, int& e, int& off,
                    int& te, int& ew) {
    if (snake && first) {  // unit == blockIdx.x
      const int q = unit / C, p = unit - q * C;
      unit = q == 0 ? p : q * C + (C - 1 - p);
    }
    tile = 0, g0 = 0, rstep = 1, e = -1, off = 0, te = 0, ew = 0;
    if (unit < n_units) {
      int u;
      if (by_group) {
        const int gi = unit / tiles;
        tile = unit - gi * tiles;
        const int gv = a.groups[1 + gi];
        u = gv >> 16;
        g0 = gv & 0xffff;
        rstep = 1 << 16;  // this group only
      } else {
        const int item = unit % n_items;
        g0 = unit / n_items;
        u = item / tiles;
        tile = item - u * tiles;
        rstep = R;
      }
      e = DENSE ? (a.active ? min(max(a.active[u], 0), a.E - 1) : u) : a.active[u];
      off = DENSE ? u * a.N : a.offsets[e];
      te = DENSE ? a.N : a.offsets[e + 1] - off;
      // where expert e's weights sit
      ew = a.w_slot ? min(max(a.w_slot[e], 0), a.n_wslots - 1) : e;
    }
  };
  // One unit: the item's weights against its routed-row groups.
  auto run_unit = [&](const int e, const int tile, const int g0, const int rstep, const int off,
                      const int te, const int ew) {
    const WTp* wrow[NT];
    int orow[NT];   // gate/up: intermediate index i; down: hidden index h
    int srow[NT];   // row of the weight matrix selected by the scale grid
    int half = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // 16-row tile index within the expert
      const int q = PAIRED ? (2 * tile + nt) * 4 + wave : (tile * 4 + wave) * NT + nt;
      if (GATEUP) {
        half = r >> 3;
        const int irow = q * 8 + (r & 7);
        orow[nt] = irow;
        srow[nt] = (e * 2 + half) * (I >> 7) + (irow >> 7);
        wrow[nt] = w13 + (static_cast<size_t>(ew * 2 + half) * I + irow) * H + 8 * g;
      } else {
        const int hrow = q * 16 + r;
        orow[nt] = hrow;
        srow[nt] = e * (H >> 7) + (hrow >> 7);
        wrow[nt] = w2 + (static_cast<size_t>(ew) * H + hrow) * I + 8 * g;
      }
    }
    const float* scales = GATEUP ? a.s13 : a.s2;
    const int nkb = K >> 7;
    // packed: this wave's fragments of the item, chunk-major (see pack_kernel);
    // paired: of the first of the two items (NT = 1 layout), the second one
    // item_stride elements further
    constexpr int PNT = PAIRED ? 1 : NT;  // tiles per wave in the packed layout
    const size_t item_stride = static_cast<size_t>(nchunks) * 16 * kFragElems;
    const WTp* pbase = static_cast<const WTp*>(GATEUP ? a.w13 : a.w2) +
                       (static_cast<size_t>(ew) * tiles * (NT / PNT) + tile * (NT / PNT)) *
                           nchunks * (16 * PNT) * kFragElems +
                       static_cast<size_t>(wave) * PNT * kFragElems + lane * 8;

    for (int mg = g0 * ROWS; mg < te; mg += rstep * ROWS) {
      // One group of routed rows mg.. with MTV 16-row M tiles: only as many
      // activation rows are staged (and MFMA tiles computed) as the group
      // has, rounded up to 16, 32 or 64 -- rows past the routed ones would
      // re-read row mg and still occupy the CU's load path.
      auto group = [&](auto mtc) {
        constexpr int MTV = decltype(mtc)::value;
        constexpr int PV = 16 * MTV / RPP;  // staging passes
        static_assert(RPP == 16 && PV == MTV, "one 16-row staging pass per M tile");
        const int mt_n = min(MTV, (te - mg + 15) >> 4);
        // Staging sources, PV rows per thread.  Rows past the routed ones
        // read row 0 of the group instead (their results are never stored), so
        // every load below is unconditional: guarded loads would make the
        // compiler's wait counting fall back to waiting for all of them.
        // (as 32-bit element offsets from src_base -- at most N*k rows of at
        // most 16384 elements, below 2^31 -- one register each, the base in
        // scalar registers)
        uint32_t src[PV];
        const int kk = (t % TPR) * 8;
#pragma unroll
        for (int p = 0; p < PV; ++p) {
          const int rr = p * RPP + t / TPR;
          const int m = mg + rr < te ? mg + rr : mg;
          const int srcrow = GATEUP ? (dense ? m : a.sorted_assign[off + m] / k) : off + m;
          src[p] = static_cast<uint32_t>(srcrow) * static_cast<uint32_t>(src_ld);
        }
        f32x4_t acc[NT][MTV];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mt = 0; mt < MTV; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Pipeline, two chunks deep for both operands: activation chunk c waits
        // in a VGPR ring of 2 until the end of chunk c-1, when it is written to
        // LDS buffer c%2; weight chunk c waits in a VGPR ring of 2.  Issue order
        // per chunk c: activations of c+2, compute c, weights of c+2, then store
        // activations of c+1.  That store waits for activations c+1 and the
        // loads older than them (vmcnt retires in issue order); weights c+1 were
        // issued after activations c+1, so no wait ever stalls on weights that
        // are not needed yet.  All loads of the steady state are unconditional;
        // columns and steps past K are clamped to valid addresses whose data is
        // never used.
        u32x4_t sv[2][PV];
        auto stage_load = [&](u32x4_t (&v)[PV], int c) {
          const int k0 = min(c * KC + kk, K - 8);
#pragma unroll
          for (int p = 0; p < PV; ++p) v[p] = *reinterpret_cast<const u32x4_t*>(src_base + (src[p] + k0));
        };
        auto stage_store = [&](const u32x4_t (&v)[PV], int buf) {
#pragma unroll
          for (int p = 0; p < PV; ++p) {
            const int rr = p * RPP + t / TPR;
            *reinterpret_cast<u32x4_t*>(&sA[buf][rr * LDK + kk]) = v[p];
          }
        };
        // weights of chunk c, and for FP8 their block scales (one per tile row
        // and 128-block: KC == 128), loaded together so that the scale is in a
        // register when the chunk is computed
        auto load_b = [&](BR (&b)[STEPS][NT], float (&bs)[NT], int c) {
          if (WK == 2) {
            const int kb = (min(c, nchunks - 1) * KC) >> 7;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bs[nt] = scales[static_cast<size_t>(srow[nt]) * nkb + kb];
          }
#pragma unroll
          for (int j = 0; j < STEPS; ++j) {
            if (PACKED) {
              const WTp* f = pbase + static_cast<size_t>((min(c, nchunks - 1) * 4 + j) * 4 * PNT) * kFragElems;
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                b[j][nt] = __builtin_nontemporal_load(reinterpret_cast<const BR*>(
                    f + (PAIRED ? nt * item_stride : static_cast<size_t>(nt) * kFragElems)));
            } else {
              const int s = min(c * STEPS + j, nsteps - 1);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                b[j][nt] = __builtin_nontemporal_load(reinterpret_cast<const BR*>(wrow[nt] + s * 32));
            }
          }
        };
        auto compute = [&](const BR (&b)[STEPS][NT], const float (&bs)[NT], int c, int buf) {
          f32x4_t tmp[NT][MTV];
          if (WK == 2) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int mt = 0; mt < MTV; ++mt) tmp[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int j = 0; j < STEPS; ++j) {
            if (c * STEPS + j >= nsteps) break;
            bf16x8_t bf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bf[nt] = to_bf16x8(b[j][nt]);
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) {
              if (mt >= mt_n) break;
              const bf16x8_t af = __builtin_bit_cast(
                  bf16x8_t, *reinterpret_cast<const u32x4_t*>(&sA[buf][(mt * 16 + r) * LDK + 32 * j + 8 * g]));
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) {
                if (WK == 2)
                  tmp[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[nt], tmp[nt][mt], 0, 0, 0);
                else
                  acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[nt], acc[nt][mt], 0, 0, 0);
              }
            }
          }
          if (WK == 2) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const float sc = bs[nt];
#pragma unroll
              for (int mt = 0; mt < MTV; ++mt) acc[nt][mt] += sc * tmp[nt][mt];
            }
          }
        };

        // Weight chunks in flight: 2 for bf16, 4 for fp8 (an fp8 chunk is half
        // the bytes; a CU streams at the rate its bytes in flight allow); 2
        // for paired items, which already carry two tiles a wave.
        constexpr int DW = (WK == 2 && !PAIRED) ? 4 : 2;
        BR bq[DW][STEPS][NT];
        float bsc[DW][NT];  // FP8 block scales of the chunks in flight
        // prologue: A0 B0 A1 B1 .. B(DW-1)
        stage_load(sv[0], 0);
        load_b(bq[0], bsc[0], 0);
        stage_load(sv[1], min(1, nchunks - 1));
#pragma unroll
        for (int d = 1; d < DW; ++d) load_b(bq[d], bsc[d], min(d, nchunks - 1));
        // down, token-major output: each routed row's assignment index, loaded
        // behind the pipeline's loads and used only by the epilogue
        const bool tok = !GATEUP && a.tok_rows && !dense;
        int my_row = 0;
        if (tok) my_row = a.sorted_assign[off + min(mg + (ROWS <= kWave ? lane : t), te - 1)];
        stage_store(sv[0], 0);
        __syncthreads();
        // chunk c: weights in ring slot c % DW, activations in VGPR ring / LDS
        // buffer c % 2.  guard: near the end, loads past the last chunk are
        // skipped (the steady state has none).
        auto body = [&](auto wc, int c, bool guard) {
          constexpr int w = decltype(wc)::value;
          constexpr int i = w & 1;
          if (!guard || c + 2 < nchunks) stage_load(sv[i], c + 2);
          compute(bq[w], bsc[w], c, i);
          if (!guard || c + DW < nchunks) load_b(bq[w], bsc[w], c + DW);
          if (!guard || c + 1 < nchunks) stage_store(sv[i ^ 1], i ^ 1);
          __syncthreads();
        };
        int c = 0;
        for (; c + 2 * DW <= nchunks; c += DW)  // every load of these DW chunks is in range
          static_for<DW>([&](auto d) { body(d, c + decltype(d)::value, false); });
        // 0 .. 2*DW-1 chunks remain; c is a multiple of DW
        static_for<2 * DW>([&](auto q) {
          constexpr int qq = decltype(q)::value;
          if (c + qq < nchunks) body(std::integral_constant<int, qq % DW>{}, c + qq, true);
        });

        if (tok) {
          if (t < ROWS) s_row[t] = my_row;
          __syncthreads();
        }
        // epilogue: lane (r, g) holds D[m = 4g + j][n = r] of each tile
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int mt = 0; mt < MTV; ++mt) {
            if (mt >= mt_n) break;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int m = mg + 16 * mt + 4 * g + j;
              const float v = acc[nt][mt][j];
              if (GATEUP) {
                const float up = __shfl_xor(v, 8, kWave);
                if (half == 0 && m < te)
                  static_cast<uint16_t*>(a.h_perm)[static_cast<size_t>(off + m) * I + orow[nt]] =
                      f32_to_bf16(silu(v) * up);
              } else if (m < te) {
                const int row = tok ? s_row[m - mg] : off + m;
                a.y_perm[static_cast<size_t>(row) * H + orow[nt]] = v;
              }
            }
          }
        }
      };
      const int rows = te - mg;
      if (rows <= 16) {
        group(std::integral_constant<int, 1>{});
      } else if (rows <= 32) {
        group(std::integral_constant<int, 2>{});
      } else if (MTMAX <= 4 || rows <= 64) {
        group(std::integral_constant<int, 4>{});
      } else {
        if constexpr (MTMAX >= 8) group(std::integral_constant<int, 8>{});
      }
    }
  };
  // A work-group with more than one unit has the parameters of its next
  // kUnitTab units decoded by kUnitTab threads at once into LDS, so that a
  // unit starts its loads without the chain in front of them; with one unit
  // every thread decodes it itself (no barriers).
  // (bf16 only: a second copy of the unit code raises the FP8 kernels'
  // register pressure past their budget of two work-groups per CU)
  const int n_iter = (n_units + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x);
  if constexpr (WK == 1) {
    if (n_iter <= 1) {
      int tile, g0, rstep, e, off, te, ew;
      decode(static_cast<int>(blockIdx.x), true, tile, g0, rstep, e, off, te, ew);
      if (e >= 0) run_unit(e, tile, g0, rstep, off, te, ew);
      return;
    }
  }
  __shared__ int s_tab[7][kUnitTab];
  for (int i0 = 0; i0 < n_iter; i0 += kUnitTab) {
    const int ni = min(kUnitTab, n_iter - i0);
    __syncthreads();  // the last table's entries are read
    if (t < ni) {
      const int base = (i0 + t) * static_cast<int>(gridDim.x);
      int unit = base + static_cast<int>(blockIdx.x);
      if (snake && base == 0) {
        const int q = unit / C, p = unit - q * C;
        unit = q == 0 ? p : q * C + (C - 1 - p);
      }
      int tile = 0, g0 = 0, rstep = 1, e = -1, off = 0, te = 0, ew = 0;
      if (unit < n_units) {
        int u;
        if (by_group) {
          const int gi = unit / tiles;
          tile = unit - gi * tiles;
          const int gv = a.groups[1 + gi];
          u = gv >> 16;
          g0 = gv & 0xffff;
          rstep = 1 << 16;  // this group only
        } else {
          const int item = unit % n_items;
          g0 = unit / n_items;
          u = item / tiles;
          tile = item - u * tiles;
          rstep = R;
        }
        e = DENSE ? (a.active ? min(max(a.active[u], 0), a.E - 1) : u) : a.active[u];
        off = DENSE ? u * a.N : a.offsets[e];
        te = DENSE ? a.N : a.offsets[e + 1] - off;
        ew = a.w_slot ? min(max(a.w_slot[e], 0), a.n_wslots - 1) : e;
      }
      s_tab[0][t] = tile;
      s_tab[1][t] = g0;
      s_tab[2][t] = rstep;
      s_tab[3][t] = e;
      s_tab[4][t] = off;
      s_tab[5][t] = te;
      s_tab[6][t] = ew;
    }
    __syncthreads();
    for (int ii = 0; ii < ni; ++ii) {
      // the same for every lane: scalar registers
      const auto rd = [&](int f) { return __builtin_amdgcn_readfirstlane(s_tab[f][ii]); };
      const int e = rd(3);
      if (e < 0) continue;  // past the units
      run_unit(e, rd(0), rd(1), rd(2), rd(4), rd(5), rd(6));
    }
  }
}

// ------------------------------------------------------------------------
// Packed expert layout.  Weights are static, so they are reordered once
// (at load time) into exactly the order the expert kernels read them: each
// wave load instruction then reads 1 KB of consecutive bytes and each
// work-group streams one contiguous region, which is what lets HBM run near
// its peak (16-row x 64-byte fragment reads of row-major weights scatter
// every instruction over 16 DRAM locations).
//
// Unit: a fragment = the B operand of one 16x16x32 MFMA for one 16-row tile
// and 32 reduction elements, stored lane-major (lane l = r + 16g holds the 8
// elements row(r), k = 32*step + 8g .. +7): 512 elements.  Tile q of an
// expert is rows 16q..16q+15 of w2, or for w13 the 8 gate rows 8q..8q+7
// followed by the 8 up rows 8q..8q+7.  A group = the 4*NT tiles of one
// work-group item (wave w: tiles w*NT .. w*NT+NT-1).  Order:
//   [expert][group][chunk of 128][step (4)][wave (4)][tile nt (NT)][lane][8]
// The reduction dimension is zero-padded to whole chunks.
constexpr int kPackNT_bf16 = 1;
constexpr int kPackNT_fp8 = 1;

template <int WK, bool GATEUP>
__global__ __launch_bounds__(256) void pack_kernel(const typename WeightT<WK>::T* __restrict__ src,
                                                   typename WeightT<WK>::T* __restrict__ dst,
                                                   int E, int H, int I) {
  using WTp = typename WeightT<WK>::T;
  constexpr int NT = WK == 2 ? kPackNT_fp8 : kPackNT_bf16;
  const int K = GATEUP ? H : I;
  const int nC = (K + kPackChunk - 1) / kPackChunk;
  const int nG = (GATEUP ? 2 * I : H) / (64 * NT);
  const size_t units = static_cast<size_t>(E) * nG * nC * 16 * NT * 64;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= units) return;
  size_t rest = idx;
  const int lane = static_cast<int>(rest % 64);
  rest /= 64;
  const int nt = static_cast<int>(rest % NT);
  rest /= NT;
  const int w = static_cast<int>(rest % 4);
  rest /= 4;
  const int j = static_cast<int>(rest % 4);
  rest /= 4;
  const int c = static_cast<int>(rest % nC);
  rest /= nC;
  const int G = static_cast<int>(rest % nG);
  const int e = static_cast<int>(rest / nG);
  const int q = (G * 4 + w) * NT + nt;
  const int r = lane & 15, g = lane >> 4;
  const int k = c * kPackChunk + 32 * j + 8 * g;
  const WTp* row;
  if (GATEUP) {
    const int half = r >> 3;
    row = src + (static_cast<size_t>(e * 2 + half) * I + q * 8 + (r & 7)) * H;
  } else {
    row = src + (static_cast<size_t>(e) * H + q * 16 + r) * I;
  }
  WTp* out = dst + idx * 8;
  if (WK == 2) {
    u32x2_t v = {0u, 0u};
    if (k < K) v = *reinterpret_cast<const u32x2_t*>(row + k);
    *reinterpret_cast<u32x2_t*>(out) = v;
  } else {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (k < K) v = *reinterpret_cast<const u32x4_t*>(row + k);
    *reinterpret_cast<u32x4_t*>(out) = v;
  }
}

}  // namespace

template <int WK>
void launch_wk(const GroupedArgs& a, hipStream_t stream, int which) {
  const int blocks = a.num_cu * 2;
  if (which != 2) gateup_kernel<WK><<<blocks, 256, 0, stream>>>(a);
  if (which != 1) down_kernel<WK><<<blocks, 256, 0, stream>>>(a);
}

// resident work-groups per CU of one kernel (queried once per process)
template <typename Kern>
int resident_per_cu(Kern kern, int fallback) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, 0) != hipSuccess || n <= 0)
    n = fallback;
  return n;
}

template <int WK, int NT, int KC, bool PACKED, int MTMAX = 4, bool PAIRED = false,
          bool DENSE = false>
void launch_lds(const GroupedArgs& a, hipStream_t stream, int which) {
  static const int occ_g =
      resident_per_cu(expert_lds_kernel<WK, true, NT, KC, PACKED, MTMAX, PAIRED, DENSE>, 2);
  static const int occ_d =
      resident_per_cu(expert_lds_kernel<WK, false, NT, KC, PACKED, MTMAX, PAIRED, DENSE>, 2);
  const int max_active = a.dense_n > 0 ? a.dense_n : (a.E < a.N * a.k ? a.E : a.N * a.k);
  const int R = a.row_groups > 1 ? a.row_groups : 1;
  if (which != 2) {
    const int items = max_active * (2 * a.I / (64 * NT)) * R;
    const int grid = items < occ_g * a.num_cu ? items : occ_g * a.num_cu;
    expert_lds_kernel<WK, true, NT, KC, PACKED, MTMAX, PAIRED, DENSE><<<grid, 256, 0, stream>>>(a);
  }
  if (which != 1) {
    const int items = max_active * (a.H / (64 * NT)) * R;
    const int grid = items < occ_d * a.num_cu ? items : occ_d * a.num_cu;
    expert_lds_kernel<WK, false, NT, KC, PACKED, MTMAX, PAIRED, DENSE><<<grid, 256, 0, stream>>>(a);
  }
}

hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream, int which) {
  const bool dense = a.dense_n > 0;
  switch (a.w_kind) {
    case 0:
      launch_wk<0>(a, stream, which);
      break;
    case 1:
      if (a.packed && a.gemm)
        launch_lds<1, 2, kPackChunk, true, 8, true>(a, stream, which);
      else if (a.packed && dense)
        launch_lds<1, kPackNT_bf16, kPackChunk, true, 4, false, true>(a, stream, which);
      else if (a.packed)
        launch_lds<1, kPackNT_bf16, kPackChunk, true>(a, stream, which);
      else if (dense)
        launch_lds<1, 1, 128, false, 4, false, true>(a, stream, which);
      else
        launch_lds<1, 1, 128, false>(a, stream, which);
      break;
    default:
      if (a.packed && a.gemm)
        launch_lds<2, 2, kPackChunk, true, 8, true>(a, stream, which);
      else if (a.packed && dense)
        launch_lds<2, kPackNT_fp8, kPackChunk, true, 4, false, true>(a, stream, which);
      else if (a.packed)
        launch_lds<2, kPackNT_fp8, kPackChunk, true>(a, stream, which);
      else if (dense)
        launch_lds<2, 1, 128, false, 4, false, true>(a, stream, which);
      else
        launch_lds<2, 1, 128, false>(a, stream, which);
      break;
  }
  return hipGetLastError();
}

size_t packed_bytes(int which, int w_kind, int E, int H, int I) {
  const int NT = w_kind == 2 ? kPackNT_fp8 : kPackNT_bf16;
  const int esize = w_kind == 2 ? 1 : 2;
  const int K = which == 0 ? H : I;
  const size_t nC = (K + kPackChunk - 1) / kPackChunk;
  const size_t nG = (which == 0 ? 2 * static_cast<size_t>(I) : H) / (64 * NT);
  return static_cast<size_t>(E) * nG * nC * 16 * NT * kFragElems * esize;
}

hipError_t launch_pack(int which, int w_kind, int E, int H, int I, const void* src, void* dst,
                       hipStream_t stream) {
  const size_t units = packed_bytes(which, w_kind, E, H, I) / ((w_kind == 2 ? 1 : 2) * 8);
  const unsigned blocks = static_cast<unsigned>((units + 255) / 256);
  if (w_kind == 2) {
    if (which == 0)
      pack_kernel<2, true><<<blocks, 256, 0, stream>>>(static_cast<const uint8_t*>(src),
                                                       static_cast<uint8_t*>(dst), E, H, I);
    else
      pack_kernel<2, false><<<blocks, 256, 0, stream>>>(static_cast<const uint8_t*>(src),
                                                        static_cast<uint8_t*>(dst), E, H, I);
  } else {
    if (which == 0)
      pack_kernel<1, true><<<blocks, 256, 0, stream>>>(static_cast<const uint16_t*>(src),
                                                       static_cast<uint16_t*>(dst), E, H, I);
    else
      pack_kernel<1, false><<<blocks, 256, 0, stream>>>(static_cast<const uint16_t*>(src),
                                                        static_cast<uint16_t*>(dst), E, H, I);
  }
  return hipGetLastError();
}

}  // namespace amoe
