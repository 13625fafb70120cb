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

#include "amoe_common.h"
#include "amoe_launch.h"

namespace amoe {

namespace {

constexpr int kMT = 4;  // M tiles (16 rows each) per pass over the weights

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

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }

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

}  // namespace

template <int WK>
void launch_wk(const GroupedArgs& a, hipStream_t stream, int which) {
  const int blocks = a.num_cu * 2;
  if (which != 2) gateup_kernel<WK><<<blocks, 256, 0, stream>>>(a);
  if (which != 1) down_kernel<WK><<<blocks, 256, 0, stream>>>(a);
}

hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream, int which) {
  switch (a.w_kind) {
    case 0:
      launch_wk<0>(a, stream, which);
      break;
    case 1:
      launch_wk<1>(a, stream, which);
      break;
    default:
      launch_wk<2>(a, stream, which);
      break;
  }
  return hipGetLastError();
}

}  // namespace amoe
