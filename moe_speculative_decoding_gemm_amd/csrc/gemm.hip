// Grouped GEMM for the experts that many routed rows reach, on gfx950
// matrix cores (bf16 weights in the packed layout, bf16 activations).
//
// [MoESD §5.1-§5.2]: as the verification batch grows, the active experts
// saturate and the routed rows per active expert keep growing, so an
// expert's FLOPs per weight byte grow with the batch until the layer turns
// from memory-bound to compute-bound.  The streaming expert kernels
// (grouped.hip) keep at most 128 routed rows per pass over an expert's
// weights; here one work-group per CU holds a 128 x 512 output tile -- 128
// routed rows of one expert against 512 weight rows (8 packed items) -- in
// 8 waves of 128 x 64 (8 x 4 MFMA tiles of 16 x 16, the accumulators in the
// accumulation registers), two waves per SIMD.
//
// Every output element takes the same v_mfma_f32_16x16x32_bf16 sequence
// over the same reduction steps (activation elements past K clamped the
// same way) as in the streaming kernels, so the results are the same bits.
//
// Work units: (row group of an expert, 512-column tile), group-major, from
// the groups table that the grouping writes for these experts.  The grid
// is one work-group per CU; work-group b runs on XCD b mod 8, so XCD x takes
// the contiguous unit range x * span .. and its CUs work on neighbouring
// units at the same time: the column tiles of one row group share its
// activation rows, and the row groups of one expert share the weights, in
// that XCD's L2.

#include "amoe_common.h"
#include "amoe_launch.h"

#include <type_traits>

namespace amoe {

namespace {

constexpr int kFragBytes = 1024;              // one MFMA operand fragment: 64 lanes x 16 B
constexpr int kFragElems = 512;               // bf16 elements of one fragment
constexpr int kStepElems = 4 * kFragElems;    // one 32-long step of one packed item
constexpr int kXcds = 8;
using lds_void = __attribute__((address_space(3))) void;

// Wave w owns item w of the tile.  A wave's weight fragments are its own:
// they go from memory straight to registers, three steps ahead, with no
// barrier.  Only the activation fragments are shared: an 8-slot LDS ring
// filled by direct loads five steps ahead (each wave 1 of the 8 fragments of
// a step).  A barrier every second step orders the ring.  The memory counter
// drains in order: waiting for the activations of steps s + 1, s + 2
// (loaded at steps s - 4, s - 3) also waits for the weights loaded before
// them, which are those of steps up to s -- so the weights keep their three
// steps.

constexpr int kWideItems = 8;        // packed items per wide tile (512 weight rows)
constexpr int kASlotElems = 8 * 64;  // one activation slot: 8 fragments as u32x4 per lane
constexpr int kWideSlots = 8;        // activation ring slots
constexpr int kAAhead = 5;           // steps the activation loads run ahead
constexpr int kBAhead = 3;           // steps the weight loads run ahead
// epilogue staging: 16 rows of the 512-column tile, fp32, rows padded by 4
// floats (the accumulator writes of a wave's four 4-row groups then fall in
// different banks)
constexpr int kStageLd = 512 + 4;

// A direct load written out (16 B per lane to lds + 16 lane): the compiler
// then does not see the ring being written and, before its own LDS reads,
// waits for nothing (ring_barrier orders the ring); its waits for the weight
// registers count one load fewer per ring load after them, i.e. wait for a
// little more than needed.  M0 (the LDS address of the load) is saved and
// restored around it.
__device__ __forceinline__ void frag_load(const void* src, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

// This wave's loads older than its last VM are done (its ring loads are in
// LDS); then the work-group barrier (other waves' loads of the same step
// are in LDS too).
template <int VM>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(VM) : "memory");
}


// Four rows of 4 MFMAs (activation fragments av[0..3] against the 4 weight
// fragments b, into the accumulators of rows ROW0 .. ROW0 + 3) with four
// fragment reads (at lds + OFF, OFF + 1024, ...) issued in front of them and
// waited for at the end of the same statement.
template <int ROW0, int OFF>
__device__ __forceinline__ void mfma_4x4(f32x4_t (&c)[8][4], const u32x4_t (&av)[4],
                                         const u32x4_t (&b)[4], uint32_t lds, u32x4_t (&r)[4]) {
  asm volatile(
      "ds_read_b128 %[r0], %[la] offset:%[o0]\n\t"
      "ds_read_b128 %[r1], %[la] offset:%[o1]\n\t"
      "ds_read_b128 %[r2], %[la] offset:%[o2]\n\t"
      "ds_read_b128 %[r3], %[la] offset:%[o3]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c02], %[a0], %[b2], %[c02]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c03], %[a0], %[b3], %[c03]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c12], %[a1], %[b2], %[c12]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c13], %[a1], %[b3], %[c13]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c20], %[a2], %[b0], %[c20]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c21], %[a2], %[b1], %[c21]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c22], %[a2], %[b2], %[c22]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c23], %[a2], %[b3], %[c23]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c30], %[a3], %[b0], %[c30]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c31], %[a3], %[b1], %[c31]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c32], %[a3], %[b2], %[c32]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c33], %[a3], %[b3], %[c33]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [c00] "+a"(c[ROW0][0]), [c01] "+a"(c[ROW0][1]), [c02] "+a"(c[ROW0][2]), [c03] "+a"(c[ROW0][3]),
        [c10] "+a"(c[ROW0 + 1][0]), [c11] "+a"(c[ROW0 + 1][1]), [c12] "+a"(c[ROW0 + 1][2]),
        [c13] "+a"(c[ROW0 + 1][3]), [c20] "+a"(c[ROW0 + 2][0]), [c21] "+a"(c[ROW0 + 2][1]),
        [c22] "+a"(c[ROW0 + 2][2]), [c23] "+a"(c[ROW0 + 2][3]), [c30] "+a"(c[ROW0 + 3][0]),
        [c31] "+a"(c[ROW0 + 3][1]), [c32] "+a"(c[ROW0 + 3][2]), [c33] "+a"(c[ROW0 + 3][3]),
        [r0] "=&v"(r[0]), [r1] "=&v"(r[1]), [r2] "=&v"(r[2]), [r3] "=&v"(r[3])
      : [a0] "v"(av[0]), [a1] "v"(av[1]), [a2] "v"(av[2]), [a3] "v"(av[3]), [b0] "v"(b[0]),
        [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [la] "v"(lds), [o0] "i"(OFF),
        [o1] "i"(OFF + 1024), [o2] "i"(OFF + 2048), [o3] "i"(OFF + 3072)
      : "memory");
}

// One work-group per CU: the tile (128 routed rows x 512 weight rows) in 8
// waves, two per SIMD: wave w owns item w (128 x 64, 4 weight fragments a
// step), so while one wave of a SIMD waits (barrier, memory) the other
// issues its MFMAs.  Per step a wave loads its 4 weight fragments (kBAhead
// steps ahead, straight to registers) and 1 of the 8 activation fragments
// (into the LDS ring, kAAhead steps ahead): 5 memory operations, the
// activation load third.  It reads the activation fragments from the ring
// half a step ahead (rows 4..7 during rows 0..3, rows 0..3 of the next step
// during rows 4..7), which keeps its registers within the budget of two
// waves per SIMD.
template <bool GATEUP>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GroupedArgs a) {
  __shared__ __attribute__((aligned(kFragBytes))) u32x4_t ring[kWideSlots * kASlotElems];
  __shared__ __attribute__((aligned(16))) float stage[2 * 16 * kStageLd];
  __shared__ int orows[128];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, k = a.k;
  const int K = GATEUP ? H : I;
  const int nsteps = ((K + 127) >> 7) * 4;  // a multiple of 4
  const int items = (GATEUP ? 2 * I : H) >> 6;
  const int ntiles = (items + kWideItems - 1) / kWideItems;
  const int32_t* groups = a.gemm_groups;
  const int n_units = groups[0] * ntiles;
  const int per_x = gridDim.x / kXcds;
  const int xcd = static_cast<int>(blockIdx.x) % kXcds;
  const int slot = static_cast<int>(blockIdx.x) / kXcds;
  const int span = (n_units + kXcds - 1) / kXcds;
  const uint16_t* wts = static_cast<const uint16_t*>(GATEUP ? a.w13 : a.w2);
  const uint16_t* src = static_cast<const uint16_t*>(GATEUP ? a.x : a.h_perm);
  const int src_ld = GATEUP ? H : I;

  for (int j = slot; j < span && xcd * span + j < n_units; j += per_x) {
    const int unit = xcd * span + j;
    const int gi = unit / ntiles;
    const int nt = unit - gi * ntiles;
    const int gv = groups[1 + gi];
    const int e = gv >> 16;
    const int m0 = (gv & 0xffff) * 128;
    const int off = a.offsets[e] + m0;
    const int rows = min(128, a.offsets[e + 1] - off);
    const int n_items = min(kWideItems, items - nt * kWideItems);

    // activation fragment `wave` of each step (rows past the group's read
    // its first row); this wave's weight item (past the expert's: its last
    // item, loaded and never used)
    const uint16_t* arow;
    {
      const int m = wave * 16 + r < rows ? wave * 16 + r : 0;
      const int srow = GATEUP ? a.sorted_assign[off + m] / k : off + m;
      arow = src + static_cast<size_t>(srow) * src_ld + 8 * g;
    }
    const int item = min(nt * kWideItems + wave, items - 1);
    const uint16_t* bsrc = wts + (static_cast<size_t>(e) * items + item) * nsteps * kStepElems + lane * 8;
    const bool busy = wave < n_items;
    int orow_t = 0;
    if (!GATEUP && t < rows) orow_t = a.tok_rows ? a.sorted_assign[off + t] : off + t;

    auto issue_a = [&](int s) {
      u32x4_t* dst = ring + (s % kWideSlots) * kASlotElems;
      const int kk = min(min(s, nsteps - 1) * 32, K - 8 - 8 * g);
      frag_load(arow + kk, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                               (lds_void*)(dst + wave * 64))));
    };
    u32x4_t bset[kBAhead + 1][4];
    auto load_b2 = [&](int s, u32x4_t(&bv)[4], int q0) {
      const size_t so = static_cast<size_t>(min(s, nsteps - 1)) * kStepElems;
#pragma unroll
      for (int q = q0; q < q0 + 2; ++q)
        bv[q] = *reinterpret_cast<const u32x4_t*>(bsrc + so + q * kFragElems);
    };
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t alo[4], ahi[4];
    const uint32_t ring_lds =
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)ring)) + lane * 16;
    // Step s: rows 0..3 with alo (step s, read during step s - 1), reading
    // rows 4..7 of step s into ahi; rows 4..7 with ahi, reading rows 0..3 of
    // step s + 1 into alo.  The loads: weights of step s + kBAhead (two,
    // then two) and this wave's activation fragment of step s + kAAhead.
    auto step = [&](int s, auto rc) {
      constexpr int R = decltype(rc)::value;
      // every second step: the activations of steps s + 1, s + 2 are in LDS
      // (the later one went out at step s - 3 as the third of its 5 loads:
      // 2 + 2 * 5 younger ones may be in flight), and every wave is past
      // step s - 1, so the slots of steps s - 3, s - 2 take the loads of
      // steps s + 5, s + 6
      if ((R & 1) == 0) ring_barrier<2 + 2 * 5>();
      const uint32_t la = ring_lds + (s % kWideSlots) * (kASlotElems * 16);
      const uint32_t ln = ring_lds + ((s + 1) % kWideSlots) * (kASlotElems * 16);
      const u32x4_t(&bc)[4] = bset[R % (kBAhead + 1)];
      u32x4_t(&bn)[4] = bset[(R + kBAhead) % (kBAhead + 1)];
      mfma_4x4<0, 4096>(acc, alo, bc, la, ahi);
      load_b2(s + kBAhead, bn, 0);
      issue_a(s + kAAhead);
      mfma_4x4<4, 0>(acc, ahi, bc, ln, alo);
      load_b2(s + kBAhead, bn, 2);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
#pragma unroll
    for (int p = 0; p < kAAhead; ++p) issue_a(p);
    asm volatile("" ::: "memory");  // the activation loads go out first
#pragma unroll
    for (int p = 0; p < kBAhead; ++p) {
      load_b2(p, bset[p], 0);
      load_b2(p, bset[p], 2);
    }
    ring_barrier<4 * kBAhead>();  // every activation load above is in LDS
    {
      const u32x4_t* sl = ring;  // step 0, rows 0..3
#pragma unroll
      for (int i = 0; i < 4; ++i) alo[i] = sl[i * 64 + lane];
    }
    for (int s = 0; s < nsteps; s += 4) {
      step(s, C0{});
      step(s + 1, C1{});
      step(s + 2, C2{});
      step(s + 3, C3{});
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue, one 16-row slab of the tile at a time through LDS (two
    // buffers): the waves write their accumulators (lane (r, g) holds
    // D[4g + jj][r] of each 16 x 16 tile; wave w's 64 columns at w * 64),
    // then the work-group writes whole row segments with 16-byte stores --
    // down: the fp32 rows; gate/up: the SwiGLU of each 16-column tile's gate
    // (columns 0..7) and up (8..15) halves, 8 bf16 of h per store.  Columns
    // of items past the expert's are not written.
    // (the thread index taken afresh: addresses derived from it are not
    // hoisted out of the unit loop to stay live, in spilled registers,
    // across the main loop)
    int te = t;
    asm volatile("" : "+v"(te));
    const int re = te & 15, ge = (te >> 4) & 3, we = te >> 6;
    if (!GATEUP && te < 128) orows[te] = orow_t;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i * 16 >= rows) break;
      float* st = stage + (i & 1) * (16 * kStageLd);
      if (busy) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            st[(4 * ge + jj) * kStageLd + we * 64 + q * 16 + re] = acc[i][q][jj];
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (GATEUP) {
        const int u = te;
        const int row = u >> 5, tile = u & 31;
        const int ml = i * 16 + row;
        if (ml < rows && (tile >> 2) < n_items) {
          const float* gp = st + row * kStageLd + tile * 16;
          const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gp);
          const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gp + 4);
          const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(gp + 8);
          const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(gp + 12);
          u32x4_t hv;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float gl = c < 2 ? g0[2 * c] : g1[2 * c - 4];
            const float gh = c < 2 ? g0[2 * c + 1] : g1[2 * c - 3];
            const float ul = c < 2 ? u0[2 * c] : u1[2 * c - 4];
            const float uh = c < 2 ? u0[2 * c + 1] : u1[2 * c - 3];
            hv[c] = static_cast<uint32_t>(f32_to_bf16(silu(gl) * ul)) |
                    (static_cast<uint32_t>(f32_to_bf16(silu(gh) * uh)) << 16);
          }
          const int qq = nt * (kWideItems * 4) + tile;
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.h_perm) +
                                      static_cast<size_t>(off + ml) * I + 8 * qq) = hv;
        }
      } else {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int u = it * 512 + te;
          const int row = u >> 7, col = (u & 127) * 4;
          const int ml = i * 16 + row;
          if (ml >= rows || col >= n_items * 64) continue;
          const int orow = orows[ml];
          *reinterpret_cast<f32x4_t*>(a.y_perm + static_cast<size_t>(orow) * H +
                                      nt * (kWideItems * 64) + col) =
              *reinterpret_cast<const f32x4_t*>(st + row * kStageLd + col);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

}  // namespace

int gemm_tile_rows() { return 128; }

bool gemm_supported(const GroupedArgs& a) {
  return a.packed && a.w_kind == 1 && a.dense_n == 0 && a.w_slot == nullptr &&
         a.H % 64 == 0 && a.I % 32 == 0 && a.num_cu >= kXcds;
}

hipError_t launch_gemm(const GroupedArgs& a, hipStream_t stream, int which) {
  const int grid = (a.num_cu / kXcds) * kXcds;  // one work-group per CU
  if (which != 2) gemm_kernel<true><<<grid, 512, 0, stream>>>(a);
  if (which != 1) gemm_kernel<false><<<grid, 512, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace amoe
