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
// 4 waves of 128 x 128 (8 x 8 MFMA tiles of 16 x 16, the accumulators in the
// accumulation registers).
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

// Wave w owns items 2 w, 2 w + 1 of the tile.  A wave's weight fragments
// are its own: they go from memory straight to registers, three steps ahead,
// with no barrier.  Only the activation fragments are shared: an 8-slot LDS ring
// filled by direct loads five steps ahead (each wave 2 of the 8 fragments of
// a step), read one step ahead into a second register set, so that the reads
// of step s + 1 overlap the MFMAs of step s.  A barrier every second step
// orders the ring.  The memory counter drains in order: waiting for the
// activations of steps s + 1, s + 2 (loaded at steps s - 4, s - 3) also
// waits for the weights loaded before them, which are those of steps up to
// s -- so the weights keep their three steps.

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


// Two rows of 8 MFMAs (activation fragments a0, a1 against the 8 weight
// fragments b) with two fragment reads of the next step (at lds + off0,
// off1) issued in front of them and waited for at the end of the same
// statement.  Written out so that the reads, and the loads the caller puts
// between these statements, go out spread over the step's MFMAs: issued as
// one burst after the barrier they hold up the MFMAs behind them.
template <int OFF0, int OFF1>
__device__ __forceinline__ void mfma_rows2(f32x4_t (&c0)[8], f32x4_t (&c1)[8], const u32x4_t& a0,
                                           const u32x4_t& a1, const u32x4_t (&b)[8], uint32_t lds,
                                           u32x4_t& r0, u32x4_t& r1) {
  asm volatile(
      "ds_read_b128 %[r0], %[la] offset:%[o0]\n\t"
      "ds_read_b128 %[r1], %[la] offset:%[o1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c02], %[a0], %[b2], %[c02]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c03], %[a0], %[b3], %[c03]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c04], %[a0], %[b4], %[c04]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c05], %[a0], %[b5], %[c05]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c06], %[a0], %[b6], %[c06]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c07], %[a0], %[b7], %[c07]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c12], %[a1], %[b2], %[c12]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c13], %[a1], %[b3], %[c13]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c14], %[a1], %[b4], %[c14]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c15], %[a1], %[b5], %[c15]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c16], %[a1], %[b6], %[c16]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c17], %[a1], %[b7], %[c17]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [c00] "+a"(c0[0]), [c01] "+a"(c0[1]), [c02] "+a"(c0[2]), [c03] "+a"(c0[3]),
        [c04] "+a"(c0[4]), [c05] "+a"(c0[5]), [c06] "+a"(c0[6]), [c07] "+a"(c0[7]),
        [c10] "+a"(c1[0]), [c11] "+a"(c1[1]), [c12] "+a"(c1[2]), [c13] "+a"(c1[3]),
        [c14] "+a"(c1[4]), [c15] "+a"(c1[5]), [c16] "+a"(c1[6]), [c17] "+a"(c1[7]),
        [r0] "=&v"(r0), [r1] "=&v"(r1)
      : [a0] "v"(a0), [a1] "v"(a1), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]),
        [b3] "v"(b[3]), [b4] "v"(b[4]), [b5] "v"(b[5]), [b6] "v"(b[6]), [b7] "v"(b[7]),
        [la] "v"(lds), [o0] "i"(OFF0), [o1] "i"(OFF1)
      : "memory");
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GroupedArgs a) {
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

    // activation fragments 2 wave, 2 wave + 1 of each step (rows past the
    // group's read its first row); this wave's weight items (past the
    // expert's: its last item, loaded and never used)
    const uint16_t* arow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int mt = 2 * wave + i;
      const int m = mt * 16 + r < rows ? mt * 16 + r : 0;
      const int srow = GATEUP ? a.sorted_assign[off + m] / k : off + m;
      arow[i] = src + static_cast<size_t>(srow) * src_ld + 8 * g;
    }
    const uint16_t* bsrc[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int item = min(nt * kWideItems + 2 * wave + ii, items - 1);
      bsrc[ii] = wts + (static_cast<size_t>(e) * items + item) * nsteps * kStepElems + lane * 8;
    }
    const bool busy = 2 * wave < n_items;
    // the output row of routed row t of the group (down), for the epilogue
    int orow_t = 0;
    if (!GATEUP && t < rows) orow_t = a.tok_rows ? a.sorted_assign[off + t] : off + t;

    // loads past the last step load the last step again (never read)
    auto issue_a = [&](int s) {
      u32x4_t* dst = ring + (s % kWideSlots) * kASlotElems;
      // activation elements past K: the last 8 of the row (their weights are 0)
      const int kk = min(min(s, nsteps - 1) * 32, K - 8 - 8 * g);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        frag_load(arow[i] + kk, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                                         (lds_void*)(dst + (2 * wave + i) * 64))));
    };
    u32x4_t bset[4][8];
    auto load_b = [&](int s, u32x4_t(&bv)[8]) {
      const size_t so = static_cast<size_t>(min(s, nsteps - 1)) * kStepElems;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        bv[q] = *reinterpret_cast<const u32x4_t*>(bsrc[q >> 2] + so + (q & 3) * kFragElems);
    };
    u32x4_t areg[2][8];
    auto read_a = [&](int s, u32x4_t(&av)[8]) {
      const u32x4_t* sl = ring + (s % kWideSlots) * kASlotElems;
#pragma unroll
      for (int i = 0; i < 8; ++i) av[i] = sl[i * 64 + lane];
    };
    f32x4_t acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Step s (slot s mod 8, weight set s mod 4, activation registers s mod
    // 2) computes with the fragments read during step s - 1 and reads those
    // of step s + 1.  At the last step the reads are of a step that does not
    // exist (the slot holds stale data, never used).
    const uint32_t ring_lds =
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)ring)) + lane * 16;
    auto load_b2 = [&](int s, u32x4_t(&bv)[8], int q0) {
      const size_t so = static_cast<size_t>(min(s, nsteps - 1)) * kStepElems;
#pragma unroll
      for (int q = q0; q < q0 + 2; ++q)
        bv[q] = *reinterpret_cast<const u32x4_t*>(bsrc[q >> 2] + so + (q & 3) * kFragElems);
    };
    // Every wave computes (one whose items are past the expert's works on
    // the clamped weights; its results are not written).  The next step's
    // fragment reads go out two per 16 MFMAs, the weight loads of step s + 3
    // two between each 16.
    auto step = [&](int s, auto rc) {
      constexpr int R = decltype(rc)::value;
      // Every second step: this wave's activation loads of steps s + 1 and
      // s + 2 are done -- the later of them went out at step s - 3 after two
      // weight loads, so the other 6 of that step and the 10 loads of each
      // of steps s - 2, s - 1 may still be in flight -- and then the barrier:
      // every wave is past step s - 1, so the slots of steps s - 3 and s - 2
      // (read at steps s - 4 and s - 3) take the loads of steps s + 5, s + 6.
      if ((R & 1) == 0) ring_barrier<6 + 2 * 10>();
      const uint32_t la = ring_lds + ((s + 1) % kWideSlots) * (kASlotElems * 16);
      u32x4_t(&an)[8] = areg[(R + 1) & 1];
      const u32x4_t(&ac)[8] = areg[R & 1];
      const u32x4_t(&bc)[8] = bset[R & 3];
      u32x4_t(&bn)[8] = bset[(R + kBAhead) & 3];
      mfma_rows2<0, 1024>(acc[0], acc[1], ac[0], ac[1], bc, la, an[0], an[1]);
      load_b2(s + kBAhead, bn, 0);
      issue_a(s + kAAhead);
      mfma_rows2<2048, 3072>(acc[2], acc[3], ac[2], ac[3], bc, la, an[2], an[3]);
      load_b2(s + kBAhead, bn, 2);
      mfma_rows2<4096, 5120>(acc[4], acc[5], ac[4], ac[5], bc, la, an[4], an[5]);
      load_b2(s + kBAhead, bn, 4);
      mfma_rows2<6144, 7168>(acc[6], acc[7], ac[6], ac[7], bc, la, an[6], an[7]);
      load_b2(s + kBAhead, bn, 6);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
#pragma unroll
    for (int p = 0; p < kAAhead; ++p) issue_a(p);
    asm volatile("" ::: "memory");  // the activation loads go out first
#pragma unroll
    for (int p = 0; p < kBAhead; ++p) load_b(p, bset[p]);
    ring_barrier<8 * kBAhead>();  // the first steps' activations are in LDS
    read_a(0, areg[0]);
    for (int s = 0; s < nsteps; s += 4) {
      step(s, C0{});
      step(s + 1, C1{});
      step(s + 2, C2{});
      step(s + 3, C3{});
    }
    // the last MFMAs' results settle before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue, one 16-row slab of the tile at a time through LDS (two
    // buffers): the waves write their accumulators (lane (r, g) holds
    // D[4g + jj][r] of each 16 x 16 tile), then the work-group writes whole
    // row segments with 16-byte stores -- down: the fp32 rows; gate/up: the
    // SwiGLU of each 16-column tile's gate (columns 0..7) and up (8..15)
    // halves, 8 bf16 of h per store.  Columns of items past the expert's
    // are not written.
    // (the thread index taken afresh: addresses derived from it are not
    // hoisted out of the unit loop to stay live, in spilled registers,
    // across the main loop)
    int te = t;
    asm volatile("" : "+v"(te));
    const int re = te & 15, ge = (te >> 4) & 3, we = te >> 6;
    if (!GATEUP && te < 128) orows[te] = orow_t;  // read after the first slab's barrier
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i * 16 >= rows) break;
      float* st = stage + (i & 1) * (16 * kStageLd);
      if (busy) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            st[(4 * ge + jj) * kStageLd + we * 128 + q * 16 + re] = acc[i][q][jj];
      }
      // the slab is in LDS (the stores of the last slab may still be in flight)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (GATEUP) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int u = it * 256 + te;
          const int row = u >> 5, tile = u & 31;  // 16-column tile of the work-group's
          const int ml = i * 16 + row;
          if (ml >= rows || (tile >> 2) >= n_items) continue;
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
          const int qq = nt * (kWideItems * 4) + tile;  // 16-row tile of the expert
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.h_perm) +
                                      static_cast<size_t>(off + ml) * I + 8 * qq) = hv;
        }
      } else {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int u = it * 256 + te;
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
    // every wave is done with the ring before the next unit's loads
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
  if (which != 2) gemm_kernel<true><<<grid, 256, 0, stream>>>(a);
  if (which != 1) gemm_kernel<false><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace amoe
