// Grouped GEMM for the experts that many routed rows reach, on gfx950
// matrix cores (bf16 weights in the packed layout, bf16 activations).
//
// [MoESD §5.1-§5.2]: as the verification batch grows, the active experts
// saturate and the routed rows per active expert keep growing, so an
// expert's FLOPs per weight byte grow with the batch until the layer turns
// from memory-bound to compute-bound.  The streaming expert kernels
// (grouped.hip) keep at most 128 routed rows per pass over an expert's
// weights; here a work-group holds a 128 x 256 output tile -- 128 routed rows
// of one expert against 256 weight rows (4 packed items) -- and two
// work-groups share each CU (kWaveRows = 2: one 256 x 256 tile per CU).
//
// Operands go from memory to LDS with gfx950's direct loads
// (global_load_lds_dwordx4: 16 B per lane, no registers in between), already
// in MFMA fragment order: one wave load instruction fills one 1 KB fragment
// (lane l's 16 B at byte 16 l), so each fragment read is one conflict-free
// ds_read_b128 per lane.  A ring of 32-long reduction steps (one slot: the
// tile's activation fragments, then its 16 weight fragments) keeps NS - 1
// steps in flight.
//
// Waves as kWaveRows x 4: wave (wm, wn) owns routed rows 128 wm .. +127 and
// weight rows 64 wn .. +63 (one packed item) of the tile, 8 x 4 MFMA tiles of
// 16 x 16.  Every output element takes the same v_mfma_f32_16x16x32_bf16
// sequence over the same reduction steps (activation elements past K clamped
// the same way) as in the streaming kernels, so the results are the same bits.
//
// Work units: (row group of an expert, 256-column tile), group-major, from
// the groups table that the grouping writes for these experts.  The grid
// is every work-group slot of the GPU; work-group b runs on XCD b mod 8, so
// XCD x takes the contiguous unit range x * span .. and its CUs work on
// neighbouring units at the same time: the column tiles of one row group
// share its activation rows, and the row groups of one expert share the
// weights, in that XCD's L2.

#include "amoe_common.h"
#include "amoe_launch.h"

namespace amoe {

namespace {

constexpr int kTileItems = 4;                 // packed 64-row weight items per tile
constexpr int kFragBytes = 1024;              // one MFMA operand fragment: 64 lanes x 16 B
constexpr int kFragElems = 512;               // bf16 elements of one fragment
constexpr int kStepElems = 4 * kFragElems;    // one 32-long step of one packed item
constexpr int kXcds = 8;
// tile height in 128-row wave rows: 2 (256 rows, 8 waves, one work-group
// per CU) or 1 (128 rows, 4 waves, two work-groups per CU)
constexpr int kWaveRows = 1;
// ring slots: 4 x 32 KB (one work-group per CU) or 3 x 24 KB (two per CU)
constexpr int kRingSlots = kWaveRows == 2 ? 4 : 3;

// one 16-byte direct load per lane into the wave's 1 KB fragment at `frag`
// in LDS (lane l's bytes land at frag + 16 l)
using lds_void = __attribute__((address_space(3))) void;
__device__ __forceinline__ void frag_load(const void* src, lds_void* frag) {
  __builtin_amdgcn_global_load_lds(src, frag, 16, 0, 0);
}

// This wave's ring loads older than its last VM are in LDS and its LDS reads
// have returned; then the work-group barrier.  The memory clobber keeps the
// compiler from moving LDS reads across it.  (__syncthreads would also wait
// for the loads still in flight for later steps.)
template <int VM>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// The 8 activation fragments and 4 weight fragments one wave uses in a
// step: ds_read_b128 at a (+ 1 KB each) and b (+ 1 KB each), LDS byte
// addresses, and the wait for all of them in the same statement.  Written
// out because the compiler cannot tell which ring slot a direct load fills:
// before its own LDS reads it would wait for every load in flight, also
// those of later steps (ring_barrier orders the ring instead).
// Early-clobber outputs: no result register may share a register with an
// address.
__device__ __forceinline__ void read_frags(uint32_t a, uint32_t b, u32x4_t (&av)[8],
                                           u32x4_t (&bv)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\t"
      "ds_read_b128 %3, %12 offset:3072\n\t"
      "ds_read_b128 %4, %12 offset:4096\n\t"
      "ds_read_b128 %5, %12 offset:5120\n\t"
      "ds_read_b128 %6, %12 offset:6144\n\t"
      "ds_read_b128 %7, %12 offset:7168\n\t"
      "ds_read_b128 %8, %13\n\t"
      "ds_read_b128 %9, %13 offset:1024\n\t"
      "ds_read_b128 %10, %13 offset:2048\n\t"
      "ds_read_b128 %11, %13 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(av[0]), "=&v"(av[1]), "=&v"(av[2]), "=&v"(av[3]), "=&v"(av[4]), "=&v"(av[5]),
        "=&v"(av[6]), "=&v"(av[7]), "=&v"(bv[0]), "=&v"(bv[1]), "=&v"(bv[2]), "=&v"(bv[3])
      : "v"(a), "v"(b)
      : "memory");
}

// LDS byte address of the ring
template <int NB>
__device__ __forceinline__ uint32_t lds_addr(const uint8_t (&ring)[NB]) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) uint8_t*)&ring[0]));
}

template <bool GATEUP, int WR, int NS>
__global__ __launch_bounds__(256 * WR, 2 / WR) void gemm_kernel(GroupedArgs a) {
  // tile: 128 WR routed rows x 256 weight rows, 4 WR waves; per step the
  // slot holds 8 WR activation fragments, then 16 weight fragments
  constexpr int kAF = 8 * WR;                       // activation fragments per step
  constexpr int kBW = 16 / (4 * WR);                // weight fragments each wave loads
  constexpr int kLoads = 2 + kBW;                   // ring loads per wave per step
  constexpr int kSlot = (kAF + 16) * kFragBytes;    // bytes of one slot
  // NS slots of one 32-long step each: NS - 1 steps in flight
  __shared__ __attribute__((aligned(kFragBytes))) uint8_t ring[NS * kSlot];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;
  const int H = a.H, I = a.I, k = a.k;
  const int K = GATEUP ? H : I;
  // packed weights come in 128-long chunks, zero-padded: every step is computed
  const int nsteps = ((K + 127) >> 7) * 4;
  const int items = (GATEUP ? 2 * I : H) >> 6;
  const int ntiles = (items + kTileItems - 1) / kTileItems;
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
    const int m0 = (gv & 0xffff) * (128 * WR);
    const int off = a.offsets[e] + m0;
    const int rows = min(128 * WR, a.offsets[e + 1] - off);
    const int n_items = min(kTileItems, items - nt * kTileItems);

    // This lane's part of the ring loads: activation fragments (row tiles)
    // 2 wave and 2 wave + 1, weight fragments kBW wave .. + kBW - 1 (item
    // f / 4 of the tile, 16-row tile f % 4).  Rows past the group's read its
    // first row, items past the expert's its last item: loaded, never stored.
    const uint16_t* arow[2];
    const uint16_t* bsrc[kBW];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int mt = 2 * wave + i;
      const int m = mt * 16 + r < rows ? mt * 16 + r : 0;
      const int srow = GATEUP ? a.sorted_assign[off + m] / k : off + m;
      arow[i] = src + static_cast<size_t>(srow) * src_ld + 8 * g;
    }
#pragma unroll
    for (int i = 0; i < kBW; ++i) {
      const int f = kBW * wave + i;
      const int item = min(nt * kTileItems + (f >> 2), items - 1);
      bsrc[i] = wts + (static_cast<size_t>(e) * items + item) * nsteps * kStepElems +
                (f & 3) * kFragElems + lane * 8;
    }
    auto issue = [&](int s) {
      const int at = (s % NS) * kSlot;
      // activation elements past K: the last 8 of the row (their weights are 0)
      const int kk = min(s * 32, K - 8 - 8 * g);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        frag_load(arow[i] + kk, (lds_void*)&ring[at + (2 * wave + i) * kFragBytes]);
#pragma unroll
      for (int i = 0; i < kBW; ++i)
        frag_load(bsrc[i] + static_cast<size_t>(s) * kStepElems,
                  (lds_void*)&ring[at + (kAF + kBW * wave + i) * kFragBytes]);
    };

    // this wave's row tiles that hold routed rows, and whether its item exists
    const int mt_n = min(8, max(0, (rows - wm * 128 + 15) >> 4));
    const bool busy = mt_n > 0 && wn < n_items;
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this lane's byte offsets of its fragments within a slot
    const uint32_t a_off = (wm * 8) * kFragBytes + lane * 16;
    const uint32_t b_off = (kAF + wn * 4) * kFragBytes + lane * 16;
    const uint32_t ring_base = lds_addr(ring);
    auto compute = [&](int s) {
      if (!busy) return;
      u32x4_t av[8], bv[4];
      const uint32_t base = ring_base + (s % NS) * kSlot;
      read_frags(base + a_off, base + b_off, av, bv);
      // only the row tiles that hold routed rows
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= mt_n) break;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[i]),
                                                              __builtin_bit_cast(bf16x8_t, bv[q]),
                                                              acc[i][q], 0, 0, 0);
      }
    };
    // Steps 0 .. NS-2 go out first; step s then waits for its own loads
    // (kLoads per wave: the loads of the up to NS-2 steps issued after it
    // stay in flight), and the barrier frees the slot of step s - 1 for step
    // s + NS - 1.  nsteps >= 4 >= NS - 1.
    constexpr int kAhead = NS - 1;
    static_assert(kAhead <= 4, "at most four steps in flight");
#pragma unroll
    for (int p = 0; p < kAhead; ++p) issue(p);
    for (int s = 0; s < nsteps; ++s) {
      const int later = min(kAhead - 1, nsteps - 1 - s);  // steps issued after s
      if (later >= 3)
        ring_barrier<3 * kLoads>();
      else if (later == 2)
        ring_barrier<2 * kLoads>();
      else if (later == 1)
        ring_barrier<kLoads>();
      else
        ring_barrier<0>();
      if (s + kAhead < nsteps) issue(s + kAhead);
      compute(s);
    }

    // epilogue: lane (r, g) holds D[m = 4g + jj][n = r] of each 16 x 16 tile
    // (the ring is free for the next unit: its first loads go to the slots
    // of the last unit's steps nsteps-4 .. nsteps-2, which every wave has
    // finished with at the last barrier)
    if (busy) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= mt_n) break;
        int orow[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int ml = (wm * 8 + i) * 16 + 4 * g + jj;
          orow[jj] = -1;
          if (ml < rows) orow[jj] = (!GATEUP && a.tok_rows) ? a.sorted_assign[off + ml] : off + ml;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int qq = (nt * kTileItems + wn) * 4 + q;  // 16-row tile of the expert
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float v = acc[i][q][jj];
            if (GATEUP) {
              // tile qq: gate rows 8 qq .. +7 in columns 0..7, up rows in 8..15
              const float up = __shfl_xor(v, 8, kWave);
              if (r < 8 && orow[jj] >= 0)
                static_cast<uint16_t*>(a.h_perm)[static_cast<size_t>(orow[jj]) * I + 8 * qq + r] =
                    f32_to_bf16(silu(v) * up);
            } else if (orow[jj] >= 0) {
              a.y_perm[static_cast<size_t>(orow[jj]) * H + qq * 16 + r] = v;
            }
          }
        }
      }
    }
  }
}

}  // namespace

int gemm_tile_rows() { return 128 * kWaveRows; }

bool gemm_supported(const GroupedArgs& a) {
  return a.packed && a.w_kind == 1 && a.dense_n == 0 && a.w_slot == nullptr &&
         a.H % 64 == 0 && a.I % 32 == 0 && a.num_cu >= kXcds;
}

hipError_t launch_gemm(const GroupedArgs& a, hipStream_t stream, int which) {
  const int grid = (a.num_cu / kXcds) * kXcds * (2 / kWaveRows);
  if (which != 2) gemm_kernel<true, kWaveRows, kRingSlots><<<grid, 256 * kWaveRows, 0, stream>>>(a);
  if (which != 1) gemm_kernel<false, kWaveRows, kRingSlots><<<grid, 256 * kWaveRows, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace amoe
