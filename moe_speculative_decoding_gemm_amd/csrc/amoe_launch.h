// Host-side launchers of the AcceptMoE kernels (one per kernel family).
// Called only by capi.cpp after it has validated every argument; each
// launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// the C ABI's structs (include/acceptmoe.h)
struct acceptmoe_shape;
struct acceptmoe_inputs;
struct acceptmoe_outputs;

namespace amoe {

struct SelectArgs {
  int N, H, E, k, n_depth, min_set, fixed_budget, reroute_budget;
  uint32_t flags;
  int act_bf16;  // 1: x and w_router are bf16, 0: fp32
  const void* x;
  const void* w_router;
  const float* b_router;
  const float* logits_in;
  const int32_t* parent;
  const int32_t* depth;
  const float* commit;
  const uint8_t* resident;
  float* logits_out;  // may be null
  uint8_t* eligible;
  int32_t* topk_idx;
  float* topk_gate;
  void* stats;  // acceptmoe_stats*
  // workspace carve-up
  float* part;         // [ksplit][N][E] router partial sums
  int ksplit;
  int kslice;
  float* logits;       // [N][E]
  float* node_m;       // [N] row max of the logits
  double* node_z;      // [N] softmax denominator
  int32_t* nat_idx;    // [N][k] natural top-k experts, slot order
  float* nat_logit;    // [N][k] their logits
  double* d_part;      // [E][groups, padded] demand summed over each 4-node group
  uint8_t* f_part;     // [E][groups, padded] bit 0: a root routes to the expert, bit 1: some node does
  int32_t* e_part;     // [groups] error bits of each node group
  int32_t* counters;   // [2]: [0] arrivals seen outside their range, [1] the grouping's
                       // arrivals (N > 256; zero between kernels)
  int32_t* gcount;     // [N/4]: K-slice arrivals per node group (zero between calls)
  int32_t* ghist;      // [ceil(N*k / 1024)][E]: per-chunk expert counts of the grouping (N > 256)
  // when non-null, the restricted top-k is followed by the grouping of the
  // assignments by expert (moe_route_permute's outputs)
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_assign;
  int32_t* inv_pos;
  int32_t* active;
  int32_t* n_active;
  int32_t* max_rows;  // or null: the most rows routed to one expert
  int32_t* groups;    // or null: the active experts' 64-row groups (see permute_block)
  int32_t* active_w;  // or null: the active experts in work order (see permute_block)
  int group_shift;    // the groups table lists (1 << group_shift)-row groups (6 .. 8)
  // when >= 0 (split mode): experts with more than split_rows routed rows go
  // to the groups table as (1 << group_shift)-row groups for launch_gemm,
  // the others to active_w, their number to n_work[0] (see permute_block);
  // -1: off
  int split_rows;
  int32_t* n_work;
};

// router product, per-node softmax / natural top-k / demand terms, set
// selection, restricted top-k, gates (and the grouping when counts is set)
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
void select_plan(int N, int H, int E, int num_cu, int* ksplit, int* kslice);
int node_workgroups(int N, int E);  // node groups of the front kernel
int group_chunks(int N, int k);  // chunks of the grouping for N > 256 (rows of ghist)
size_t dpart_elems(int N, int E);  // doubles of d_part (expert-major rows of group partials)
size_t fpart_bytes(int N, int E);  // bytes of f_part (same rows)

// grouping of the N*k assignments by expert; resident/stats may be null
hipError_t launch_permute(int N, int k, int E, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_assign, int32_t* inv_pos,
                          int32_t* active, int32_t* n_active, const uint8_t* resident,
                          void* stats, hipStream_t stream);

// w_kind: 0 fp32, 1 bf16, 2 fp8 e4m3fn (+ scales); act_bf16 as above
struct GroupedArgs {
  int N, k, E, H, I;
  int w_kind;
  int act_bf16;
  const void* x;
  const void* w13;
  const void* w2;
  const float* s13;
  const float* s2;
  const int32_t* offsets;
  const int32_t* sorted_assign;
  const int32_t* active;
  const int32_t* n_active;
  float* y_perm;
  void* h_perm;  // [N*k][I] bf16 (fp32 when w_kind == 0)
  int num_cu;
  int packed;    // w13 / w2 are in the packed layout (pack_experts)
  // bf16 / fp8 down projection: write the output of routed row t to row
  // sorted_assign[t] of y_perm (token-major assignment order, i*k + j)
  // instead of row t
  int tok_rows;
  // bf16 / fp8: work units per item (>= 1).  Unit r of an item runs its
  // routed-row groups r, r + row_groups, ... (64 rows each), so an expert
  // with many rows (the shared expert: all N tokens) spreads over more
  // work-groups; the units of one item read the same weights at the same
  // time.
  int row_groups;
  // bf16 / fp8: when set, expert e's weights are entry w_slot[e] of w13 / w2
  // (an expert cache of n_wslots device slots; an entry outside them is
  // clamped, so a bad table cannot send a load out of the buffers); FP8
  // scales stay indexed by e
  const int32_t* w_slot;
  int n_wslots;
  // when both are set and some expert has more than 64 routed rows: the
  // work units are (64-row group, item) pairs from the groups table, so an
  // expert with many rows spreads its row groups over as many units, which
  // read the item's weights at about the same time
  const int32_t* max_rows;
  const int32_t* groups;
  // bf16 / fp8: the active list is in work order (heaviest cost class first,
  // see permute_block): a grid of whole rounds of one work-group per CU
  // deals the items in a snake over the rounds
  int snake;
  // packed bf16 / fp8: GEMM tiling for many rows per expert (two 64-row
  // items per work-group, up to 128 routed rows a pass; the groups table, if
  // used, then lists 128-row groups)
  int gemm;
  // packed bf16: the groups table for launch_gemm (gemm_tile_rows()-row
  // groups of the experts with more than 64 routed rows, (expert << 16) |
  // group, see permute_block)
  const int32_t* gemm_groups;
  // bf16 / fp8, when > 0: dense mode -- dense_n experts (active[0..dense_n),
  // or 0..dense_n-1 when active is null; offsets, sorted_assign and
  // n_active unused) each over all N rows: row m of expert u is node m's x,
  // written to row u*N + m of h_perm and y_perm
  int dense_n;
};
// which: 0 both projections, 1 gate/up only, 2 down only
hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream, int which = 0);

// The tiled grouped GEMM (gemm.hip) over a.gemm_groups: packed bf16
// weights only (gemm_supported).  which as above.
bool gemm_supported(const GroupedArgs& a);
int gemm_tile_rows();  // routed rows per GEMM tile (the groups table's group size)
hipError_t launch_gemm(const GroupedArgs& a, hipStream_t stream, int which = 0);

// Packed expert layout (bf16 / fp8 weights): see grouped.hip.  which: 0 for
// w13 ([E,2,I,H] -> packed), 1 for w2 ([E,H,I] -> packed).
size_t packed_bytes(int which, int w_kind, int E, int H, int I);
hipError_t launch_pack(int which, int w_kind, int E, int H, int I, const void* src, void* dst,
                       hipStream_t stream);

struct CombineArgs {
  int N, k, H, act_bf16;
  const float* y_perm;
  const int32_t* inv_pos;  // nullptr: y_perm rows are in token-major order (i*k + j)
  const float* gate;       // [N][k]
  const float* y_shared;   // [N][H] or nullptr
  void* y;                 // [N][H] act dtype
};
hipError_t launch_combine(const CombineArgs& c, hipStream_t stream);

// identity grouping for the shared expert: offsets {0,N}, sorted_assign 0..N-1,
// active {0}, n_active {1}
hipError_t launch_shared_grouping(int N, int32_t* offsets, int32_t* sorted_assign,
                                  int32_t* active, int32_t* n_active, hipStream_t stream);

// Host helpers of capi.cpp for other entry points of the library.
// check_verify_args: verify_block's argument checks (return code as the C
// ABI's, detail in acceptmoe_last_error) and the workspace bytes it needs.
// workspace_counter_bytes: the leading bytes of every workspace that hold
// the kernels' arrival counters (zero between calls).  set_error: record a
// detail string, return `code`.
int check_verify_args(const ::acceptmoe_shape* s, const ::acceptmoe_inputs* in,
                      const ::acceptmoe_outputs* out, size_t* need);
size_t workspace_counter_bytes();
int set_error(int code, const char* msg);

}  // namespace amoe
