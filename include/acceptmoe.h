/*
 * acceptmoe.h -- C ABI of the AcceptMoE verify-block MoE layer for MI355X (gfx950).
 *
 * One MoE layer forward over one speculative-decoding verification block: a
 * draft tree (or a forest of trees for batched verification) of N nodes.
 * Sources, cited per entry point below:
 *   [AcceptMoE news]     news article on AcceptMoE (Imperial College London /
 *                        Tile-AI), sections 01-04
 *   [AcceptMoE abstract] arXiv 2608.02989, English abstract
 *   [MoE-SD blog]        "MoE 与推测解码：计算、通信和接受率的联合优化"
 *                        (charlestar.github.io): the single-GPU MoE layer pipeline
 *   [EcoSpec]            arXiv 2607.12696, Figure 1 (latency linear in active
 *                        experts; 44.04 MB per FP8 DeepSeek-V3.1 expert)
 *
 * Conventions shared by every entry point
 *   - Arrays are dense, row-major, and live in DEVICE memory unless a comment
 *     says "host".  The caller owns every buffer; the library allocates no
 *     memory and keeps no state between calls (it is reentrant).
 *   - All work is enqueued on the caller's stream; nothing synchronises and
 *     nothing reads device memory on the host, so every call may be captured
 *     in a hipGraph.
 *   - Return value: 0 on success or a negative ACCEPTMOE_E* code, decided on
 *     the host before anything is enqueued (except ACCEPTMOE_EHIP, a failed
 *     launch).  acceptmoe_last_error() gives a detail string for the calling
 *     thread.  Problems only the device can see (a malformed tree, a depth
 *     out of range, a bad commitment table, a non-finite logit) set bits in
 *     acceptmoe_stats.err_flags; the other outputs are then unspecified but
 *     every index the library writes stays in range.
 *   - dtype pairs (activations, expert weights): (F32, F32), (BF16, BF16),
 *     (BF16, FP8_E4M3FN).  FP8 weights come with one fp32 scale per 128 x 128
 *     block of each [out, in] matrix: w = decode(q) * s.
 *   - Limits: 1 <= N <= 4096, 1 <= k <= 16, k <= E <= 256, H and I multiples
 *     of 64 (128 with FP8 weights), H, I <= 16384.
 */
#ifndef ACCEPTMOE_H
#define ACCEPTMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ACCEPTMOE_OK = 0,
  ACCEPTMOE_EINVAL = -1,  /* a bad argument: NULL, out-of-range size, small workspace */
  ACCEPTMOE_ENOTSUP = -2, /* an unsupported dtype pair or flag                        */
  ACCEPTMOE_EHIP = -3     /* a kernel launch failed (hipGetLastError)                 */
};

typedef enum {
  ACCEPTMOE_F32 = 0,
  ACCEPTMOE_BF16 = 1,
  ACCEPTMOE_FP8_E4M3FN = 2
} acceptmoe_dtype;

/* Layout of the expert weights (w13, w2 and the shared expert's). */
typedef enum {
  ACCEPTMOE_LAYOUT_ROWMAJOR = 0, /* w13 [E,2,I,H], w2 [E,H,I] as documented below            */
  ACCEPTMOE_LAYOUT_PACKED = 1    /* reordered once by acceptmoe_pack_experts (BF16 / FP8 only) */
} acceptmoe_layout;

enum {
  ACCEPTMOE_F_NATURAL = 1u << 0,   /* every expert eligible: natural routing (standard SD) */
  ACCEPTMOE_F_NO_RENORM = 1u << 1, /* gates = raw softmax scores of the chosen experts     */
  ACCEPTMOE_F_LOGITS_IN = 1u << 2, /* read logits_in instead of computing x W_r^T + b_r    */
  /* Selector variants on the same kernels ([AcceptMoE news §01, §04]).
   * MoE-Spec keeps a fixed number B of the highest-ranked experts and weighs
   * every draft position alike: F_UNIT_COMMIT | F_NO_ANCHOR with
   * fixed_budget = B.  AcceptMoE-B: fixed_budget = B alone.               */
  ACCEPTMOE_F_DEMAND_FULL = 1u << 3, /* demand sums every expert's score, not only each node's
                                        natural top-k                                       */
  ACCEPTMOE_F_NO_ANCHOR = 1u << 4,   /* no root anchor                                       */
  ACCEPTMOE_F_UNIT_COMMIT = 1u << 5  /* every draft position weighs 1 (commit table ignored
                                        for the demand; still validated)                    */
};

/* bits of acceptmoe_stats.err_flags */
enum {
  ACCEPTMOE_ERR_BAD_TREE = 1u << 0,  /* parent not an earlier node, or depth != parent's + 1 */
  ACCEPTMOE_ERR_DEPTH = 1u << 1,     /* depth outside [0, n_depth)                          */
  ACCEPTMOE_ERR_NONFINITE = 1u << 2, /* a router logit is NaN or infinite                   */
  ACCEPTMOE_ERR_COMMIT = 1u << 3,    /* a commitment probability is negative or not finite  */
  ACCEPTMOE_ERR_WORKSPACE = 1u << 4  /* an arrival counter of the workspace was not zero at
                                        the start of the call (not zero-filled before its
                                        first use, or shared by calls that overlap); the
                                        counters are zero again afterwards                 */
};

/* Problem description; passed by HOST pointer and read during the call. */
typedef struct acceptmoe_shape {
  int32_t N;              /* verify nodes (all trees of the block)                         */
  int32_t H;              /* hidden size                                                   */
  int32_t I;              /* expert intermediate size                                      */
  int32_t E;              /* routed experts                                                */
  int32_t k;              /* experts per node                                              */
  int32_t n_depth;        /* entries of commit[]                                           */
  int32_t min_set;        /* smallest eligible set; the floor is max(k, min_set)           */
  int32_t fixed_budget;   /* 0: self-size (AcceptMoE); B > 0: set size B (AcceptMoE-B)     */
  int32_t reroute_budget; /* R: most experts residency-aware pruning may drop              */
  uint32_t flags;         /* ACCEPTMOE_F_*                                                 */
  int32_t act_dtype;      /* acceptmoe_dtype of x, w_router and y                          */
  int32_t w_dtype;        /* acceptmoe_dtype of the expert weights                         */
  int32_t w_layout;       /* acceptmoe_layout of the expert weights                        */
} acceptmoe_shape;

/* Per-block statistics, written by the device. */
typedef struct acceptmoe_stats {
  int32_t n_anchor;             /* |A|: experts in the roots' natural top-k               */
  int32_t n_selfsize;           /* |S| after self-sizing, before pruning                  */
  int32_t n_eligible;           /* |S| after pruning                                       */
  int32_t n_pruned;             /* experts removed by residency-aware pruning              */
  int32_t n_active;             /* U: unique experts of the restricted assignments         */
  int32_t n_active_nonresident; /* of those, not resident (0 without a mask)               */
  int32_t n_natural_union;      /* unique experts of the natural top-k assignments         */
  int32_t err_flags;            /* ACCEPTMOE_ERR_* bits                                    */
  double r_eff;                 /* effective rank exp(H(D / sum D)); 0 if sum D = 0        */
  double demand_total;          /* sum of D                                               */
} acceptmoe_stats;

/* ---------------------------------------------------------------------------
 * acceptmoe_select -- router, AcceptMoE eligibility, restricted top-k, gates.
 *
 * [MoE-SD blog, MoE layer]: logits l = x W_r^T + b_r; scores p = softmax(l)
 *   over all E experts; each node's natural top-k by l (ties: lower index).
 * [AcceptMoE news §02, abstract]: demand D_e = sum over nodes i of
 *   commit[depth_i] * p_ie for e in node i's natural top-k; anchor A = union of
 *   the roots' natural top-k; set size n = min(E, max(round-half-up(r_eff) or
 *   fixed_budget, |A|, max(k, min_set))) with r_eff = exp(entropy of D/sum D);
 *   S = A + the highest-demand others (ties: lower index).  With a resident
 *   mask, non-resident non-anchor members of S are dropped in (demand
 *   ascending, index descending) order, at most reroute_budget of them, never
 *   below max(k, min_set).
 * [AcceptMoE abstract]: each node's top-k is then taken over S only; gates
 *   are the chosen scores renormalised to sum to one (F_NO_RENORM: raw).
 *
 *   x         [N,H] act_dtype        w_router [E,H] act_dtype
 *   b_router  [E] fp32 or NULL       logits_in [N,E] fp32, used iff F_LOGITS_IN
 *   parent    [N] int32: -1 for a root, else an earlier node index
 *   depth     [N] int32: 0 for a root, parent's depth + 1 otherwise
 *   commit    [n_depth] fp32: commitment probability per depth, >= 0
 *   resident  [E] uint8 (nonzero = resident) or NULL: no pruning
 *   logits_out [N,E] fp32 or NULL    eligible [E] uint8 (1 = in S)
 *   topk_idx  [N,k] int32            topk_gate [N,k] fp32
 *   stats     one acceptmoe_stats (device)
 *   ws        workspace of at least acceptmoe_select_workspace_size(shape) bytes,
 *             device memory owned by the caller.  It holds the kernels'
 *             arrival counters: zero-fill the workspace once before its first
 *             use (hipMemset at allocation); every call leaves the counters
 *             at zero again, so it needs no clearing between calls, also when
 *             the shape changes.  Calls that share a workspace must not
 *             overlap in time (same stream, or synchronised).  A call that
 *             finds a counter not at zero (a workspace not zero-filled, or
 *             shared by overlapping calls) sets ACCEPTMOE_ERR_WORKSPACE in
 *             stats->err_flags -- its other outputs are then unspecified, with
 *             every index in range -- and sets the counters back to zero, so
 *             the next call on that workspace is valid again.
 *   stats->n_active / n_active_nonresident: U and the non-resident part of
 *             it, counted from the restricted top-k (no grouping needed).
 * ------------------------------------------------------------------------- */
size_t acceptmoe_select_workspace_size(const acceptmoe_shape* shape);
int acceptmoe_select(const acceptmoe_shape* shape, const void* x, const void* w_router,
                     const float* b_router, const float* logits_in, const int32_t* parent,
                     const int32_t* depth, const float* commit, const uint8_t* resident,
                     float* logits_out, uint8_t* eligible, int32_t* topk_idx, float* topk_gate,
                     acceptmoe_stats* stats, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_route_permute -- group the N*k assignments by expert.
 *
 * [MoE-SD blog, MoE layer]: assignment a = i*k + j goes to expert
 * topk_idx[a]; counts[e] = assignments of e; offsets[E+1] = exclusive prefix
 * sum of counts; sorted_assign[N*k] = assignment ids stably sorted by expert;
 * inv_pos[sorted_assign[t]] = t; active[0..n_active) = experts with
 * counts > 0, ascending (entries past n_active are left untouched).
 * Every topk_idx entry must lie in [0, E) (an entry outside is clamped into
 * range: no access leaves its buffer, the grouping is then unspecified).
 * The result is deterministic.
 * ------------------------------------------------------------------------- */
int moe_route_permute(int32_t N, int32_t k, int32_t E, const int32_t* topk_idx, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_assign, int32_t* inv_pos,
                      int32_t* active, int32_t* n_active, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_swiglu -- SwiGLU experts over the unique active experts only.
 *
 * [MoE-SD blog, MoE layer; EcoSpec Fig. 1]: for every active expert e and
 * every row t in [offsets[e], offsets[e+1]), with token i = sorted_assign[t]/k:
 *   y_perm[t,:] = (silu(x_i Wg_e^T) * (x_i Wu_e^T)) Wd_e^T
 * Each active expert's weights are streamed from HBM once per group of at most
 * 64 rows.  silu(z) = z / (1 + exp(-z)); the SwiGLU hidden is rounded to bf16
 * before the down projection unless w_dtype is F32.
 *
 *   x   [N,H] act_dtype
 *   w13 [E,2,I,H] w_dtype (gate rows, then up rows)   w2 [E,H,I] w_dtype
 *     (or, with w_layout = PACKED, the buffers acceptmoe_pack_experts wrote)
 *   s13 [E,2,I/128,H/128] fp32, s2 [E,H/128,I/128] fp32: FP8 only, else NULL
 *   offsets [E+1], sorted_assign [N*k], active [E], n_active [1]: as written
 *     by moe_route_permute
 *   y_perm [N*k,H] fp32 (rows of inactive experts are not written)
 *   ws  at least moe_grouped_swiglu_workspace_size(N, k, I, w_dtype) bytes
 * The shared expert of a layer is this call with E = 1, k = 1,
 * offsets = {0, N}, sorted_assign = 0..N-1, active = {0}, n_active = {1}.
 * ------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_workspace_size(int32_t N, int32_t k, int32_t I, int32_t w_dtype);
int moe_grouped_swiglu(int32_t N, int32_t k, int32_t E, int32_t H, int32_t I,
                       int32_t act_dtype, int32_t w_dtype, int32_t w_layout, const void* x,
                       const void* w13,
                       const void* w2, const float* s13, const float* s2,
                       const int32_t* offsets, const int32_t* sorted_assign,
                       const int32_t* active, const int32_t* n_active, float* y_perm,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * acceptmoe_pack_experts -- reorder expert weights into the packed layout.
 *
 * Weights are static, so they can be laid out once in the exact order the
 * gfx950 expert kernels stream them: every load instruction then reads 1 KB
 * of consecutive bytes and every work-group one contiguous region, which
 * keeps HBM near its peak ([EcoSpec, Fig. 1]: verification time is the
 * active experts' weight traffic).  Values are unchanged; the reduction
 * dimension is zero-padded to a multiple of 128.  FP8 scales keep their
 * row-major layout.  BF16 and FP8 weights only.
 *   n_experts  E for the routed experts, 1 for a shared expert
 *   w13 [n,2,I,H], w2 [n,H,I] row-major (device) -> w13_packed, w2_packed of
 *   acceptmoe_packed_size(shape, 0, n) and (shape, 1, n) bytes (device);
 *   either pair may be NULL to pack only the other.
 * ------------------------------------------------------------------------- */
size_t acceptmoe_packed_size(const acceptmoe_shape* shape, int32_t which /* 0: w13, 1: w2 */,
                             int32_t n_experts);
int acceptmoe_pack_experts(const acceptmoe_shape* shape, int32_t n_experts, const void* w13,
                           const void* w2, void* w13_packed, void* w2_packed, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine -- unpermute and gate-weighted sum.
 *
 * [MoE-SD blog, MoE layer]: y[i,:] = sum_j topk_gate[i,j] * y_perm[inv_pos[i*k+j],:]
 * (+ y_shared[i,:], the always-on shared expert, unweighted), written in
 * act_dtype (bf16: round to nearest even).
 *   y_perm [N*k,H] fp32, inv_pos [N*k], topk_gate [N,k] fp32,
 *   y_shared [N,H] fp32 or NULL, y [N,H] act_dtype
 * ------------------------------------------------------------------------- */
int moe_combine(int32_t N, int32_t k, int32_t H, int32_t act_dtype, const float* y_perm,
                const int32_t* inv_pos, const float* topk_gate, const float* y_shared, void* y,
                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * verify_block -- the whole layer for one verification block:
 * acceptmoe_select -> moe_route_permute -> moe_grouped_swiglu (+ shared
 * expert) -> moe_combine, enqueued back to back on one stream.
 * ------------------------------------------------------------------------- */
typedef struct acceptmoe_inputs {  /* device pointers, as in the calls above */
  const void* x;
  const void* w_router;
  const float* b_router;     /* or NULL */
  const float* logits_in;    /* used iff F_LOGITS_IN */
  const int32_t* parent;
  const int32_t* depth;
  const float* commit;
  const uint8_t* resident;   /* or NULL */
  const void* w13;
  const void* w2;
  const float* s13;          /* FP8 only */
  const float* s2;           /* FP8 only */
  const void* w13_shared;    /* [2,I,H] or NULL: no shared expert */
  const void* w2_shared;     /* [H,I] */
  const float* s13_shared;   /* [2,I/128,H/128], FP8 only */
  const float* s2_shared;    /* [H/128,I/128],   FP8 only */
} acceptmoe_inputs;

typedef struct acceptmoe_outputs { /* device pointers; only y is required */
  void* y;                   /* [N,H] act_dtype */
  float* logits_out;         /* [N,E] */
  uint8_t* eligible;         /* [E] */
  int32_t* topk_idx;         /* [N,k] */
  float* topk_gate;          /* [N,k] */
  int32_t* counts;           /* [E] */
  int32_t* active;           /* [E] */
  acceptmoe_stats* stats;    /* [1] */
} acceptmoe_outputs;

/* ws: at least acceptmoe_workspace_size(shape) bytes, zero-filled once before
 * its first use and not shared by overlapping calls, as for acceptmoe_select
 * (the select stage's counters sit at the same offsets). */
size_t acceptmoe_workspace_size(const acceptmoe_shape* shape);
int verify_block(const acceptmoe_shape* shape, const acceptmoe_inputs* in,
                 const acceptmoe_outputs* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * verify_block_overlap -- verify_block with the layer's shared expert on a
 * second stream, so it runs while the selection and the routed experts do.
 * Same outputs, bit for bit.
 *
 * [MoE-SD blog, MoE layer]: an always-on shared expert adds its output to
 * every token, unweighted; it depends on x alone, not on the routing, so it
 * need not wait for the selection.  [EcoSpec, Fig. 1]: verification time is
 * the experts' weight traffic; streaming the shared expert's weights next to
 * the selection (which moves little) takes them off the block's critical
 * path.  The side stream forks from `stream` at the start of the call and is
 * joined back into it before the combine.  Without a shared expert, or with
 * F32 weights, the call is verify_block.
 *
 *   ov->side   a second stream of the caller, of the same (default) priority
 *              as `stream`, not `stream` itself; the call is still ordered
 *              as a whole on `stream`, and can be captured in a HIP graph (the
 *              side stream joins the capture through the events)
 *   ov->start, ov->done   two events of the caller, re-recorded by every call
 *              (timing may be disabled)
 *   ws         as verify_block
 * Calls that share a workspace or a side stream must not overlap in time.
 * ------------------------------------------------------------------------- */
typedef struct acceptmoe_overlap {
  hipStream_t side;
  hipEvent_t start;
  hipEvent_t done;
} acceptmoe_overlap;

int verify_block_overlap(const acceptmoe_shape* shape, const acceptmoe_inputs* in,
                         const acceptmoe_outputs* out, const acceptmoe_overlap* ov, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * verify_block_noalloc -- verify_block for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that never call hipMalloc): the workspace is the library's own device
 * array of ACCEPTMOE_NOALLOC_WORKSPACE_BYTES (one per GPU the library runs
 * on, held until the process ends), so the call takes no ws argument and
 * allocates nothing.  Inputs and outputs are the caller's, as for
 * verify_block, and the results are the same.
 *   Errors: as verify_block; a shape whose workspace
 *   (acceptmoe_workspace_size) exceeds ACCEPTMOE_NOALLOC_WORKSPACE_BYTES is
 *   rejected with ACCEPTMOE_EINVAL before anything is enqueued (every
 *   64-node block of hidden size <= 4096 fits; the 256-node DeepSeek-shaped
 *   block does not).  ACCEPTMOE_EHIP if the array's device address cannot be
 *   looked up.
 *   Each call clears the array's arrival counters on `stream` first (a
 *   kernel, so the call can be captured in a graph).  Every call on one GPU
 *   shares that GPU's array and leaves the last call's contents in it: calls
 *   that overlap in time on one GPU race -- serialise them (one stream, or
 *   events).
 * ------------------------------------------------------------------------- */
#define ACCEPTMOE_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)
int verify_block_noalloc(const acceptmoe_shape* shape, const acceptmoe_inputs* in,
                         const acceptmoe_outputs* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Profiling aid: per-thread stage timer.  After
 * acceptmoe_set_stage_timer(stage, start, stop), every later verify_block call
 * on this host thread records `start` on its stream right before the first
 * kernel of `stage` and `stop` right after its last kernel, so
 * hipEventElapsedTime(start, stop) is that stage's device time.  stage = 0
 * (or NULL events) turns it off.  The events belong to the caller.  Returns
 * ACCEPTMOE_EINVAL for an unknown stage.
 * ------------------------------------------------------------------------- */
enum {
  ACCEPTMOE_STAGE_NONE = 0,
  ACCEPTMOE_STAGE_SELECT = 1,   /* router, per-node scores, set selection, restricted top-k,
                                   group by expert                                          */
  ACCEPTMOE_STAGE_PERMUTE = 2,  /* reserved: grouping runs inside the SELECT stage          */
  ACCEPTMOE_STAGE_GATEUP = 3,   /* routed experts: gate/up projections + SwiGLU             */
  ACCEPTMOE_STAGE_DOWN = 4,     /* routed experts: down projection                          */
  ACCEPTMOE_STAGE_EXPERTS = 5,  /* routed experts: both projections                         */
  ACCEPTMOE_STAGE_COMBINE = 6,  /* shared expert (if any) + unpermute/combine               */
  ACCEPTMOE_STAGE_FETCH = 7     /* verify_block_cached: host-to-device expert copies        */
};
int acceptmoe_set_stage_timer(int32_t stage, hipEvent_t start, hipEvent_t stop);

/* ---------------------------------------------------------------------------
 * Physical expert offload: a per-layer cache of device expert slots.
 *
 * [AcceptMoE news §02]: under offload an expert that is already on the GPU
 * runs at once and one that is not has to be loaded from CPU memory first;
 * residency-aware pruning drops low-demand non-resident experts from the
 * eligible set.  [AcceptMoE news §03]: 48 expert slots per layer; the
 * measures are host-to-device expert bytes and the expert-cache hit rate.
 * The pages give no replacement policy; this one is least recently used.
 *
 * The caller keeps every expert's packed weights (acceptmoe_pack_experts
 * layout) in host memory -- pinned (hipHostMalloc) for asynchronous DMA --
 * and owns n_slots + n_spill device slots of packed weights.  Slots
 * 0..n_slots-1 are persistent: their experts form the resident set.  The
 * spill slots hold experts that miss when every persistent slot holds an
 * expert of the same block; they are loaded again on their next use.
 *
 * acceptmoe_cache_state (host memory, owned by the caller; zero counters and
 * clock, slot_expert / expert_slot -1 and resident 0 for an empty cache, or
 * fill a warm start consistently: slot_expert[q] = e <=> expert_slot[e] = q,
 * resident[e] = 1).
 *
 * acceptmoe_cache_plan (host only, no GPU): for the ascending active expert
 * ids of one block, hits keep their slot and take the current clock; each
 * miss, in ascending expert order, takes the lowest empty persistent slot,
 * else evicts the least recently used persistent slot whose expert is not
 * active in this block (ties: lowest slot), else takes the next spill slot
 * n_slots + j.  Writes the fetches (expert, slot) in that order and updates
 * the state and its counters.  ACCEPTMOE_EINVAL (state unchanged) when the
 * misses need more than n_spill spill slots, or for a malformed state /
 * active list (ids outside [0, E) or repeated).
 *
 * verify_block_cached: verify_block with the routed experts' weights taken
 * from the cache.  The selection's resident mask is cache->dev_resident (so
 * residency-aware pruning applies when reroute_budget > 0); the
 * active experts are copied back to the host and the stream is synchronized
 * once; the plan's missing experts are copied host -> device into their
 * slots with hipMemcpyAsync on `stream`, followed by dev_expert_slot and
 * dev_resident; then the expert kernels read expert e's weights from slot
 * dev_expert_slot[e].  in->w13, in->w2 and in->resident are not used; FP8
 * scales (in->s13, in->s2, all E experts) and the shared expert stay on the
 * device.  Packed BF16 or FP8 weights only (else ACCEPTMOE_ENOTSUP).  Not
 * capturable in a HIP graph (it synchronizes).  The state's tables must not
 * change while the call's copies are pending on the stream.  report (host,
 * may be NULL) receives this call's counts.
 *
 * Overlap: with copy_stream, copy_done and dev_lists set (a stream of the
 * default priority, an event, 2E+3 device ints, all the caller's), the
 * missing experts are copied on copy_stream, one after another, while the
 * experts that hit run on `stream`; each missing expert's kernels then run
 * on `stream` as soon as its own copy has landed (copy_done is re-recorded
 * after every copy), so the computation of one fetched expert overlaps the
 * copy of the next ([MoE-SD blog, CPU offload section] counts the overlap
 * of transfers with compute among the measures of an offload system).
 * Results are identical: every expert's rows are computed by the same
 * kernels, only in more launches.
 * ------------------------------------------------------------------------- */
typedef struct acceptmoe_cache_state {
  int32_t E;              /* routed experts                                      */
  int32_t n_slots;        /* persistent device slots                             */
  int32_t n_spill;        /* spill slots after them                              */
  int32_t _pad;
  int32_t* slot_expert;   /* [n_slots] expert held, -1 = empty                   */
  int32_t* expert_slot;   /* [E] slot (persistent or spill) for the last block, -1 = none */
  uint8_t* resident;      /* [E] 1 iff the expert holds a persistent slot        */
  int64_t* last_use;      /* [n_slots] clock of the slot's last use              */
  int64_t clock;          /* blocks planned                                      */
  int64_t hits, misses, spills, h2d_bytes;  /* running totals                    */
} acceptmoe_cache_state;

typedef struct acceptmoe_expert_cache {
  acceptmoe_cache_state* state;   /* host                                          */
  const void* host_w13;           /* host, packed w13 of all E experts             */
  const void* host_w2;            /* host, packed w2 of all E experts              */
  void* dev_w13;                  /* device, packed w13 of n_slots + n_spill slots */
  void* dev_w2;                   /* device, packed w2 of n_slots + n_spill slots  */
  int32_t* dev_expert_slot;       /* device [E]                                    */
  uint8_t* dev_resident;          /* device [E]                                    */
  hipStream_t copy_stream;        /* or NULL: the copies run on the call's stream  */
  hipEvent_t copy_done;           /* with copy_stream                              */
  int32_t* dev_lists;             /* device [2E+3], with copy_stream               */
} acceptmoe_expert_cache;

typedef struct acceptmoe_cache_report {  /* one verify_block_cached call      */
  int32_t n_active, n_hits, n_fetched, n_spilled;
  int64_t h2d_bytes;
} acceptmoe_cache_report;

int acceptmoe_cache_plan(acceptmoe_cache_state* state, const int32_t* active /* host */,
                         int32_t n_active, int32_t* fetch_expert /* host [n_active] */,
                         int32_t* fetch_slot /* host [n_active] */, int32_t* n_fetch);
int verify_block_cached(const acceptmoe_shape* shape, const acceptmoe_inputs* in,
                        const acceptmoe_expert_cache* cache, const acceptmoe_outputs* out,
                        acceptmoe_cache_report* report, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Messages and version (host). */
const char* acceptmoe_strerror(int code);
const char* acceptmoe_last_error(void);
const char* acceptmoe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ACCEPTMOE_H */
