// C ABI of the AcceptMoE verify-block MoE layer (see include/acceptmoe.h).
// Host side only: argument checks, workspace carve-up, kernel launches on the
// caller's stream.  No allocation, no synchronisation, no device reads.

#include "acceptmoe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "amoe_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

// per-thread stage timer (acceptmoe_set_stage_timer)
thread_local int g_timer_stage = 0;
thread_local hipEvent_t g_timer_start = nullptr;
thread_local hipEvent_t g_timer_stop = nullptr;

void timer_mark(int stage, bool begin, hipStream_t stream) {
  if (g_timer_stage != stage || !g_timer_start || !g_timer_stop) return;
  (void)hipEventRecord(begin ? g_timer_start : g_timer_stop, stream);
}

constexpr int kMaxDevices = 64;
// split mode starts where the experts average this many routed rows (N*k/E)
constexpr int64_t kSplitRows = 32;
// in split mode, experts with at most kSmallRows routed rows take the
// streaming kernels -- below kAllGemmRows mean routed rows per expert; from
// there on every active expert runs in the GEMM tiles (Qwen3-30B-shaped
// layer, natural routing: N = 512 296 vs 307 us, N = 1024 368 vs 357 us,
// N = 2048 513 vs 480 us)
constexpr int kSmallRows = 64;
constexpr int64_t kAllGemmRows = 64;
std::atomic<int> g_num_cu[kMaxDevices];

// compute units of the current device (queried once per device)
int num_cu() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_num_cu[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_num_cu[dev].store(n, std::memory_order_relaxed);
  return n;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align256(count * sizeof(T));
    return p;
  }
};

bool dtype_pair_ok(int act, int w) {
  return (act == ACCEPTMOE_F32 && w == ACCEPTMOE_F32) ||
         (act == ACCEPTMOE_BF16 && w == ACCEPTMOE_BF16) ||
         (act == ACCEPTMOE_BF16 && w == ACCEPTMOE_FP8_E4M3FN);
}

int check_sizes(int N, int k, int E, int H, int I, int w_dtype, bool need_h, bool need_i) {
  if (N < 1 || N > 4096) return fail(ACCEPTMOE_EINVAL, "N=%d outside [1, 4096]", N);
  if (k < 1 || k > 16) return fail(ACCEPTMOE_EINVAL, "k=%d outside [1, 16]", k);
  if (E < k || E > 256) return fail(ACCEPTMOE_EINVAL, "E=%d outside [k=%d, 256]", E, k);
  const int mult = w_dtype == ACCEPTMOE_FP8_E4M3FN ? 128 : 64;
  if (need_h && (H < mult || H > 16384 || H % mult))
    return fail(ACCEPTMOE_EINVAL, "H=%d must be a multiple of %d in [%d, 16384]", H, mult, mult);
  if (need_i && (I < mult || I > 16384 || I % mult))
    return fail(ACCEPTMOE_EINVAL, "I=%d must be a multiple of %d in [%d, 16384]", I, mult, mult);
  return ACCEPTMOE_OK;
}

int check_shape(const acceptmoe_shape* s, bool need_i) {
  if (!s) return fail(ACCEPTMOE_EINVAL, "shape is NULL");
  if (!dtype_pair_ok(s->act_dtype, s->w_dtype))
    return fail(ACCEPTMOE_ENOTSUP, "unsupported dtype pair (act %d, weights %d)", s->act_dtype,
                s->w_dtype);
  if (s->flags & ~63u) return fail(ACCEPTMOE_ENOTSUP, "unknown flag bits %#x", s->flags);
  if (s->w_layout != ACCEPTMOE_LAYOUT_ROWMAJOR && s->w_layout != ACCEPTMOE_LAYOUT_PACKED)
    return fail(ACCEPTMOE_ENOTSUP, "unknown weight layout %d", s->w_layout);
  if (s->w_layout == ACCEPTMOE_LAYOUT_PACKED && s->w_dtype == ACCEPTMOE_F32)
    return fail(ACCEPTMOE_ENOTSUP, "the packed layout needs BF16 or FP8 weights");
  int rc = check_sizes(s->N, s->k, s->E, s->H, s->I, s->w_dtype, true, need_i);
  if (rc) return rc;
  if (s->n_depth < 1) return fail(ACCEPTMOE_EINVAL, "n_depth=%d < 1", s->n_depth);
  if (s->min_set < 0 || s->min_set > s->E)
    return fail(ACCEPTMOE_EINVAL, "min_set=%d outside [0, E]", s->min_set);
  if (s->fixed_budget < 0 || s->fixed_budget > s->E)
    return fail(ACCEPTMOE_EINVAL, "fixed_budget=%d outside [0, E]", s->fixed_budget);
  if (s->reroute_budget < 0) return fail(ACCEPTMOE_EINVAL, "reroute_budget < 0");
  return ACCEPTMOE_OK;
}

// workspace of the selection stage, carved in a fixed order
struct SelectWs {
  float* part;
  float* logits;
  float* node_m;
  double* node_z;
  int32_t* nat_idx;
  float* nat_logit;
  double* d_part;
  uint8_t* f_part;
  int32_t* e_part;
  int32_t* counters;
  int32_t* gcount;
  int32_t* ghist;
  int ksplit, kslice;
};

SelectWs carve_select(Carver& c, const acceptmoe_shape* s) {
  SelectWs w;
  amoe::select_plan(s->N, s->H, s->E, 0, &w.ksplit, &w.kslice);
  // arrival counters first, at offsets that do not depend on the shape: the
  // kernels leave them at zero, so a zero-filled workspace stays valid
  w.counters = c.take<int32_t>(2);
  w.gcount = c.take<int32_t>(4096 / 4);
  const size_t NE = static_cast<size_t>(s->N) * s->E;
  w.part = c.take<float>(static_cast<size_t>(w.ksplit) * NE);
  w.logits = c.take<float>(NE);
  w.node_m = c.take<float>(s->N);
  w.node_z = c.take<double>(s->N);
  w.nat_idx = c.take<int32_t>(static_cast<size_t>(s->N) * s->k);
  w.nat_logit = c.take<float>(static_cast<size_t>(s->N) * s->k);
  w.ghist = c.take<int32_t>(static_cast<size_t>(amoe::group_chunks(s->N, s->k)) * s->E);
  const size_t nwg = amoe::node_workgroups(s->N, s->E);
  w.d_part = c.take<double>(amoe::dpart_elems(s->N, s->E));
  w.f_part = c.take<uint8_t>(amoe::fpart_bytes(s->N, s->E));
  w.e_part = c.take<int32_t>(nwg);
  return w;
}

size_t hidden_elem_bytes(int w_dtype) { return w_dtype == ACCEPTMOE_F32 ? 4 : 2; }

struct VerifyWs {
  SelectWs sel;
  uint8_t* eligible;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_assign;
  int32_t* inv_pos;
  int32_t* active;
  int32_t* n_active;
  int32_t* groups;
  int32_t* active_w;
  acceptmoe_stats* stats;
  void* h_perm;
  float* y_perm;
  int32_t* sh_offsets;
  int32_t* sh_sorted;
  int32_t* sh_active;
  int32_t* sh_n_active;
  void* sh_h;
  float* sh_y;
};

VerifyWs carve_verify(Carver& c, const acceptmoe_shape* s, bool shared) {
  VerifyWs w;
  w.sel = carve_select(c, s);
  const size_t NK = static_cast<size_t>(s->N) * s->k;
  w.eligible = c.take<uint8_t>(s->E);
  w.topk_idx = c.take<int32_t>(NK);
  w.topk_gate = c.take<float>(NK);
  w.counts = c.take<int32_t>(s->E);
  w.offsets = c.take<int32_t>(s->E + 1);
  w.sorted_assign = c.take<int32_t>(NK);
  w.inv_pos = c.take<int32_t>(NK);
  w.active = c.take<int32_t>(s->E);
  // [1]: the most rows routed to one expert; [2]: the small experts' count
  // (split mode)
  w.n_active = c.take<int32_t>(4);
  // 64-row groups of the active experts: at most N*k/64 + E, plus the count
  w.groups = c.take<int32_t>(2 + NK / 64 + s->E);
  // the active experts in the order the expert kernels take them
  w.active_w = c.take<int32_t>(s->E);
  w.stats = c.take<acceptmoe_stats>(1);
  w.h_perm = c.take<char>(NK * s->I * hidden_elem_bytes(s->w_dtype));
  w.y_perm = c.take<float>(NK * s->H);
  w.sh_offsets = w.sh_sorted = w.sh_active = w.sh_n_active = nullptr;
  w.sh_h = nullptr;
  w.sh_y = nullptr;
  if (shared) {
    w.sh_offsets = c.take<int32_t>(2);
    w.sh_sorted = c.take<int32_t>(s->N);
    w.sh_active = c.take<int32_t>(1);
    w.sh_n_active = c.take<int32_t>(1);
    w.sh_h = c.take<char>(static_cast<size_t>(s->N) * s->I * hidden_elem_bytes(s->w_dtype));
    w.sh_y = c.take<float>(static_cast<size_t>(s->N) * s->H);
  }
  return w;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(ACCEPTMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ACCEPTMOE_OK;
}

amoe::SelectArgs select_args(const acceptmoe_shape* s, const SelectWs& w) {
  amoe::SelectArgs a;
  std::memset(&a, 0, sizeof(a));
  a.N = s->N;
  a.H = s->H;
  a.E = s->E;
  a.k = s->k;
  a.n_depth = s->n_depth;
  a.min_set = s->min_set;
  a.fixed_budget = s->fixed_budget;
  a.reroute_budget = s->reroute_budget;
  a.flags = s->flags;
  a.act_bf16 = s->act_dtype == ACCEPTMOE_BF16;
  a.part = w.part;
  a.ksplit = w.ksplit;
  a.kslice = w.kslice;
  a.logits = w.logits;
  a.node_m = w.node_m;
  a.node_z = w.node_z;
  a.nat_idx = w.nat_idx;
  a.nat_logit = w.nat_logit;
  a.d_part = w.d_part;
  a.f_part = w.f_part;
  a.e_part = w.e_part;
  a.counters = w.counters;
  a.gcount = w.gcount;
  a.ghist = w.ghist;
  a.group_shift = 6;
  a.split_rows = -1;
  return a;
}

int w_kind(int w_dtype) {
  return w_dtype == ACCEPTMOE_F32 ? 0 : (w_dtype == ACCEPTMOE_BF16 ? 1 : 2);
}

// ------------------------------------------------------------ expert cache --
int check_state(const acceptmoe_cache_state* st) {
  if (!st) return fail(ACCEPTMOE_EINVAL, "cache state is NULL");
  if (st->E < 1 || st->E > 256 || st->n_slots < 0 || st->n_slots > st->E || st->n_spill < 0 ||
      st->n_spill > st->E)
    return fail(ACCEPTMOE_EINVAL, "cache state: E=%d, n_slots=%d, n_spill=%d out of range", st->E,
                st->n_slots, st->n_spill);
  if (!st->slot_expert || !st->expert_slot || !st->resident || !st->last_use)
    return fail(ACCEPTMOE_EINVAL, "cache state: a table pointer is NULL");
  for (int q = 0; q < st->n_slots; ++q) {
    const int e = st->slot_expert[q];
    if (e < -1 || e >= st->E || (e >= 0 && (st->expert_slot[e] != q || !st->resident[e])))
      return fail(ACCEPTMOE_EINVAL, "cache state: slot %d holds expert %d inconsistently", q, e);
  }
  // the other direction: a resident expert names a persistent slot that
  // holds it; a non-resident expert names no persistent slot (a spill slot
  // from the last block, n_slots .. n_slots + n_spill - 1, or -1)
  for (int e = 0; e < st->E; ++e) {
    const int q = st->expert_slot[e];
    if (st->resident[e]) {
      if (q < 0 || q >= st->n_slots || st->slot_expert[q] != e)
        return fail(ACCEPTMOE_EINVAL, "cache state: resident expert %d names slot %d, which "
                    "does not hold it", e, q);
    } else if (q < -1 || (q >= 0 && q < st->n_slots) || q >= st->n_slots + st->n_spill) {
      return fail(ACCEPTMOE_EINVAL, "cache state: non-resident expert %d names slot %d", e, q);
    }
  }
  return ACCEPTMOE_OK;
}

// The fetch plan for one block's active experts (ascending ids).  Hits keep
// their slot and take the current clock.  Each miss, in ascending expert
// order, takes the lowest empty persistent slot, else evicts the least
// recently used persistent slot whose expert is not active in this block
// (ties: lowest slot), else a spill slot n_slots + j (held for this block
// only, not resident afterwards).  The whole plan is checked before the
// state changes: too few spill slots leaves it untouched.
int plan_fetches(acceptmoe_cache_state* st, const int32_t* active, int n_active,
                 int32_t* fetch_expert, int32_t* fetch_slot, int32_t* n_fetch,
                 acceptmoe_cache_report* rep) {
  const int E = st->E, S = st->n_slots;
  uint8_t act[256];
  std::memset(act, 0, sizeof(act));
  int misses = 0;
  for (int u = 0; u < n_active; ++u) {
    const int e = active[u];
    if (e < 0 || e >= E || act[e]) return fail(ACCEPTMOE_EINVAL, "bad active expert %d", e);
    act[e] = 1;
    if (!st->resident[e]) ++misses;
  }
  int free_or_evictable = 0;
  for (int q = 0; q < S; ++q) {
    const int e = st->slot_expert[q];
    if (e < 0 || !act[e]) ++free_or_evictable;
  }
  const int spill = misses > free_or_evictable ? misses - free_or_evictable : 0;
  if (spill > st->n_spill)
    return fail(ACCEPTMOE_EINVAL, "%d active experts miss the cache; %d slots and %d spill slots "
                "cannot hold them", misses, free_or_evictable, st->n_spill);
  st->clock += 1;
  // a spill slot holds its expert for one block only
  for (int e = 0; e < E; ++e)
    if (!st->resident[e]) st->expert_slot[e] = -1;
  int nf = 0, hits = 0, spilled = 0;
  for (int u = 0; u < n_active; ++u) {
    const int e = active[u];
    if (st->resident[e]) {
      st->last_use[st->expert_slot[e]] = st->clock;
      ++hits;
      continue;
    }
    int slot = -1;
    for (int q = 0; q < S && slot < 0; ++q)
      if (st->slot_expert[q] < 0) slot = q;
    if (slot < 0) {
      for (int q = 0; q < S; ++q) {
        const int o = st->slot_expert[q];
        if (o < 0 || act[o]) continue;
        if (slot < 0 || st->last_use[q] < st->last_use[slot]) slot = q;
      }
    }
    if (slot >= 0) {
      const int old = st->slot_expert[slot];
      if (old >= 0) {
        st->resident[old] = 0;
        st->expert_slot[old] = -1;
      }
      st->slot_expert[slot] = e;
      st->resident[e] = 1;
      st->last_use[slot] = st->clock;
    } else {
      slot = S + spilled++;
    }
    st->expert_slot[e] = slot;
    fetch_expert[nf] = e;
    fetch_slot[nf] = slot;
    ++nf;
  }
  *n_fetch = nf;
  st->hits += hits;
  st->misses += nf;
  st->spills += spilled;
  if (rep) {
    rep->n_active = n_active;
    rep->n_hits = hits;
    rep->n_fetched = nf;
    rep->n_spilled = spilled;
    rep->h2d_bytes = 0;
  }
  return ACCEPTMOE_OK;
}

int check_cache(const acceptmoe_shape* s, const acceptmoe_expert_cache* c) {
  if (s->w_layout != ACCEPTMOE_LAYOUT_PACKED || s->w_dtype == ACCEPTMOE_F32)
    return fail(ACCEPTMOE_ENOTSUP, "the expert cache holds packed BF16 or FP8 weights");
  int rc = check_state(c->state);
  if (rc) return rc;
  if (c->state->n_slots + c->state->n_spill < 1)
    return fail(ACCEPTMOE_EINVAL, "the cache has no device slots");
  if (c->state->E != s->E)
    return fail(ACCEPTMOE_EINVAL, "cache state E=%d != shape E=%d", c->state->E, s->E);
  if (!c->host_w13 || !c->host_w2 || !c->dev_w13 || !c->dev_w2 || !c->dev_expert_slot ||
      !c->dev_resident)
    return fail(ACCEPTMOE_EINVAL, "a cache pointer is NULL");
  return ACCEPTMOE_OK;
}

// The missing experts of one block: (expert, slot) in plan order, and the
// bytes of one expert's packed weights.
struct FetchPlan {
  int nf = 0;
  int32_t fe[256], fs[256];
  size_t b13 = 0, b2 = 0;
};

// Host-to-device copy of fetched expert f's packed weights into its slot.
hipError_t copy_expert(const acceptmoe_expert_cache* c, const FetchPlan& p, int f,
                       hipStream_t cs) {
  const char* h13 = static_cast<const char*>(c->host_w13);
  const char* h2 = static_cast<const char*>(c->host_w2);
  char* d13 = static_cast<char*>(c->dev_w13);
  char* d2 = static_cast<char*>(c->dev_w2);
  hipError_t e = hipMemcpyAsync(d13 + p.b13 * p.fs[f], h13 + p.b13 * p.fe[f], p.b13,
                                hipMemcpyHostToDevice, cs);
  if (e == hipSuccess)
    e = hipMemcpyAsync(d2 + p.b2 * p.fs[f], h2 + p.b2 * p.fe[f], p.b2, hipMemcpyHostToDevice, cs);
  return e;
}

// After the selection: read the active experts back (one stream
// synchronization), plan, upload the slot table and resident mask, and copy
// the missing experts' packed weights from host memory into their slots --
// unless the cache has a copy stream (*overlap): then the copies are left to
// the caller, which interleaves them with the fetched experts' kernels.
int cache_fetch(const acceptmoe_shape* s, const acceptmoe_expert_cache* c, const int32_t* active,
                const int32_t* n_active, acceptmoe_cache_report* report, hipStream_t stream,
                bool* overlap, FetchPlan* plan) {
  acceptmoe_cache_state* st = c->state;
  int32_t host_n = 0;
  int32_t host_active[256];
  hipError_t e = hipMemcpyAsync(&host_n, n_active, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(host_active, active, sizeof(int32_t) * s->E, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  int rc = hip_status(e, "verify_block_cached/read active experts");
  if (rc) return rc;
  if (host_n < 0 || host_n > s->E)
    return fail(ACCEPTMOE_EINVAL, "verify_block_cached: device reported %d active experts", host_n);
  acceptmoe_cache_report rep;
  int32_t* fe = plan->fe;
  int32_t* fs = plan->fs;
  int nf = 0;
  rc = plan_fetches(st, host_active, host_n, fe, fs, &nf, &rep);
  if (rc) return rc;
  const int wk = w_kind(s->w_dtype);
  plan->nf = nf;
  plan->b13 = amoe::packed_bytes(0, wk, 1, s->H, s->I);
  plan->b2 = amoe::packed_bytes(1, wk, 1, s->H, s->I);
  const size_t b13 = plan->b13, b2 = plan->b2;
  // the slot table and resident mask first, on the launch stream: every
  // expert kernel of this block reads the table
  e = hipMemcpyAsync(c->dev_expert_slot, st->expert_slot, sizeof(int32_t) * s->E,
                     hipMemcpyHostToDevice, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->dev_resident, st->resident, s->E, hipMemcpyHostToDevice, stream);
  // with a copy stream, the hit experts run while the missing ones are
  // copied in, then each missing expert as its copy lands:
  // lists [hits (E)] [n_hits] [misses (E)] [n_misses] [1]
  *overlap = c->copy_stream != nullptr && c->copy_done != nullptr && c->dev_lists != nullptr &&
             nf > 0;
  if (*overlap && e == hipSuccess) {
    const int E = s->E;
    int32_t lists[2 * 256 + 3];
    uint8_t miss[256];
    std::memset(miss, 0, sizeof(miss));
    for (int f = 0; f < nf; ++f) miss[fe[f]] = 1;
    int nh = 0;
    for (int u = 0; u < host_n; ++u)
      if (!miss[host_active[u]]) lists[nh++] = host_active[u];
    for (int u = nh; u < E; ++u) lists[u] = 0;
    lists[E] = nh;
    for (int f = 0; f < nf; ++f) lists[E + 1 + f] = fe[f];
    for (int f = nf; f < E; ++f) lists[E + 1 + f] = 0;
    lists[2 * E + 1] = nf;
    lists[2 * E + 2] = 1;
    e = hipMemcpyAsync(c->dev_lists, lists, sizeof(int32_t) * (2 * E + 3), hipMemcpyHostToDevice,
                       stream);
  }
  if (!*overlap) {
    timer_mark(ACCEPTMOE_STAGE_FETCH, true, stream);
    for (int f = 0; f < nf && e == hipSuccess; ++f) e = copy_expert(c, *plan, f, stream);
    timer_mark(ACCEPTMOE_STAGE_FETCH, false, stream);
  }
  rc = hip_status(e, "verify_block_cached/fetch");
  if (rc) return rc;
  rep.h2d_bytes = static_cast<int64_t>(nf) * static_cast<int64_t>(b13 + b2);
  st->h2d_bytes += rep.h2d_bytes;
  if (report) *report = rep;
  return ACCEPTMOE_OK;
}

// Argument checks of verify_block / verify_block_cached, apart from the
// workspace pointer: returns the workspace bytes the call needs in *need.
int check_block_args(const acceptmoe_shape* s, const acceptmoe_inputs* in,
                     const acceptmoe_expert_cache* cache, const acceptmoe_outputs* out,
                     size_t* need) {
  int rc = check_shape(s, true);
  if (rc) return rc;
  if (!in || !out) return fail(ACCEPTMOE_EINVAL, "inputs or outputs is NULL");
  const bool lin = (s->flags & ACCEPTMOE_F_LOGITS_IN) != 0;
  if (lin ? !in->logits_in : (!in->x || !in->w_router))
    return fail(ACCEPTMOE_EINVAL, lin ? "logits_in is NULL" : "x or w_router is NULL");
  if (!in->x || !in->parent || !in->depth || !in->commit || !out->y)
    return fail(ACCEPTMOE_EINVAL, "a required pointer is NULL");
  if (!cache && (!in->w13 || !in->w2)) return fail(ACCEPTMOE_EINVAL, "w13 or w2 is NULL");
  if (cache) {
    rc = check_cache(s, cache);
    if (rc) return rc;
  }
  const bool fp8 = s->w_dtype == ACCEPTMOE_FP8_E4M3FN;
  if (fp8 && (!in->s13 || !in->s2)) return fail(ACCEPTMOE_EINVAL, "FP8 weights need s13 and s2");
  const bool shared = in->w13_shared != nullptr;
  if (shared && (!in->w2_shared || (fp8 && (!in->s13_shared || !in->s2_shared))))
    return fail(ACCEPTMOE_EINVAL, "incomplete shared-expert weights");
  Carver c(nullptr);
  carve_verify(c, s, true);
  *need = c.used;
  return ACCEPTMOE_OK;
}

}  // namespace

namespace amoe {

int check_verify_args(const acceptmoe_shape* s, const acceptmoe_inputs* in,
                      const acceptmoe_outputs* out, size_t* need) {
  return check_block_args(s, in, nullptr, out, need);
}

size_t workspace_counter_bytes() {
  // the arrival counters are the first two allocations of every workspace
  Carver c(nullptr);
  c.take<int32_t>(2);
  c.take<int32_t>(4096 / 4);
  return c.used;
}

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

}  // namespace amoe

namespace {

// The shared expert's two projections, in dense mode over all N rows (bf16 /
// fp8; fp32 weights take the identity grouping), on `stream`.
int launch_shared(const acceptmoe_shape* s, const acceptmoe_inputs* in, const VerifyWs& w,
                  const amoe::GroupedArgs& g, hipStream_t stream) {
  amoe::GroupedArgs gs = g;
  gs.k = 1;
  gs.E = 1;
  gs.w13 = in->w13_shared;
  gs.w2 = in->w2_shared;
  gs.s13 = in->s13_shared;
  gs.s2 = in->s2_shared;
  gs.y_perm = w.sh_y;
  gs.h_perm = w.sh_h;
  gs.tok_rows = 0;
  gs.w_slot = nullptr;
  gs.n_wslots = 0;
  gs.max_rows = nullptr;
  gs.groups = nullptr;
  gs.snake = 0;
  gs.gemm = 0;
  gs.row_groups = (s->N + 63) / 64;  // the shared expert takes all N rows
  if (g.w_kind != 0) {
    gs.dense_n = 1;
    gs.active = nullptr;
    gs.n_active = nullptr;
    gs.offsets = nullptr;
    gs.sorted_assign = nullptr;
  } else {
    int rc = hip_status(amoe::launch_shared_grouping(s->N, w.sh_offsets, w.sh_sorted,
                                                     w.sh_active, w.sh_n_active, stream),
                        "verify_block/shared grouping");
    if (rc) return rc;
    gs.dense_n = 0;
    gs.offsets = w.sh_offsets;
    gs.sorted_assign = w.sh_sorted;
    gs.active = w.sh_active;
    gs.n_active = w.sh_n_active;
  }
  return hip_status(amoe::launch_grouped(gs, stream), "verify_block/shared expert");
}

// verify_block, and with `cache` set verify_block_cached: the expert weights
// then come from the cache's device slots, after the missing ones are copied
// in (one stream synchronization after the selection).  With `ov` set
// (verify_block_overlap), the shared expert, which depends on x alone, runs
// on the caller's side stream while the selection and the routed experts
// run, and is joined before the combine.
int run_block(const acceptmoe_shape* s, const acceptmoe_inputs* in,
              const acceptmoe_expert_cache* cache, const acceptmoe_outputs* out,
              acceptmoe_cache_report* report, const acceptmoe_overlap* ov, void* ws,
              size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  int rc = check_block_args(s, in, cache, out, &need);
  if (rc) return rc;
  if (!ws) return fail(ACCEPTMOE_EINVAL, "a required pointer is NULL");
  if (ws_bytes < need)
    return fail(ACCEPTMOE_EINVAL, "workspace %zu bytes < %zu required", ws_bytes, need);
  const bool shared = in->w13_shared != nullptr;
  const int wk = w_kind(s->w_dtype);
  // the shared expert (bf16 / fp8 weights) on the side stream
  const bool sh_side = ov != nullptr && !cache && wk != 0 && shared;

  Carver c(ws);
  const VerifyWs w = carve_verify(c, s, shared);
  uint8_t* eligible = out->eligible ? out->eligible : w.eligible;
  int32_t* topk_idx = out->topk_idx ? out->topk_idx : w.topk_idx;
  float* topk_gate = out->topk_gate ? out->topk_gate : w.topk_gate;
  int32_t* counts = out->counts ? out->counts : w.counts;
  int32_t* active = out->active ? out->active : w.active;
  acceptmoe_stats* stats = out->stats ? out->stats : w.stats;

  amoe::SelectArgs a = select_args(s, w.sel);
  a.x = in->x;
  a.w_router = in->w_router;
  a.b_router = in->b_router;
  a.logits_in = in->logits_in;
  a.parent = in->parent;
  a.depth = in->depth;
  a.commit = in->commit;
  a.resident = cache ? cache->dev_resident : in->resident;
  a.logits_out = out->logits_out;
  a.eligible = eligible;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.stats = stats;
  // the selection stage also groups the assignments by expert
  a.counts = counts;
  a.offsets = w.offsets;
  a.sorted_assign = w.sorted_assign;
  a.inv_pos = w.inv_pos;
  a.active = active;
  a.n_active = w.n_active;
  a.max_rows = w.n_active + 1;
  a.groups = w.groups;
  a.active_w = w.active_w;
  // blocks whose experts average 256 routed rows or more (N*k >= 256*E),
  // packed weights: the expert kernels' GEMM tiling (128-row groups; pairs of
  // 64-row items, so 2I and H must be multiples of 128).  Measured on the
  // Qwen3-30B-shaped layer it pays from about that size on (N = 4096 natural
  // routing: 1292 -> 1191 us per block) and not below (N = 512 .. 2048:
  // 1-10 % slower).
  bool gemm = static_cast<int64_t>(s->N) * s->k >= 256ll * s->E &&
              s->w_layout == ACCEPTMOE_LAYOUT_PACKED && wk != 0 && !cache &&
              s->H % 128 == 0;

  amoe::GroupedArgs g = {};
  g.N = s->N;
  g.k = s->k;
  g.E = s->E;
  g.H = s->H;
  g.I = s->I;
  g.w_kind = wk;
  g.act_bf16 = s->act_dtype == ACCEPTMOE_BF16;
  g.x = in->x;
  g.w13 = cache ? cache->dev_w13 : in->w13;
  g.w2 = cache ? cache->dev_w2 : in->w2;
  g.s13 = in->s13;
  g.s2 = in->s2;
  g.offsets = w.offsets;
  g.sorted_assign = w.sorted_assign;
  g.y_perm = w.y_perm;
  g.h_perm = w.h_perm;
  g.num_cu = num_cu();
  g.packed = s->w_layout == ACCEPTMOE_LAYOUT_PACKED;
  // bf16 / fp8 weights: the down projection writes token-major rows, so the
  // combine gathers without inv_pos (same values, same arithmetic)
  g.tok_rows = wk != 0;
  g.row_groups = 1;
  g.w_slot = cache ? cache->dev_expert_slot : nullptr;
  g.n_wslots = cache ? cache->state->n_slots + cache->state->n_spill : 0;
  // Split mode (packed bf16 weights, blocks whose experts average kSplitRows
  // routed rows or more): the experts with more than small_rows routed rows
  // (every active expert from kAllGemmRows mean rows on) run in the GEMM
  // kernels (gemm.hip), the others in the streaming kernels.
  const bool split = !cache && s->N > 64 &&
                     static_cast<int64_t>(s->N) * s->k >= kSplitRows * s->E &&
                     amoe::gemm_supported(g);
  if (split) gemm = false;
  g.gemm = gemm;
  a.group_shift = split ? (amoe::gemm_tile_rows() == 128 ? 7 : 8) : (gemm ? 7 : 6);
  const bool all_gemm = static_cast<int64_t>(s->N) * s->k >= kAllGemmRows * s->E;
  const int small_rows = all_gemm ? 0 : kSmallRows;
  a.split_rows = split ? small_rows : -1;
  a.n_work = w.n_active + 2;

  if (sh_side) {
    // the side stream starts after everything enqueued on `stream` before
    // the call; the main chain is enqueued first, so a graph captured from
    // the call keeps it on one queue
    rc = hip_status(hipEventRecord(ov->start, stream), "verify_block_overlap/fork");
    if (rc) return rc;
  }
  timer_mark(ACCEPTMOE_STAGE_SELECT, true, stream);
  rc = hip_status(amoe::launch_select(a, stream), "verify_block/select");
  if (rc) return rc;
  timer_mark(ACCEPTMOE_STAGE_SELECT, false, stream);
  if (sh_side) {
    rc = hip_status(hipStreamWaitEvent(ov->side, ov->start, 0), "verify_block_overlap/fork");
    if (!rc) rc = launch_shared(s, in, w, g, ov->side);
    if (!rc) rc = hip_status(hipEventRecord(ov->done, ov->side), "verify_block_overlap/join");
    if (rc) return rc;
  }
  bool overlap = false;
  FetchPlan plan;
  if (cache) {
    rc = cache_fetch(s, cache, active, w.n_active, report, stream, &overlap, &plan);
    if (rc) return rc;
  }
  // the expert kernels take the active experts most-routed first: the work
  // items of the few experts with many rows (the longest ones) then start on
  // separate CUs, and the lightest items are the ones that share a CU last
  g.active = w.active_w;
  g.n_active = w.n_active;
  g.snake = 1;
  g.max_rows = w.n_active + 1;
  g.groups = w.groups;
  timer_mark(ACCEPTMOE_STAGE_EXPERTS, true, stream);
  if (overlap) {
    // the hit experts while the missing ones are copied in on the copy
    // stream, then each missing expert once its own copy has landed (the
    // event is re-recorded after every copy; each wait binds to the record
    // enqueued just before it).  The row-group table indexes the full active
    // list: not used for these lists.
    const int32_t* lists = cache->dev_lists;
    hipStream_t cs = cache->copy_stream;
    g.groups = nullptr;
    g.snake = 0;
    g.active = lists;
    g.n_active = lists + s->E;
    rc = hip_status(amoe::launch_grouped(g, stream), "verify_block_cached/hit experts");
    if (rc) return rc;
    timer_mark(ACCEPTMOE_STAGE_FETCH, true, cs);
    for (int f = 0; f < plan.nf; ++f) {
      rc = hip_status(copy_expert(cache, plan, f, cs), "verify_block_cached/fetch");
      if (!rc) {
        if (f == plan.nf - 1) timer_mark(ACCEPTMOE_STAGE_FETCH, false, cs);
        rc = hip_status(hipEventRecord(cache->copy_done, cs), "verify_block_cached/fetch");
      }
      if (!rc) rc = hip_status(hipStreamWaitEvent(stream, cache->copy_done, 0),
                               "verify_block_cached/wait");
      if (rc) return rc;
      g.active = lists + s->E + 1 + f;
      g.n_active = lists + 2 * s->E + 2;  // 1
      rc = hip_status(amoe::launch_grouped(g, stream), "verify_block_cached/fetched expert");
      if (rc) return rc;
    }
  } else if (split) {
    // the large experts' row groups (GEMM), then the small experts
    // (work order, at most 64 rows each: one row group per item)
    amoe::GroupedArgs gs = g;
    gs.gemm_groups = w.groups;
    amoe::GroupedArgs gm = g;
    gm.active = w.active_w;
    gm.n_active = w.n_active + 2;
    gm.groups = nullptr;
    gm.max_rows = nullptr;
    timer_mark(ACCEPTMOE_STAGE_GATEUP, true, stream);
    rc = hip_status(amoe::launch_gemm(gs, stream, 1), "verify_block/large experts gate-up");
    if (!rc && small_rows > 0)
      rc = hip_status(amoe::launch_grouped(gm, stream, 1), "verify_block/experts gate-up");
    if (rc) return rc;
    timer_mark(ACCEPTMOE_STAGE_GATEUP, false, stream);
    timer_mark(ACCEPTMOE_STAGE_DOWN, true, stream);
    rc = hip_status(amoe::launch_gemm(gs, stream, 2), "verify_block/large experts down");
    if (!rc && small_rows > 0)
      rc = hip_status(amoe::launch_grouped(gm, stream, 2), "verify_block/experts down");
    if (rc) return rc;
    timer_mark(ACCEPTMOE_STAGE_DOWN, false, stream);
  } else {
    timer_mark(ACCEPTMOE_STAGE_GATEUP, true, stream);
    rc = hip_status(amoe::launch_grouped(g, stream, 1), "verify_block/experts gate-up");
    if (rc) return rc;
    timer_mark(ACCEPTMOE_STAGE_GATEUP, false, stream);
    timer_mark(ACCEPTMOE_STAGE_DOWN, true, stream);
    rc = hip_status(amoe::launch_grouped(g, stream, 2), "verify_block/experts down");
    if (rc) return rc;
    timer_mark(ACCEPTMOE_STAGE_DOWN, false, stream);
  }
  timer_mark(ACCEPTMOE_STAGE_EXPERTS, false, stream);
  timer_mark(ACCEPTMOE_STAGE_COMBINE, true, stream);
  if (shared && !sh_side) {
    rc = launch_shared(s, in, w, g, stream);
    if (rc) return rc;
  }
  if (sh_side) {
    rc = hip_status(hipStreamWaitEvent(stream, ov->done, 0), "verify_block_overlap/join");
    if (rc) return rc;
  }
  amoe::CombineArgs cb = {};
  cb.N = s->N;
  cb.k = s->k;
  cb.H = s->H;
  cb.act_bf16 = s->act_dtype == ACCEPTMOE_BF16;
  cb.y_perm = w.y_perm;
  cb.inv_pos = g.tok_rows ? nullptr : w.inv_pos;
  cb.gate = topk_gate;
  cb.y_shared = shared ? w.sh_y : nullptr;
  cb.y = out->y;
  rc = hip_status(amoe::launch_combine(cb, stream), "verify_block/combine");
  timer_mark(ACCEPTMOE_STAGE_COMBINE, false, stream);
  return rc;
}

}  // namespace

extern "C" {

const char* acceptmoe_version(void) { return "acceptmoe-mi355x 0.1 (gfx950)"; }

const char* acceptmoe_last_error(void) { return g_err; }

const char* acceptmoe_strerror(int code) {
  switch (code) {
    case ACCEPTMOE_OK:
      return "success";
    case ACCEPTMOE_EINVAL:
      return "invalid argument";
    case ACCEPTMOE_ENOTSUP:
      return "unsupported dtype or flag";
    case ACCEPTMOE_EHIP:
      return "HIP launch failure";
    default:
      return "unknown error";
  }
}

int acceptmoe_set_stage_timer(int32_t stage, hipEvent_t start, hipEvent_t stop) {
  if (stage < ACCEPTMOE_STAGE_NONE || stage > ACCEPTMOE_STAGE_FETCH)
    return fail(ACCEPTMOE_EINVAL, "unknown stage %d", stage);
  g_timer_stage = (start && stop) ? stage : 0;
  g_timer_start = start;
  g_timer_stop = stop;
  return ACCEPTMOE_OK;
}

size_t acceptmoe_select_workspace_size(const acceptmoe_shape* s) {
  if (check_shape(s, false)) return 0;
  Carver c(nullptr);
  carve_select(c, s);
  return c.used;
}

int acceptmoe_select(const acceptmoe_shape* s, const void* x, const void* w_router,
                     const float* b_router, const float* logits_in, const int32_t* parent,
                     const int32_t* depth, const float* commit, const uint8_t* resident,
                     float* logits_out, uint8_t* eligible, int32_t* topk_idx, float* topk_gate,
                     acceptmoe_stats* stats, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s, false);
  if (rc) return rc;
  const bool lin = (s->flags & ACCEPTMOE_F_LOGITS_IN) != 0;
  if (lin ? !logits_in : (!x || !w_router))
    return fail(ACCEPTMOE_EINVAL, lin ? "logits_in is NULL" : "x or w_router is NULL");
  if (!parent || !depth || !commit || !eligible || !topk_idx || !topk_gate || !stats || !ws)
    return fail(ACCEPTMOE_EINVAL, "a required pointer is NULL");
  const size_t need = acceptmoe_select_workspace_size(s);
  if (ws_bytes < need)
    return fail(ACCEPTMOE_EINVAL, "workspace %zu bytes < %zu required", ws_bytes, need);
  Carver c(ws);
  const SelectWs w = carve_select(c, s);
  amoe::SelectArgs a = select_args(s, w);
  a.x = x;
  a.w_router = w_router;
  a.b_router = b_router;
  a.logits_in = logits_in;
  a.parent = parent;
  a.depth = depth;
  a.commit = commit;
  a.resident = resident;
  a.logits_out = logits_out;
  a.eligible = eligible;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.stats = stats;
  return hip_status(amoe::launch_select(a, stream), "acceptmoe_select");
}

int moe_route_permute(int32_t N, int32_t k, int32_t E, const int32_t* topk_idx, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_assign, int32_t* inv_pos,
                      int32_t* active, int32_t* n_active, hipStream_t stream) {
  int rc = check_sizes(N, k, E, 0, 0, ACCEPTMOE_F32, false, false);
  if (rc) return rc;
  if (!topk_idx || !counts || !offsets || !sorted_assign || !inv_pos || !active || !n_active)
    return fail(ACCEPTMOE_EINVAL, "a required pointer is NULL");
  return hip_status(amoe::launch_permute(N, k, E, topk_idx, counts, offsets, sorted_assign,
                                         inv_pos, active, n_active, nullptr, nullptr, stream),
                    "moe_route_permute");
}

size_t moe_grouped_swiglu_workspace_size(int32_t N, int32_t k, int32_t I, int32_t w_dtype) {
  if (N < 1 || k < 1 || I < 1) return 0;
  return align256(static_cast<size_t>(N) * k * I * hidden_elem_bytes(w_dtype));
}

int moe_grouped_swiglu(int32_t N, int32_t k, int32_t E, int32_t H, int32_t I,
                       int32_t act_dtype, int32_t w_dtype, int32_t w_layout, const void* x,
                       const void* w13, const void* w2, const float* s13, const float* s2,
                       const int32_t* offsets, const int32_t* sorted_assign,
                       const int32_t* active, const int32_t* n_active, float* y_perm,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_pair_ok(act_dtype, w_dtype))
    return fail(ACCEPTMOE_ENOTSUP, "unsupported dtype pair (act %d, weights %d)", act_dtype,
                w_dtype);
  if (w_layout != ACCEPTMOE_LAYOUT_ROWMAJOR && w_layout != ACCEPTMOE_LAYOUT_PACKED)
    return fail(ACCEPTMOE_ENOTSUP, "unknown weight layout %d", w_layout);
  if (w_layout == ACCEPTMOE_LAYOUT_PACKED && w_dtype == ACCEPTMOE_F32)
    return fail(ACCEPTMOE_ENOTSUP, "the packed layout needs BF16 or FP8 weights");
  // the shared expert is a call with E = 1, k = 1
  if (N < 1 || N > 4096) return fail(ACCEPTMOE_EINVAL, "N=%d outside [1, 4096]", N);
  if (k < 1 || k > 16 || E < 1 || E > 256)
    return fail(ACCEPTMOE_EINVAL, "k=%d or E=%d out of range", k, E);
  int rc = check_sizes(N, 1, 256, H, I, w_dtype, true, true);
  if (rc) return rc;
  if (!x || !w13 || !w2 || !offsets || !sorted_assign || !active || !n_active || !y_perm || !ws)
    return fail(ACCEPTMOE_EINVAL, "a required pointer is NULL");
  if (w_dtype == ACCEPTMOE_FP8_E4M3FN && (!s13 || !s2))
    return fail(ACCEPTMOE_EINVAL, "FP8 weights need s13 and s2");
  const size_t need = moe_grouped_swiglu_workspace_size(N, k, I, w_dtype);
  if (ws_bytes < need)
    return fail(ACCEPTMOE_EINVAL, "workspace %zu bytes < %zu required", ws_bytes, need);
  amoe::GroupedArgs a = {};
  a.N = N;
  a.k = k;
  a.E = E;
  a.H = H;
  a.I = I;
  a.w_kind = w_kind(w_dtype);
  a.act_bf16 = act_dtype == ACCEPTMOE_BF16;
  a.x = x;
  a.w13 = w13;
  a.w2 = w2;
  a.s13 = s13;
  a.s2 = s2;
  a.offsets = offsets;
  a.sorted_assign = sorted_assign;
  a.active = active;
  a.n_active = n_active;
  a.y_perm = y_perm;
  a.h_perm = ws;
  a.num_cu = num_cu();
  a.packed = w_layout == ACCEPTMOE_LAYOUT_PACKED;
  a.tok_rows = 0;
  // one expert (the shared expert) takes every row: spread its row groups
  a.row_groups = E == 1 ? (N * k + 63) / 64 : 1;
  a.w_slot = nullptr;
  a.n_wslots = 0;
  a.max_rows = nullptr;
  a.groups = nullptr;
  a.snake = 0;
  return hip_status(amoe::launch_grouped(a, stream), "moe_grouped_swiglu");
}

int moe_combine(int32_t N, int32_t k, int32_t H, int32_t act_dtype, const float* y_perm,
                const int32_t* inv_pos, const float* topk_gate, const float* y_shared, void* y,
                hipStream_t stream) {
  if (act_dtype != ACCEPTMOE_F32 && act_dtype != ACCEPTMOE_BF16)
    return fail(ACCEPTMOE_ENOTSUP, "unsupported activation dtype %d", act_dtype);
  if (N < 1 || N > 4096 || k < 1 || k > 16 || H < 64 || H > 16384 || H % 64)
    return fail(ACCEPTMOE_EINVAL, "bad sizes N=%d k=%d H=%d", N, k, H);
  if (!y_perm || !inv_pos || !topk_gate || !y)
    return fail(ACCEPTMOE_EINVAL, "a required pointer is NULL");
  amoe::CombineArgs cb = {};
  cb.N = N;
  cb.k = k;
  cb.H = H;
  cb.act_bf16 = act_dtype == ACCEPTMOE_BF16;
  cb.y_perm = y_perm;
  cb.inv_pos = inv_pos;
  cb.gate = topk_gate;
  cb.y_shared = y_shared;
  cb.y = y;
  return hip_status(amoe::launch_combine(cb, stream), "moe_combine");
}

size_t acceptmoe_packed_size(const acceptmoe_shape* s, int32_t which, int32_t n_experts) {
  if (check_shape(s, true)) return 0;
  if (s->w_dtype == ACCEPTMOE_F32 || (which != 0 && which != 1) || n_experts < 1 ||
      n_experts > 256)
    return 0;
  return amoe::packed_bytes(which, w_kind(s->w_dtype), n_experts, s->H, s->I);
}

int acceptmoe_pack_experts(const acceptmoe_shape* s, int32_t n_experts, const void* w13,
                           const void* w2, void* w13_packed, void* w2_packed,
                           hipStream_t stream) {
  int rc = check_shape(s, true);
  if (rc) return rc;
  if (s->w_dtype == ACCEPTMOE_F32)
    return fail(ACCEPTMOE_ENOTSUP, "the packed layout needs BF16 or FP8 weights");
  if (n_experts < 1 || n_experts > 256)
    return fail(ACCEPTMOE_EINVAL, "n_experts=%d outside [1, 256]", n_experts);
  if ((w13 == nullptr) != (w13_packed == nullptr) || (w2 == nullptr) != (w2_packed == nullptr) ||
      (!w13 && !w2))
    return fail(ACCEPTMOE_EINVAL, "give a source and a destination for w13 and/or w2");
  const int wk = w_kind(s->w_dtype);
  if (w13) {
    rc = hip_status(amoe::launch_pack(0, wk, n_experts, s->H, s->I, w13, w13_packed, stream),
                    "acceptmoe_pack_experts/w13");
    if (rc) return rc;
  }
  if (w2)
    rc = hip_status(amoe::launch_pack(1, wk, n_experts, s->H, s->I, w2, w2_packed, stream),
                    "acceptmoe_pack_experts/w2");
  return rc;
}

size_t acceptmoe_workspace_size(const acceptmoe_shape* s) {
  if (check_shape(s, true)) return 0;
  Carver c(nullptr);
  carve_verify(c, s, true);
  return c.used;
}

int verify_block(const acceptmoe_shape* s, const acceptmoe_inputs* in,
                 const acceptmoe_outputs* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_block(s, in, nullptr, out, nullptr, nullptr, ws, ws_bytes, stream);
}

int verify_block_overlap(const acceptmoe_shape* s, const acceptmoe_inputs* in,
                         const acceptmoe_outputs* out, const acceptmoe_overlap* ov, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (!ov || !ov->side || !ov->start || !ov->done)
    return fail(ACCEPTMOE_EINVAL, "verify_block_overlap: a side stream and two events are "
                "required");
  if (ov->side == stream)
    return fail(ACCEPTMOE_EINVAL, "verify_block_overlap: the side stream is the call's stream");
  return run_block(s, in, nullptr, out, nullptr, ov, ws, ws_bytes, stream);
}

int verify_block_cached(const acceptmoe_shape* s, const acceptmoe_inputs* in,
                        const acceptmoe_expert_cache* cache, const acceptmoe_outputs* out,
                        acceptmoe_cache_report* report, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (!cache) return fail(ACCEPTMOE_EINVAL, "cache is NULL");
  return run_block(s, in, cache, out, report, nullptr, ws, ws_bytes, stream);
}

int acceptmoe_cache_plan(acceptmoe_cache_state* st, const int32_t* active, int32_t n_active,
                         int32_t* fetch_expert, int32_t* fetch_slot, int32_t* n_fetch) {
  int rc = check_state(st);
  if (rc) return rc;
  if (n_active < 0 || n_active > st->E || (n_active > 0 && !active) || !fetch_expert ||
      !fetch_slot || !n_fetch)
    return fail(ACCEPTMOE_EINVAL, "acceptmoe_cache_plan: bad active list or output pointer");
  return plan_fetches(st, active, n_active, fetch_expert, fetch_slot, n_fetch, nullptr);
}

}  // extern "C"
