"""Plain, slow CPU oracle of the AcceptMoE verify-block MoE layer (numpy, fp64).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library and does not load it.

What it computes, step by step, in the order the sources give it (citation
tags are defined in :mod:`oracle`):

1. router logits and softmax scores               [MoE-SD blog, MoE layer]
2. each node's natural top-k experts               [MoE-SD blog, MoE layer]
3. commitment-weighted demand per expert           [AcceptMoE news §02; abstract]
4. root anchor (roots' natural top-k)              [AcceptMoE news §02]
5. self-sizing from the effective rank of demand   [AcceptMoE news §02]
6. residency-aware pruning                         [AcceptMoE news §02; abstract]
7. top-k restricted to the eligible set, gates     [AcceptMoE abstract; MoE-SD blog]
8. permute / group by expert                       [MoE-SD blog, MoE layer]
9. SwiGLU experts over the unique active experts   [MoE-SD blog, MoE layer]
10. unpermute and gate-weighted combine            [MoE-SD blog, MoE layer]

Readings taken where the pages are silent (each also listed in the design doc):

* effective rank = exp(Shannon entropy, natural log) of the normalised demand,
  with 0 ln 0 = 0; a demand total of zero gives effective rank 0.
* demand sums, over nodes, the commitment probability of the node's depth
  times the node's softmax score of every expert in the node's natural top-k
  (not of all experts).
* the set size is round-half-up of the effective rank (or the fixed budget B),
  clamped below by the anchor size and by n_min = max(k, min_set), above by E.
* fill order and the top-k order: larger value first, lower expert index on
  ties; -0.0 and +0.0 compare equal.
* pruning removes non-resident, non-anchor eligible experts in the order
  (demand ascending, index descending), at most R of them, stopping at n_min,
  with no replacement.
* gates are the softmax scores of the chosen k renormalised to sum to one
  (raw scores under ``F_NO_RENORM``).
* selector variants ([AcceptMoE news §01, §04]): MoE-Spec keeps a fixed
  number B of the highest-ranked experts per layer and weighs every draft
  position the same when it aggregates router scores; here that is
  ``F_UNIT_COMMIT | F_NO_ANCHOR`` with ``fixed_budget = B``, the scores
  aggregated as in AcceptMoE (natural top-k of each node).  AcceptMoE-B is
  AcceptMoE with ``fixed_budget = B``.  ``F_DEMAND_FULL`` takes the literal
  alternative reading of the demand: every expert's softmax score counts.
* the expert FFN is SwiGLU: silu(x Wg^T) * (x Wu^T), then times Wd^T, no biases.

Parity status: every public function here is pinned by the CPU tests
(``tests/test_oracle_pins.py``, ``tests/test_oracle_bruteforce.py``,
``tests/test_oracle_invariants.py``).  The readings above have no worked
example on the pages; they are pinned only by closed forms, invariants and
brute force under the stated reading.
"""

from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np

# flags (same meaning as the library's, defined independently here)
F_NATURAL = 1 << 0    # every expert eligible: natural routing
F_NO_RENORM = 1 << 1  # gates are the raw softmax scores of the chosen experts
F_LOGITS_IN = 1 << 2  # logits are given, the router product is skipped
# selector variants on the same steps (baselines the pages compare against)
F_DEMAND_FULL = 1 << 3   # demand sums every expert's score, not only the natural top-k's
F_NO_ANCHOR = 1 << 4     # no root anchor
F_UNIT_COMMIT = 1 << 5   # every draft position weighs 1 (commitment table ignored)

# error bits for inputs the method cannot process
ERR_BAD_TREE = 1 << 0   # a node's parent is not an earlier node, or depths disagree
ERR_DEPTH = 1 << 1      # a depth outside [0, n_depth)
ERR_NONFINITE = 1 << 2  # a non-finite router logit
ERR_COMMIT = 1 << 3     # a negative or non-finite commitment probability

NEAR_TIE_REL = 1e-9


class OracleInputError(ValueError):
    """Raised for inputs that the method does not define (carries error bits)."""

    def __init__(self, flags: int, msg: str):
        super().__init__(msg)
        self.flags = flags


# ---------------------------------------------------------------- step 1 --
def router_logits(x, w_router, b_router=None) -> np.ndarray:
    """Router logits l = x W_r^T (+ b_r) for every node.

    [MoE-SD blog, MoE layer]: the router scores each expert from the token's
    hidden state through a linear map; the optional per-expert bias is the
    configs' shared bias.  Products are summed in fp64 from the exact input
    values and the result is rounded once to fp32, the precision the scores
    are kept in from here on.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_router, dtype=np.float64)
    logits = x64 @ w64.T
    if b_router is not None:
        logits = logits + np.asarray(b_router, dtype=np.float64)[None, :]
    return logits.astype(np.float32)


def softmax64(logits) -> np.ndarray:
    """Row softmax in fp64: p_ie = exp(l_ie - m_i) / sum_e exp(l_ie - m_i).

    [MoE-SD blog, MoE layer]: the router's scores are a softmax over all E
    routed experts.  m_i is the row maximum (it cancels; it keeps exp finite).
    """
    l64 = np.asarray(logits, dtype=np.float64)
    m = l64.max(axis=1, keepdims=True)
    e = np.exp(l64 - m)
    return e / e.sum(axis=1, keepdims=True)


def _order_desc(values, candidates) -> list:
    """Candidates sorted by (value descending, index ascending)."""
    return sorted(candidates, key=lambda e: (-float(values[e]), e))


def natural_topk(logits, k: int) -> np.ndarray:
    """Each node's natural top-k experts, best first.

    [MoE-SD blog, MoE layer]: a node is routed to the k experts with the
    highest router score.  The softmax is monotone, so ranking fp32 logits
    ranks the scores; ties go to the lower expert index.
    """
    logits = np.asarray(logits)
    n, e = logits.shape
    out = np.empty((n, k), dtype=np.int32)
    for i in range(n):
        out[i] = _order_desc(logits[i], range(e))[:k]
    return out


# ---------------------------------------------------------------- checks --
def validate_tree(parent, depth, n_depth: int) -> int:
    """Error bits for a draft tree given as parent pointers and depths.

    [MoE-SD blog, chain vs tree drafts; KV rollback]: a verification block is
    a tree (a forest for batched blocks) of draft nodes; each node has one
    parent and lies one level below it.  Nodes are in topological order here:
    a root has parent -1 and depth 0; every other node's parent is an earlier
    node.
    """
    parent = np.asarray(parent)
    depth = np.asarray(depth)
    flags = 0
    n = len(parent)
    for i in range(n):
        p = int(parent[i])
        d = int(depth[i])
        if d < 0 or d >= n_depth:
            flags |= ERR_DEPTH
        if p == -1:
            if d != 0:
                flags |= ERR_BAD_TREE
        elif not (0 <= p < i):
            flags |= ERR_BAD_TREE
        elif d != int(depth[p]) + 1:
            flags |= ERR_BAD_TREE
    return flags


# ---------------------------------------------------------------- step 3 --
def demand(p, nat, depth, commit, full: bool = False) -> np.ndarray:
    """Commitment-weighted demand D_e = sum_i c[depth_i] * p_ie * [e in nat_i].

    [AcceptMoE news §02; AcceptMoE abstract]: the router's scores are weighted
    by each node's commitment probability (the chance that the node ends up in
    the accepted prefix, estimated offline per draft position) and summed per
    expert.  Only the experts a node would itself route to count for it.
    ``full``: the literal alternative reading, D_e = sum_i c[depth_i] * p_ie
    over every expert.  Nodes are summed in index order.
    """
    p = np.asarray(p, dtype=np.float64)
    nat = np.asarray(nat)
    n, e = p.shape
    D = np.zeros(e, dtype=np.float64)
    for i in range(n):
        w = float(commit[int(depth[i])])
        experts = range(e) if full else (int(ex) for ex in nat[i])
        for ex in experts:
            D[ex] += w * p[i, ex]
    return D


# ---------------------------------------------------------------- step 4 --
def root_anchor(nat, parent) -> set:
    """Anchor set: the natural top-k experts of every root node.

    [AcceptMoE news §02]: the root is always committed, so the experts it
    routes to are always kept.  A batched block has one root per sequence.
    """
    nat = np.asarray(nat)
    parent = np.asarray(parent)
    anchor = set()
    for i in range(len(parent)):
        if int(parent[i]) == -1:
            anchor.update(int(ex) for ex in nat[i])
    return anchor


# ---------------------------------------------------------------- step 5 --
def effective_rank(D) -> float:
    """exp(H(q)) with q = D / sum(D), H the Shannon entropy in nats.

    [AcceptMoE news §02]: the size of the eligible set follows the effective
    rank of the demand distribution (concentrated demand, small set).  The
    pages give no formula; the entropy form is the stated reading.
    """
    D = np.asarray(D, dtype=np.float64)
    total = float(D.sum())
    if total == 0.0:
        return 0.0
    h = 0.0
    for d in D:
        if d > 0.0:
            q = float(d) / total
            h -= q * math.log(q)
    return math.exp(h)


def self_size(r_eff: float, n_anchor: int, E: int, k: int, min_set: int,
              fixed_budget: int):
    """Eligible-set size n and the floor n_min.

    [AcceptMoE news §02, §04]: AcceptMoE sizes the set itself; AcceptMoE-B
    uses a fixed budget B.  n = min(E, max(round_half_up(r_eff) or B, |A|,
    n_min)), n_min = max(k, min_set).
    """
    n_raw = fixed_budget if fixed_budget > 0 else int(math.floor(r_eff + 0.5))
    n_min = max(k, min_set)
    n = min(E, max(n_raw, n_anchor, n_min))
    return n, n_min


def fill_eligible(D, anchor, n: int):
    """S = anchor plus the (n - |anchor|) highest-demand other experts.

    [AcceptMoE news §02]: after the anchor, the rest of the set is taken by
    demand.  Order: demand descending, lower index first on ties.  Returns the
    eligible mask and the ordered list of non-anchor experts (for margins).
    """
    D = np.asarray(D, dtype=np.float64)
    E = len(D)
    rest = _order_desc(D, [e for e in range(E) if e not in anchor])
    take = n - len(anchor)
    eligible = np.zeros(E, dtype=bool)
    for e in anchor:
        eligible[e] = True
    for e in rest[:take]:
        eligible[e] = True
    return eligible, rest, take


# ---------------------------------------------------------------- step 6 --
def residency_prune(eligible, anchor, D, resident, R: int, n_min: int):
    """Residency-aware pruning.

    [AcceptMoE news §02; AcceptMoE abstract]: under offloading, eligibility
    follows what is resident on the GPU: low-demand non-resident experts are
    examined first and dropped, within the rerouting budget R and without
    shrinking the set below its minimum size.  Anchors are never dropped.
    Returns (new mask, ordered candidate list, number removed).
    """
    D = np.asarray(D, dtype=np.float64)
    elig = np.array(eligible, dtype=bool).copy()
    cand = [e for e in range(len(D))
            if elig[e] and e not in anchor and not bool(resident[e])]
    cand = sorted(cand, key=lambda e: (float(D[e]), -e))
    n_remove = max(0, min(R, int(elig.sum()) - n_min, len(cand)))
    for e in cand[:n_remove]:
        elig[e] = False
    return elig, cand, n_remove


# ---------------------------------------------------------------- step 7 --
def restricted_topk(logits, eligible, k: int) -> np.ndarray:
    """Each node's top-k over the eligible experts only.

    [AcceptMoE abstract]: AcceptMoE constrains which target experts are
    eligible; the node then routes as usual among them.  Same order and tie
    rule as the natural top-k.
    """
    logits = np.asarray(logits)
    allowed = [e for e in range(logits.shape[1]) if eligible[e]]
    out = np.empty((logits.shape[0], k), dtype=np.int32)
    for i in range(logits.shape[0]):
        out[i] = _order_desc(logits[i], allowed)[:k]
    return out


def gates(p, sel, renorm: bool = True) -> np.ndarray:
    """Gate weights of the chosen experts (fp64 arithmetic, stored as fp32).

    [MoE-SD blog, MoE layer]: the layer output weights each chosen expert by
    a gate g_e(x); here the chosen experts' softmax scores, renormalised to
    sum to one unless ``renorm`` is False.
    """
    p = np.asarray(p, dtype=np.float64)
    sel = np.asarray(sel)
    g = np.empty(sel.shape, dtype=np.float64)
    for i in range(sel.shape[0]):
        ps = np.array([p[i, int(e)] for e in sel[i]], dtype=np.float64)
        g[i] = ps / ps.sum() if renorm else ps
    return g.astype(np.float32)


# ---------------------------------------------------------------- step 8 --
def permute(topk_idx, E: int) -> dict:
    """Group the N*k assignments by expert.

    [MoE-SD blog, MoE layer]: assignments a = i*k + j are grouped by expert
    so each active expert runs once on its tokens.  counts[e], exclusive
    offsets[E+1], sorted_assign = stable sort of the assignments by expert,
    inv_pos = its inverse, active = experts with at least one assignment in
    ascending order.
    """
    flat = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_assign = np.argsort(flat, kind="stable").astype(np.int32)
    inv_pos = np.empty_like(sorted_assign)
    inv_pos[sorted_assign] = np.arange(len(flat), dtype=np.int32)
    active = np.nonzero(counts)[0].astype(np.int32)
    return dict(counts=counts, offsets=offsets, sorted_assign=sorted_assign,
                inv_pos=inv_pos, active=active, n_active=int(len(active)))


# ---------------------------------------------------------------- step 9 --
def swiglu(x_rows, w_gate, w_up, w_down) -> np.ndarray:
    """One SwiGLU expert: (silu(x Wg^T) * (x Wu^T)) Wd^T, in fp64.

    The expert FFN form comes from the model shapes (gated linear unit with
    SiLU); the pages only define E_e(x) abstractly [MoE-SD blog, MoE layer].
    silu(z) = z / (1 + exp(-z)).
    """
    x = np.asarray(x_rows, dtype=np.float64)
    g = x @ np.asarray(w_gate, dtype=np.float64).T
    u = x @ np.asarray(w_up, dtype=np.float64).T
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return h @ np.asarray(w_down, dtype=np.float64).T


ExpertFn = Callable[[int], tuple]


def grouped_swiglu(x, expert_fn: ExpertFn, perm: dict, k: int) -> np.ndarray:
    """Run each active expert once on its grouped tokens -> y_perm[N*k, H].

    [MoE-SD blog, MoE layer; EcoSpec Fig. 1]: only the unique active experts
    are evaluated; each processes the tokens assigned to it, in grouped order.
    ``expert_fn(e)`` returns (Wg [I,H], Wu [I,H], Wd [H,I]) as exact values.
    """
    x = np.asarray(x, dtype=np.float64)
    offsets = perm["offsets"]
    sorted_assign = perm["sorted_assign"]
    rows = len(sorted_assign)
    y_perm = None
    for e in perm["active"]:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        toks = sorted_assign[lo:hi] // k
        wg, wu, wd = expert_fn(int(e))
        ye = swiglu(x[toks], wg, wu, wd)
        if y_perm is None:
            y_perm = np.zeros((rows, ye.shape[1]), dtype=np.float64)
        y_perm[lo:hi] = ye
    if y_perm is None:
        y_perm = np.zeros((rows, x.shape[1]), dtype=np.float64)
    return y_perm


# --------------------------------------------------------------- step 10 --
def combine(y_perm, inv_pos, gate, k: int, y_shared=None) -> np.ndarray:
    """y_i = sum_j g_ij * y_perm[inv_pos[i*k+j]] (+ shared expert output).

    [MoE-SD blog, MoE layer]: outputs are un-permuted and summed with the
    gate weights; an always-on shared expert adds its output unweighted.
    """
    gate = np.asarray(gate, dtype=np.float64)
    n = gate.shape[0]
    y = np.zeros((n, y_perm.shape[1]), dtype=np.float64)
    for i in range(n):
        for j in range(k):
            y[i] += gate[i, j] * y_perm[int(inv_pos[i * k + j])]
    if y_shared is not None:
        y = y + np.asarray(y_shared, dtype=np.float64)
    return y


def token_outputs(x, sel, gate, expert_fn: ExpertFn, shared_fn=None,
                  tokens=None) -> np.ndarray:
    """The layer output straight from its definition, one token at a time.

    [MoE-SD blog, MoE layer]: y = sum over the token's chosen experts of
    g_e(x) E_e(x), plus E_shared(x).  No grouping; used for sampled checks at
    full size.
    """
    x = np.asarray(x, dtype=np.float64)
    tokens = range(x.shape[0]) if tokens is None else tokens
    out = []
    for i in tokens:
        acc = None
        for j in range(len(sel[i])):
            wg, wu, wd = expert_fn(int(sel[i][j]))
            term = float(gate[i][j]) * swiglu(x[i:i + 1], wg, wu, wd)[0]
            acc = term if acc is None else acc + term
        if shared_fn is not None:
            wg, wu, wd = shared_fn()
            acc = acc + swiglu(x[i:i + 1], wg, wu, wd)[0]
        out.append(acc)
    return np.array(out)


# ------------------------------------------------------------- composite --
def _rel_gap(a: float, b: float) -> float:
    if a == b == 0.0:
        return math.inf  # exact zeros compare the same on every machine
    return abs(a - b) / max(abs(a), abs(b))


def select(*, k: int, parent, depth, commit, x=None, w_router=None,
           b_router=None, logits_in=None, resident=None, min_set: int = 0,
           fixed_budget: int = 0, reroute_budget: int = 0,
           flags: int = 0) -> dict:
    """Steps 1-7 for one verification block; returns every intermediate.

    Raises :class:`OracleInputError` (with error bits) for a malformed tree,
    an out-of-range depth, a bad commitment table or a non-finite logit.

    ``near_tie`` reports whether a decision rests on an fp64 comparison within
    a relative 1e-9 (the fill boundary, the pruning boundary, or the effective
    rank within 1e-9 of a half-integer); such a block may legitimately differ
    from another correct implementation by that one decision.
    """
    parent = np.asarray(parent)
    depth = np.asarray(depth)
    commit = np.asarray(commit, dtype=np.float64)
    n_depth = len(commit)
    err = validate_tree(parent, depth, n_depth)
    if not np.all(np.isfinite(commit)) or np.any(commit < 0):
        err |= ERR_COMMIT
    if logits_in is not None:
        logits = np.asarray(logits_in, dtype=np.float32)
    else:
        logits = router_logits(x, w_router, b_router)
    if not np.all(np.isfinite(logits)):
        err |= ERR_NONFINITE
    if err:
        raise OracleInputError(err, f"invalid verification block (bits {err:#x})")
    N, E = logits.shape
    p = softmax64(logits)
    nat = natural_topk(logits, k)
    weights = np.ones(n_depth, dtype=np.float64) if flags & F_UNIT_COMMIT else commit
    D = demand(p, nat, depth, weights, full=bool(flags & F_DEMAND_FULL))
    anchor = set() if flags & F_NO_ANCHOR else root_anchor(nat, parent)
    r_eff = effective_rank(D)
    n, n_min = self_size(r_eff, len(anchor), E, k, min_set, fixed_budget)
    margins = {}
    natural = bool(flags & F_NATURAL)
    if natural:
        eligible = np.ones(E, dtype=bool)
        n_selfsize = E
        n_pruned = 0
    else:
        eligible, rest, take = fill_eligible(D, anchor, n)
        n_selfsize = int(eligible.sum())
        if 0 < take < len(rest):
            margins["fill"] = _rel_gap(float(D[rest[take - 1]]), float(D[rest[take]]))
        if fixed_budget == 0 and r_eff > 0.0:
            margins["r_eff"] = abs(r_eff - (math.floor(r_eff) + 0.5)) / max(r_eff, 1.0)
        n_pruned = 0
        if resident is not None:
            eligible, cand, n_pruned = residency_prune(
                eligible, anchor, D, np.asarray(resident), reroute_budget, n_min)
            if 0 < n_pruned < len(cand):
                margins["prune"] = _rel_gap(float(D[cand[n_pruned - 1]]),
                                            float(D[cand[n_pruned]]))
    sel = restricted_topk(logits, eligible, k)
    g = gates(p, sel, renorm=not (flags & F_NO_RENORM))
    union_nat = len(set(int(e) for e in nat.reshape(-1)))
    used = sorted(set(int(e) for e in sel.reshape(-1)))
    n_nonres = 0 if resident is None else sum(1 for e in used if not resident[e])
    stats = dict(
        n_anchor=len(anchor), n_selfsize=n_selfsize,
        n_eligible=int(eligible.sum()), n_pruned=int(n_pruned),
        n_active=len(used), n_active_nonresident=int(n_nonres),
        n_natural_union=union_nat, r_eff=float(r_eff),
        demand_total=float(D.sum()), err_flags=0,
        reuse=1.0 - len(used) / float(N * k),
    )
    near_tie = any(v < NEAR_TIE_REL for v in margins.values())
    return dict(logits=logits, p=p, nat=nat, demand=D, anchor=anchor,
                r_eff=r_eff, n=n, n_min=n_min, eligible=eligible, topk_idx=sel,
                topk_gate=g, stats=stats, margins=margins, near_tie=near_tie)


def verify_block(*, k: int, x, expert_fn: ExpertFn, parent, depth, commit,
                 w_router=None, b_router=None, logits_in=None, resident=None,
                 min_set: int = 0, fixed_budget: int = 0,
                 reroute_budget: int = 0, flags: int = 0,
                 shared_fn: Optional[Callable[[], tuple]] = None) -> dict:
    """The whole layer for one verification block: steps 1-10."""
    s = select(k=k, parent=parent, depth=depth, commit=commit, x=x,
               w_router=w_router, b_router=b_router, logits_in=logits_in,
               resident=resident, min_set=min_set, fixed_budget=fixed_budget,
               reroute_budget=reroute_budget, flags=flags)
    E = s["logits"].shape[1]
    perm = permute(s["topk_idx"], E)
    y_perm = grouped_swiglu(x, expert_fn, perm, k)
    y_shared = None
    if shared_fn is not None:
        wg, wu, wd = shared_fn()
        y_shared = swiglu(x, wg, wu, wd)
    y = combine(y_perm, perm["inv_pos"], s["topk_gate"], k, y_shared)
    s.update(perm=perm, y_perm=y_perm, y_shared=y_shared, y=y)
    return s


# ---------------------------------------------------------- expert access --
def dense_expert_fn(w13, w2) -> ExpertFn:
    """Expert accessor for float weights w13[E,2,I,H] (gate, up), w2[E,H,I]."""
    def fn(e):
        return (np.asarray(w13[e][0], dtype=np.float64),
                np.asarray(w13[e][1], dtype=np.float64),
                np.asarray(w2[e], dtype=np.float64))
    return fn
