"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names what it pins and where the fact comes from.  None of them
re-types the oracle's own formula: they use the pages' worked examples
(tests/golden), closed forms, special cases that reduce to a library routine
(scipy / torch), or alternative characterisations (brute force over subsets).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle as O
from oracle import acceptmoe as A
from oracle import fp8 as F8

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _logits_for_sets(sets, E):
    """Logits whose natural top-k are the given ordered sets (2.0, 1.0, ...)."""
    L = np.zeros((len(sets), E), dtype=np.float32)
    for i, s in enumerate(sets):
        for r, e in enumerate(s):
            L[i, e] = float(len(s) - r)
    return L


# ------------------------------------------------------------ page examples --
def test_blog_16x2_example_union_and_permute():
    """MoE-SD blog, dense vs MoE verification: 4 candidates, 8 assignments,
    5 unique experts, at most 8 (pins natural top-k, permute, reuse)."""
    g = _load("blog_16x2_example.json")
    E, k = g["E"], g["k"]
    L = _logits_for_sets(g["candidates"], E)
    nat = O.natural_topk(L, k)
    assert nat.tolist() == g["candidates"]
    perm = O.permute(nat, E)
    assert int(perm["counts"].sum()) == g["assignments"]
    assert perm["n_active"] == g["unique_experts"]
    assert perm["n_active"] <= g["max_unique_if_disjoint"] == len(g["candidates"]) * k
    want = {}
    for s in g["candidates"]:
        for e in s:
            want[e] = want.get(e, 0) + 1
    assert {int(e): int(perm["counts"][e]) for e in perm["active"]} == want
    # blog's reuse metric for this example: 1 - 5/8
    reuse = 1.0 - perm["n_active"] / float(len(g["candidates"]) * k)
    assert reuse == pytest.approx(0.375)
    # all-eligible selection is natural routing
    s = O.select(k=k, parent=[-1, 0, 1, 2], depth=[0, 1, 2, 3], commit=[1, .7, .45, .3],
                 logits_in=L, flags=O.F_NATURAL)
    assert s["topk_idx"].tolist() == g["candidates"]
    assert s["stats"]["n_active"] == 5 and s["stats"]["reuse"] == pytest.approx(0.375)


def test_blog_16x2_example_as_chain_end_to_end():
    """The blog's 16-expert / top-2 example (dense vs MoE verification) run
    as a draft chain with the tiny layer's commitment table [1, .7, .45, .3]:
    every AcceptMoE step end to end (demand reading, effective rank,
    round-half-up set size, anchor + fill order, restricted top-k with the
    lower-index tie rule, gates, grouping).  The expected values are derived
    here in closed form from the example's logits (2 for a candidate's first
    expert, 1 for its second, 0 elsewhere), not taken from the oracle."""
    g = _load("blog_16x2_example.json")
    E, k = g["E"], g["k"]
    cand = g["candidates"]                      # [[2,7],[2,7],[2,9],[4,11]]
    L = _logits_for_sets(cand, E)
    commit = [1.0, 0.7, 0.45, 0.3]
    s = O.select(k=k, parent=[-1, 0, 1, 2], depth=[0, 1, 2, 3], commit=commit, logits_in=L)
    # scores: exp(2), exp(1), 1 over the row's sum exp(2) + exp(1) + 14
    zr = math.exp(2) + math.exp(1) + 14.0
    p1, p2 = math.exp(2) / zr, math.exp(1) / zr
    want_D = np.zeros(E)
    for i, (a, b) in enumerate(cand):           # a node's demand: c * p of its own top-2
        want_D[a] += commit[i] * p1
        want_D[b] += commit[i] * p2
    np.testing.assert_allclose(s["demand"], want_D, rtol=1e-14, atol=0)
    assert want_D[2] == pytest.approx(2.15 * p1) and want_D[7] == pytest.approx(1.7 * p2)
    r_eff = math.exp(scipy.stats.entropy(want_D[want_D > 0]))
    assert s["r_eff"] == pytest.approx(r_eff, rel=1e-12)
    assert 2.9 < r_eff < 3.0                    # rounds half up to 3
    assert s["n"] == 3 and s["anchor"] == {2, 7}
    # anchor {2, 7}, then the highest remaining demand: E4 (0.3 p1 > 0.45 p2)
    assert sorted(np.nonzero(s["eligible"])[0].tolist()) == [2, 4, 7]
    # node 2 keeps E2 and takes E4 over E7 (both logit 0: lower index);
    # node 3 keeps E4 and takes E2 over E7 the same way
    assert s["topk_idx"].tolist() == [[2, 7], [2, 7], [2, 4], [4, 2]]
    e = math.e
    want_g = [[e / (e + 1), 1 / (e + 1)]] * 2 + [[e * e / (e * e + 1), 1 / (e * e + 1)]] * 2
    np.testing.assert_allclose(s["topk_gate"], np.array(want_g, np.float32), rtol=0, atol=0)
    perm = O.permute(s["topk_idx"], E)
    # assignments i*2+j -> experts [2,7,2,7,2,4,4,2]: stable grouping by expert
    assert perm["sorted_assign"].tolist() == [0, 2, 4, 7, 5, 6, 1, 3]
    assert perm["inv_pos"].tolist() == [0, 6, 1, 7, 2, 4, 5, 3]
    assert {int(x): int(perm["counts"][x]) for x in perm["active"]} == {2: 4, 4: 2, 7: 2}
    assert s["stats"]["n_active"] == 3 and s["stats"]["n_natural_union"] == 5
    assert not s["near_tie"]


def test_blog_tree_example_union():
    """MoE-SD blog, chain vs tree drafts: nodes A..E touch 9 experts."""
    g = _load("blog_tree_example.json")
    names = g["nodes"][1:]
    sets = [g["experts"][n] for n in names]
    L = _logits_for_sets(sets, 11)
    nat = O.natural_topk(L, 2)
    perm = O.permute(nat, 11)
    assert perm["n_active"] == g["unique_experts"]
    assert O.validate_tree(g["parent"], [0, 1, 2, 2, 1, 2], 3) == 0


def test_moesd_expected_union_monte_carlo():
    """MoESD §5.3: with E experts and K uniformly chosen per token, t tokens
    touch E[1 - ((E-K)/E)^t] experts on average.  iid continuous logits make
    every natural top-K set uniform, so the oracle's mean union must match."""
    rng = np.random.default_rng(11)
    for E, K, t, trials in [(16, 2, 4, 4000), (128, 8, 64, 300), (128, 4, 64, 300)]:
        us = []
        for _ in range(trials):
            L = rng.standard_normal((t, E)).astype(np.float32)
            us.append(O.permute(O.natural_topk(L, K), E)["n_active"])
        us = np.array(us, dtype=np.float64)
        expect = E * (1.0 - ((E - K) / E) ** t)
        sem = us.std(ddof=1) / math.sqrt(trials)
        assert abs(us.mean() - expect) < 4 * sem + 1e-9, (E, K, t, us.mean(), expect)


# --------------------------------------------------------------- router ----
def test_router_logits_unit_vectors_and_bias():
    """x = unit vector h picks column h of W_r (catches a transposed operand);
    the bias is added per expert."""
    rng = np.random.default_rng(0)
    E, H = 5, 7
    W = rng.standard_normal((E, H))
    b = rng.standard_normal(E)
    X = np.eye(H)[:4]
    L = O.router_logits(X, W, b)
    assert L.shape == (4, E) and L.dtype == np.float32
    np.testing.assert_array_equal(L, (W[:, :4].T + b[None, :]).astype(np.float32))
    np.testing.assert_array_equal(O.router_logits(2 * X, W), (2 * W[:, :4].T).astype(np.float32))


def test_router_logits_rounds_once_from_exact():
    """fp64 sums of exact products, rounded once: equals an fp64 library
    product (torch) rounded to fp32, not an fp32-accumulated one."""
    rng = np.random.default_rng(1)
    X = rng.standard_normal((6, 300)).astype(np.float32)
    W = rng.standard_normal((9, 300)).astype(np.float32)
    ref = torch.nn.functional.linear(torch.from_numpy(X).double(),
                                     torch.from_numpy(W).double()).float().numpy()
    np.testing.assert_array_equal(O.router_logits(X, W), ref)


# -------------------------------------------------------------- softmax ----
def test_softmax_closed_forms():
    # two experts: logistic function
    a, b = 0.3, -1.7
    p = O.softmax64(np.array([[a, b]], dtype=np.float32))
    assert p[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(float(np.float32(b)) - float(np.float32(a)))), rel=1e-15)
    # equal logits: uniform
    p = O.softmax64(np.zeros((2, 8), dtype=np.float32))
    np.testing.assert_allclose(p, 1.0 / 8, rtol=1e-15)
    # large shift does not overflow; shift invariant
    L = np.array([[1000.0, 999.0, 0.0]], dtype=np.float32)
    np.testing.assert_allclose(O.softmax64(L), O.softmax64(L - 999.0), rtol=1e-14)


def test_softmax_matches_scipy():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((5, 33)).astype(np.float32) * 4
    np.testing.assert_allclose(O.softmax64(L), scipy.special.softmax(L.astype(np.float64), axis=1),
                               rtol=1e-13)


# ---------------------------------------------------------------- top-k ----
def _brute_topk(values, allowed, k):
    """The k-subset whose members each beat every non-member under
    (value desc, index asc), listed best first; found by enumeration."""
    allowed = list(allowed)
    best = None
    for T in itertools.combinations(allowed, k):
        rest = [e for e in allowed if e not in T]
        ok = all((values[a] > values[r]) or (values[a] == values[r] and a < r)
                 for a in T for r in rest)
        if ok:
            assert best is None
            best = sorted(T, key=lambda e: (-values[e], e))
    return best


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(3)
    for _ in range(300):
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        row = rng.integers(0, 3, E).astype(np.float32)  # many ties
        got = O.natural_topk(row[None, :], k)[0].tolist()
        assert got == _brute_topk(row.tolist(), range(E), k)
        mask = rng.integers(0, 2, E).astype(bool)
        if mask.sum() >= k:
            got = O.restricted_topk(row[None, :], mask, k)[0].tolist()
            assert got == _brute_topk(row.tolist(), np.nonzero(mask)[0].tolist(), k)


def test_topk_signed_zero_equal():
    row = np.array([[-0.0, 0.0, -1.0, 0.0]], dtype=np.float32)
    assert O.natural_topk(row, 2)[0].tolist() == [0, 1]
    row = np.array([[0.0, -0.0, -1.0]], dtype=np.float32)
    assert O.natural_topk(row, 2)[0].tolist() == [0, 1]


# ----------------------------------------------------------------- tree -----
def test_validate_tree_bits():
    assert O.validate_tree([-1, 0, 0, 1], [0, 1, 1, 2], 3) == 0
    assert O.validate_tree([-1, 0, -1, 2], [0, 1, 0, 1], 2) == 0          # forest
    assert O.validate_tree([-1, 2, 0], [0, 2, 1], 3) & O.ERR_BAD_TREE        # parent later
    assert O.validate_tree([-1, 0, 1], [0, 1, 1], 3) & O.ERR_BAD_TREE        # depth mismatch
    assert O.validate_tree([-1, 0], [1, 2], 3) & O.ERR_BAD_TREE              # root depth != 0
    assert O.validate_tree([-1, 0, 1], [0, 1, 2], 2) == O.ERR_DEPTH          # too deep
    assert O.validate_tree([0], [0], 1) & O.ERR_BAD_TREE                     # self parent


def test_select_rejects_bad_inputs():
    L = np.zeros((2, 4), dtype=np.float32)
    with pytest.raises(O.OracleInputError) as e:
        O.select(k=1, parent=[-1, 0], depth=[0, 1], commit=[1.0, -0.5], logits_in=L)
    assert e.value.flags == O.ERR_COMMIT
    L[1, 2] = np.inf
    with pytest.raises(O.OracleInputError) as e:
        O.select(k=1, parent=[-1, 0], depth=[0, 1], commit=[1.0, 0.5], logits_in=L)
    assert e.value.flags == O.ERR_NONFINITE


# --------------------------------------------------------------- demand -----
def test_demand_single_root_is_its_scores_on_its_topk():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((1, 10)).astype(np.float32)
    p = scipy.special.softmax(L.astype(np.float64), axis=1)
    nat = O.natural_topk(L, 3)
    D = O.demand(p, nat, [0], [0.8])
    for e in range(10):
        assert D[e] == pytest.approx(0.8 * p[0, e] if e in nat[0] else 0.0, rel=1e-15)


def test_demand_commit_indexed_by_depth():
    """A commit table that is 1 at one depth and 0 elsewhere leaves exactly
    the nodes at that depth (catches a node-indexed or off-by-one commit)."""
    rng = np.random.default_rng(5)
    parent = np.array([-1, 0, 0, 1, 1, 2, 5])
    depth = np.array([0, 1, 1, 2, 2, 2, 3])
    L = rng.standard_normal((7, 12)).astype(np.float32)
    p = O.softmax64(L)
    nat = O.natural_topk(L, 2)
    for d in range(4):
        c = np.zeros(4)
        c[d] = 1.0
        D = O.demand(p, nat, depth, c)
        only = [i for i in range(7) if depth[i] == d]
        D2 = O.demand(p[only], nat[only], np.zeros(len(only), int), [1.0])
        np.testing.assert_allclose(D, D2, rtol=1e-15, atol=0)
    # linear in c, zero outside the natural union, never negative
    c = np.array([1.0, 0.7, 0.4, 0.2])
    D = O.demand(p, nat, depth, c)
    np.testing.assert_allclose(O.demand(p, nat, depth, 2 * c), 2 * D, rtol=1e-15)
    union = set(nat.reshape(-1).tolist())
    assert all((D[e] > 0) == (e in union) for e in range(12))


def test_root_anchor_is_roots_topk_only():
    nat = np.array([[0, 1], [2, 3], [4, 5], [6, 7]])
    assert O.root_anchor(nat, [-1, 0, -1, 2]) == {0, 1, 4, 5}
    assert O.root_anchor(nat, [-1, 0, 1, 2]) == {0, 1}


# ------------------------------------------------------------- self-size ----
def test_effective_rank_closed_forms():
    assert O.effective_rank(np.array([0.3, 0.3, 0.3, 0.0])) == pytest.approx(3.0, rel=1e-14)
    assert O.effective_rank(np.array([5.0])) == pytest.approx(1.0)
    assert O.effective_rank(np.zeros(4)) == 0.0
    a = 0.2
    h2 = -(a * math.log(a) + (1 - a) * math.log(1 - a))
    assert O.effective_rank(np.array([a, 0.0, 1 - a]) * 7) == pytest.approx(math.exp(h2), rel=1e-14)
    # entropy via scipy on a random distribution
    rng = np.random.default_rng(6)
    D = rng.random(40) * (rng.random(40) > 0.3)
    assert O.effective_rank(D) == pytest.approx(math.exp(scipy.stats.entropy(D)), rel=1e-12)


def test_self_size_rules():
    E, k = 16, 2
    assert O.self_size(5.49, 2, E, k, 0, 0)[0] == 5
    assert O.self_size(5.5, 2, E, k, 0, 0)[0] == 6        # half rounds up
    assert O.self_size(1.2, 2, E, k, 0, 0)[0] == 2        # at least k
    assert O.self_size(1.2, 4, E, k, 0, 0)[0] == 4        # at least the anchor
    assert O.self_size(3.0, 2, E, k, 7, 0)[0] == 7        # at least min_set
    assert O.self_size(30.0, 2, E, k, 0, 0)[0] == 16      # at most E
    assert O.self_size(30.0, 2, E, k, 0, 9)[0] == 9       # fixed budget B
    assert O.self_size(30.0, 2, E, k, 3, 0)[1] == 3       # n_min


def _brute_fill(D, anchor, n):
    """Among all n-sets containing the anchor, the one whose non-anchor part
    is best under (demand desc, index asc), found by enumeration."""
    rest = [e for e in range(len(D)) if e not in anchor]
    best = None
    for T in itertools.combinations(rest, n - len(anchor)):
        others = [e for e in rest if e not in T]
        if all(D[a] > D[r] or (D[a] == D[r] and a < r) for a in T for r in others):
            assert best is None
            best = set(T) | set(anchor)
    return best


def test_fill_bruteforce():
    rng = np.random.default_rng(7)
    for _ in range(300):
        E = int(rng.integers(2, 8))
        D = rng.integers(0, 4, E).astype(np.float64) * rng.random()   # ties and zeros
        anchor = set(rng.choice(E, int(rng.integers(0, E)), replace=False).tolist())
        n = int(rng.integers(len(anchor), E + 1))
        mask, _, _ = O.fill_eligible(D, anchor, n)
        assert set(np.nonzero(mask)[0].tolist()) == _brute_fill(D, anchor, n)


def test_fill_max_demand_sum_when_distinct():
    """With distinct demands the filled set maximises total demand among all
    n-sets that contain the anchor."""
    rng = np.random.default_rng(8)
    for _ in range(100):
        E = 7
        D = rng.random(E)
        anchor = {int(rng.integers(E))}
        n = int(rng.integers(1, E + 1))
        mask, _, _ = O.fill_eligible(D, anchor, n)
        best = max((set(T) for T in itertools.combinations(range(E), n) if anchor <= set(T)),
                   key=lambda T: sum(D[e] for e in T))
        assert set(np.nonzero(mask)[0].tolist()) == best


# ------------------------------------------------------------------ RAP -----
def test_prune_bruteforce_and_limits():
    rng = np.random.default_rng(9)
    for _ in range(400):
        E = int(rng.integers(3, 9))
        D = rng.integers(0, 4, E).astype(np.float64)
        elig = rng.random(E) < 0.7
        anchor = set(e for e in np.nonzero(elig)[0].tolist() if rng.random() < 0.3)
        resident = (rng.random(E) < 0.5).astype(np.uint8)
        R = int(rng.integers(0, 4))
        n_min = int(rng.integers(1, max(2, elig.sum() + 1)))
        if elig.sum() < n_min:
            continue
        new, cand, nrm = O.residency_prune(elig, anchor, D, resident, R, n_min)
        removed = set(np.nonzero(elig & ~new)[0].tolist())
        kept = set(np.nonzero(new)[0].tolist())
        assert kept <= set(np.nonzero(elig)[0].tolist())
        assert len(removed) == nrm <= R
        assert new.sum() >= n_min
        assert all(not resident[e] and e not in anchor for e in removed)
        pool = [e for e in np.nonzero(elig)[0] if not resident[e] and e not in anchor]
        # as many removed as the limits allow
        assert nrm == min(R, int(elig.sum()) - n_min, len(pool))
        # every removed expert precedes every kept candidate in (D asc, idx desc)
        for r in removed:
            for q in pool:
                if q not in removed:
                    assert D[r] < D[q] or (D[r] == D[q] and r > q)
        # all-resident mask: no-op
        new2, _, n2 = O.residency_prune(elig, anchor, D, np.ones(E, np.uint8), R, n_min)
        assert n2 == 0 and (new2 == elig).all()


# ---------------------------------------------------------------- gates -----
def test_gates_closed_forms():
    rng = np.random.default_rng(10)
    L = rng.standard_normal((4, 9)).astype(np.float32)
    p = O.softmax64(L)
    sel = O.natural_topk(L, 3)
    g = O.gates(p, sel)
    np.testing.assert_allclose(g.astype(np.float64).sum(1), 1.0, rtol=1e-6)
    for i in range(4):
        a, b = sel[i, 0], sel[i, 1]
        assert g[i, 0] / g[i, 1] == pytest.approx(math.exp(float(L[i, a]) - float(L[i, b])), rel=1e-6)
    assert (O.gates(p, sel[:, :1]) == 1.0).all()
    graw = O.gates(p, sel, renorm=False)
    np.testing.assert_allclose(graw, np.take_along_axis(scipy.special.softmax(L.astype(np.float64), 1), sel, 1),
                               rtol=1e-7)


# -------------------------------------------------------------- permute -----
def test_permute_properties():
    rng = np.random.default_rng(12)
    for _ in range(50):
        E = int(rng.integers(1, 20))
        N = int(rng.integers(1, 30))
        k = int(rng.integers(1, min(E, 4) + 1))
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(N)])
        P = O.permute(idx, E)
        flat = idx.reshape(-1)
        assert P["offsets"][0] == 0 and P["offsets"][-1] == N * k
        for e in range(E):
            seg = P["sorted_assign"][P["offsets"][e]:P["offsets"][e + 1]]
            assert (flat[seg] == e).all()
            assert (np.diff(seg) > 0).all()          # stable: ascending assignment ids
        assert (P["sorted_assign"][P["inv_pos"]] == np.arange(N * k)).all()
        assert P["active"].tolist() == sorted(set(flat.tolist()))


# -------------------------------------------------------------- experts -----
def test_swiglu_matches_torch_dense_ffn():
    """E = 1, k = 1 reduces the layer to a dense SwiGLU FFN (torch)."""
    rng = np.random.default_rng(13)
    N, H, I = 5, 16, 24
    x = rng.standard_normal((N, H))
    wg, wu, wd = (rng.standard_normal((I, H)) * 0.3, rng.standard_normal((I, H)) * 0.3,
                  rng.standard_normal((H, I)) * 0.3)
    t = lambda a: torch.from_numpy(a)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(t(x), t(wg))) *
        torch.nn.functional.linear(t(x), t(wu)), t(wd)).numpy()
    np.testing.assert_allclose(O.swiglu(x, wg, wu, wd), ref, rtol=1e-12, atol=1e-12)
    w13 = np.stack([wg, wu])[None]
    w2 = wd[None]
    out = O.verify_block(k=1, x=x, expert_fn=A.dense_expert_fn(w13, w2),
                         parent=[-1] + list(range(N - 1)), depth=list(range(N)),
                         commit=[1.0] * N, logits_in=np.zeros((N, 1), np.float32))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_give_routing_independent_output():
    """Every expert equal and gates summing to one: y_i = SwiGLU(x_i) whatever
    the routing (catches a wrong inv_pos / gate pairing or a dropped term)."""
    rng = np.random.default_rng(14)
    N, E, k, H, I = 9, 6, 3, 8, 12
    x = rng.standard_normal((N, H))
    wg, wu, wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    fn = lambda e: (wg, wu, wd)
    L = rng.standard_normal((N, E)).astype(np.float32)
    parent = [-1] + [int(rng.integers(i)) for i in range(1, N)]
    depth = [0] * N
    for i in range(1, N):
        depth[i] = depth[parent[i]] + 1
    out = O.verify_block(k=k, x=x, expert_fn=fn, parent=parent, depth=depth,
                         commit=[1.0] * (max(depth) + 1), logits_in=L)
    # gates are stored in fp32, so they sum to one within fp32 rounding
    ref = O.swiglu(x, wg, wu, wd)
    np.testing.assert_allclose(out["y"], ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_grouped_equals_per_token_definition():
    """The grouped pipeline (permute, group GEMM, combine) equals the layer's
    per-token definition y = sum_j g_j E_j(x) + E_shared(x)."""
    rng = np.random.default_rng(15)
    N, E, k, H, I = 11, 7, 2, 8, 10
    x = rng.standard_normal((N, H))
    w13 = rng.standard_normal((E, 2, I, H))
    w2 = rng.standard_normal((E, H, I))
    sh = (rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))
    fn = A.dense_expert_fn(w13, w2)
    L = rng.standard_normal((N, E)).astype(np.float32)
    out = O.verify_block(k=k, x=x, expert_fn=fn, parent=[-1] * N, depth=[0] * N,
                         commit=[1.0], logits_in=L, shared_fn=lambda: sh, min_set=4)
    ref = O.token_outputs(x, out["topk_idx"], out["topk_gate"], fn, shared_fn=lambda: sh)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ fp8 -----
def test_fp8_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F8.decode_table()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_fp8_decode_spec_points():
    for pt in _load("ocp_e4m3fn_points.json")["points"]:
        v = F8.decode_e4m3fn(int(pt["code"], 16))
        if pt["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == pt["value"] and math.copysign(1, v) == math.copysign(1, pt["value"])


def test_fp8_block_scales_index_rows_then_cols():
    """A scale grid that differs per block row and column maps block (r, c)
    to rows 128r.. and columns 128c.. (catches transposed scale indexing)."""
    codes = np.full((256, 384), 0x38, dtype=np.uint8)       # every weight 1.0
    scales = np.arange(6, dtype=np.float64).reshape(2, 3) + 1
    w = F8.dequant_blocks(codes, scales)
    for r in range(2):
        for c in range(3):
            assert (w[128 * r:128 * (r + 1), 128 * c:128 * (c + 1)] == scales[r, c]).all()


def test_bytes_per_fp8_expert_matches_ecospec():
    """EcoSpec Fig. 1(c): one DeepSeek-V3.1 FP8 expert moves 44.04 MB."""
    import workloads as W
    cfg = W.CONFIGS["dsv31"]
    assert cfg.expert_bytes() == 7168 * 2048 * 3
    assert round(cfg.expert_bytes() / 1e6, 2) == 44.04
