"""Pins for the selector variants of the oracle (flags on the same steps).

[AcceptMoE news §01, §04]: MoE-Spec keeps a fixed number B of the
highest-ranked experts per layer and weighs every draft position the same;
AcceptMoE-B is AcceptMoE with a fixed budget B.  Here MoE-Spec is
F_UNIT_COMMIT | F_NO_ANCHOR with fixed_budget = B, and F_DEMAND_FULL is the
literal alternative reading of the demand (every expert's score counts).

Pins: closed forms (a softmax row sums to one, so full demand sums to the
commitment weights), special cases that reduce to the standard selection
(k = E, a table of ones), brute force over all experts on small blocks, and a
hand-built block whose sets follow from its construction.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as W


def _sel(b, cfg, **kw):
    args = dict(k=cfg.k, parent=b.parent, depth=b.depth, commit=b.commit,
                x=W.to_exact_f64(b.x), w_router=W.to_exact_f64(b.w_router),
                b_router=None if b.b_router is None else b.b_router.numpy(),
                min_set=cfg.min_set, fixed_budget=cfg.fixed_budget)
    args.update(kw)
    return O.select(**args)


def _brute_top(D, n):
    """The n experts of largest demand, lower index first on ties."""
    return sorted(sorted(range(len(D)), key=lambda e: e), key=lambda e: -D[e])[:n]


@pytest.mark.parametrize("name,over", [("tiny", {}), ("qwen3_30b", dict(E=32, H=128, N=20)),
                                       ("gptoss_120b", dict(E=24, H=64, N=30))])
def test_full_demand_sums_to_commit_weights(name, over):
    cfg = W.CONFIGS[name].with_(**over)
    for seed in range(3):
        b = W.make_block(cfg, seed)
        s = _sel(b, cfg, flags=O.F_DEMAND_FULL)
        want = sum(float(b.commit[int(d)]) for d in b.depth)
        assert abs(s["demand"].sum() - want) <= 1e-12 * want
        # every expert gets demand from every node with a nonzero weight
        if all(float(b.commit[int(d)]) > 0 for d in b.depth):
            assert (s["demand"] > 0).all()


def test_full_demand_equals_topk_demand_when_k_is_E():
    cfg = W.CONFIGS["tiny"].with_(k=16)
    for seed in range(4):
        b = W.make_block(cfg, seed)
        a = _sel(b, cfg)
        f = _sel(b, cfg, flags=O.F_DEMAND_FULL)
        assert np.array_equal(a["demand"], f["demand"])
        assert np.array_equal(a["eligible"], f["eligible"])


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b"])
def test_unit_commit_is_a_table_of_ones(name):
    cfg = W.CONFIGS[name].with_(E=24, H=64, N=16) if name != "tiny" else W.CONFIGS[name]
    for seed in range(3):
        b = W.make_block(cfg, seed)
        u = _sel(b, cfg, flags=O.F_UNIT_COMMIT)
        o = _sel(b, cfg, commit=np.ones_like(b.commit))
        assert np.array_equal(u["demand"], o["demand"])
        assert np.array_equal(u["eligible"], o["eligible"])
        assert np.array_equal(u["topk_idx"], o["topk_idx"])


@pytest.mark.parametrize("budget", [0, 3, 6])
def test_no_anchor_set_is_the_top_demand_experts(budget):
    cfg = W.CONFIGS["qwen3_30b"].with_(E=20, H=64, N=12, k=2, fixed_budget=budget)
    for seed in range(6):
        b = W.make_block(cfg, seed)
        s = _sel(b, cfg, flags=O.F_NO_ANCHOR)
        D = s["demand"]
        n_raw = budget if budget > 0 else int(math.floor(s["r_eff"] + 0.5))
        n = min(cfg.E, max(n_raw, cfg.k))
        assert s["stats"]["n_anchor"] == 0
        assert sorted(np.flatnonzero(s["eligible"]).tolist()) == sorted(_brute_top(D, n))


@pytest.mark.parametrize("budget", [2, 4, 8])
def test_moe_spec_keeps_the_budget(budget):
    cfg = W.CONFIGS["qwen3_30b"].with_(E=24, H=64, N=16, k=2, fixed_budget=budget)
    for seed in range(4):
        b = W.make_block(cfg, seed)
        s = _sel(b, cfg, flags=O.F_UNIT_COMMIT | O.F_NO_ANCHOR)
        # position-uniform demand, recomputed by brute force from the scores
        p, nat = s["p"], s["nat"]
        D = np.zeros(cfg.E)
        for i in range(cfg.N):
            for e in nat[i]:
                D[int(e)] += p[i, int(e)]
        assert np.allclose(D, s["demand"], rtol=1e-14, atol=0)
        assert int(s["eligible"].sum()) == max(budget, cfg.k)
        assert sorted(np.flatnonzero(s["eligible"]).tolist()) == sorted(
            _brute_top(s["demand"], max(budget, cfg.k)))


def test_anchor_and_commitment_decide_a_small_budget():
    """Root 0 routes to experts 0, 1 with low scores; three children at depth
    1 route to 2, 3 with high scores.  Budget 2, k = 2, E = 6.
    AcceptMoE-B: the anchor {0, 1} fills the budget.  MoE-Spec: no anchor,
    the children's demand wins: {2, 3}.  With commitment 0 for depth 1 the
    children's demand vanishes and even without the anchor {0, 1} is kept."""
    E, k = 6, 2
    lg = np.full((4, E), -4.0, dtype=np.float32)
    lg[0, 0], lg[0, 1] = 1.0, 0.9          # root: experts 0, 1
    for i in (1, 2, 3):
        lg[i, 2], lg[i, 3] = 3.0, 2.5      # children: experts 2, 3
    parent = np.array([-1, 0, 0, 0])
    depth = np.array([0, 1, 1, 1])
    common = dict(k=k, parent=parent, depth=depth, logits_in=lg, fixed_budget=2)
    acc_b = O.select(commit=np.array([1.0, 0.5]), **common)
    assert np.flatnonzero(acc_b["eligible"]).tolist() == [0, 1]
    spec = O.select(commit=np.array([1.0, 0.5]), flags=O.F_UNIT_COMMIT | O.F_NO_ANCHOR, **common)
    assert np.flatnonzero(spec["eligible"]).tolist() == [2, 3]
    nochild = O.select(commit=np.array([1.0, 0.0]), flags=O.F_NO_ANCHOR, **common)
    assert np.flatnonzero(nochild["eligible"]).tolist() == [0, 1]
    # every node's top-k inside the set: children of AcceptMoE-B reroute to {0, 1}
    assert acc_b["topk_idx"][1].tolist() == [0, 1]
    assert spec["topk_idx"][0].tolist() == [2, 3]
