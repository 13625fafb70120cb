"""Brute force on tiny blocks: the oracle's selection against an enumeration.

Every set decision (natural top-k, fill, pruning, restricted top-k) is found
here by enumerating subsets and keeping the one that satisfies the defining
property, instead of by sorting; the composite is checked over every
topological tree with up to 4 nodes, several logit draws, every resident mask
on 5 experts, several pruning budgets and minimum sizes.
"""

import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle as O


def _beats(vals, a, b, desc=True):
    if desc:
        return vals[a] > vals[b] or (vals[a] == vals[b] and a < b)
    return vals[a] < vals[b] or (vals[a] == vals[b] and a > b)


def _best_subset(pool, size, vals, desc=True):
    for T in itertools.combinations(pool, size):
        others = [e for e in pool if e not in T]
        if all(_beats(vals, a, r, desc) for a in T for r in others):
            return set(T)
    raise AssertionError("no subset satisfies the order")


def _brute_select(L, parent, depth, commit, k, resident, R, min_set, budget, natural):
    N, E = L.shape
    vals = [[float(v) for v in row] for row in L]
    p = scipy.special.softmax(L.astype(np.float64), axis=1)
    nat = [_best_subset(list(range(E)), k, vals[i]) for i in range(N)]
    D = [0.0] * E
    for i in range(N):
        for e in sorted(nat[i]):
            D[e] += commit[depth[i]] * p[i, e]
    anchor = set()
    for i in range(N):
        if parent[i] == -1:
            anchor |= nat[i]
    tot = sum(D)
    reff = 0.0 if tot == 0 else math.exp(-sum((d / tot) * math.log(d / tot) for d in D if d > 0))
    n_min = max(k, min_set)
    n = min(E, max(budget if budget > 0 else int(math.floor(reff + 0.5)), len(anchor), n_min))
    if natural:
        S = set(range(E))
    else:
        rest = [e for e in range(E) if e not in anchor]
        S = anchor | _best_subset(rest, n - len(anchor), D)
        if resident is not None:
            cand = [e for e in sorted(S) if e not in anchor and not resident[e]]
            m = max(0, min(R, len(S) - n_min, len(cand)))
            S = S - _best_subset(cand, m, D, desc=False)
    sel = [sorted(_best_subset(sorted(S), k, vals[i]), key=lambda e: (-vals[i][e], e))
           for i in range(N)]
    return S, sel, reff


def _trees(nmax):
    for n in range(1, nmax + 1):
        for par in itertools.product(*[range(-1, i) for i in range(n)]):
            depth = []
            for i, p in enumerate(par):
                depth.append(0 if p == -1 else depth[p] + 1)
            yield list(par), depth


@pytest.mark.parametrize("k", [1, 2])
def test_select_matches_bruteforce_exhaustive_small(k):
    rng = np.random.default_rng(100 + k)
    E = 5
    masks = [None] + [np.array(m, dtype=np.uint8) for m in itertools.product([0, 1], repeat=E)]
    checked = 0
    for parent, depth in _trees(4):
        commit = [1.0, 0.6, 0.35, 0.2]
        for draw in range(2):
            # coarse logits create ties in both scores and demand
            L = (rng.integers(-2, 3, (len(parent), E)) * 0.5).astype(np.float32)
            if draw == 1:
                L = rng.standard_normal((len(parent), E)).astype(np.float32)
            for mi, res in enumerate(masks):
                if mi % 4 != draw * 2 % 4 and res is not None:
                    continue
                for R, min_set, budget in [(0, 0, 0), (1, 0, 0), (3, 0, 0), (2, 3, 0), (5, 0, 4)]:
                    S, sel, reff = _brute_select(L, parent, depth, commit, k, res, R,
                                                 min_set, budget, False)
                    got = O.select(k=k, parent=parent, depth=depth, commit=commit,
                                   logits_in=L, resident=res, reroute_budget=R,
                                   min_set=min_set, fixed_budget=budget)
                    assert set(np.nonzero(got["eligible"])[0].tolist()) == S
                    assert got["topk_idx"].tolist() == sel
                    assert got["r_eff"] == pytest.approx(reff, rel=1e-12, abs=1e-15)
                    checked += 1
            S, sel, _ = _brute_select(L, parent, depth, commit, k, None, 0, 0, 0, True)
            got = O.select(k=k, parent=parent, depth=depth, commit=commit, logits_in=L,
                           flags=O.F_NATURAL)
            assert got["topk_idx"].tolist() == sel and got["eligible"].all()
    assert checked > 1000
