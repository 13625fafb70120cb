"""The expert cache's fetch plan (acceptmoe_cache_plan, host only) against the
oracle's LRU model, a hand-traced sequence, brute force over the block
history, and its error handling.  No GPU: the plan is host code."""

import numpy as np
import pytest

from oracle.cache import LRUExpertCache


@pytest.fixture(scope="module")
def m():
    import moe_speculative_decoding_gemm_amd as m
    return m


def make(m, E, n_slots, n_spill):
    shape = m.make_shape(64, 256, 256, E, 4, 6)
    return m.ExpertCache(shape, n_slots, n_spill)


def test_hand_traced_sequence(m):
    # 4 slots, 2 spill slots.  Block 2: expert 2 hits; 5 takes the empty slot
    # 3; 7 evicts slot 0 (experts 1 and 3 are equally old: lowest slot); 9
    # evicts slot 2.  Block 3: 1 evicts slot 0 (7, 2, 9 equally old), 5 hits,
    # 10 and 11 take slots 1 and 2, and 12 finds every slot held by an
    # expert of this block: spill slot 4.
    c = make(m, 16, 4, 2)
    assert c.plan([1, 2, 3]) == [(1, 0), (2, 1), (3, 2)]
    assert c.plan([2, 5, 7, 9]) == [(5, 3), (7, 0), (9, 2)]
    assert c.plan([1, 5, 10, 11, 12]) == [(1, 0), (10, 1), (11, 2), (12, 4)]
    assert c.resident_set() == {1, 5, 10, 11}
    cnt = c.counters()
    assert (cnt["clock"], cnt["hits"], cnt["misses"], cnt["spills"]) == (3, 2, 10, 1)
    # the spilled expert has a slot for this block only; next time it misses
    assert int(c.expert_slot[12]) == 4 and int(c.resident[12]) == 0
    # every persistent slot was last used in block 3: the lowest is evicted
    assert c.plan([12]) == [(12, 0)]
    assert c.resident_set() == {12, 5, 10, 11}
    o = LRUExpertCache(4, 2)
    for a in ([1, 2, 3], [2, 5, 7, 9], [1, 5, 10, 11, 12]):
        o.step(a)
    assert o.step([12]) == [(12, 0)]


def zipf_blocks(rng, E, n_blocks, lo, hi):
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    perm = rng.permutation(E)
    out = []
    for _ in range(n_blocks):
        n = int(rng.integers(lo, hi + 1))
        out.append(sorted(int(perm[i]) for i in rng.choice(E, size=n, replace=False, p=p)))
    return out


@pytest.mark.parametrize("E,slots,spill,lo,hi", [(64, 16, 64, 4, 24), (128, 48, 80, 10, 60),
                                                  (16, 4, 12, 1, 16), (32, 0, 32, 1, 8)])
def test_plan_matches_oracle(m, E, slots, spill, lo, hi):
    rng = np.random.default_rng([E, slots, spill])
    c = make(m, E, slots, spill)
    o = LRUExpertCache(slots, spill)
    for a in zipf_blocks(rng, E, 150, lo, hi):
        assert c.plan(a) == o.step(a)
        assert c.resident_set() == o.resident()
        for q in range(slots):
            e = int(c.slot_expert[q])
            assert (None if e < 0 else e) == o.holder[q]
    cnt = c.counters()
    assert (cnt["hits"], cnt["misses"], cnt["spills"]) == (o.hits, o.misses, o.spills)


def test_warm_start_and_lru_by_brute_force(m):
    # every eviction must take, among resident experts not active in the
    # block, the one whose last active block (from the whole history; 0 for a
    # warm-start expert never used) is oldest, lowest slot on ties
    E, S = 48, 12
    rng = np.random.default_rng(5)
    c = make(m, E, S, E)
    warm = list(range(S))
    c.reset(warm)
    last = {e: 0 for e in warm}
    for b, a in enumerate(zipf_blocks(rng, E, 200, 2, 14), start=1):
        before = {q: int(c.slot_expert[q]) for q in range(S)}
        res_before = c.resident_set()
        fetches = c.plan(a)
        assert [e for e, _ in fetches] == [e for e in a if e not in res_before]
        assert set(a) <= c.resident_set() | {e for e, q in fetches if q >= S}
        taken = set()
        for e, q in fetches:
            if q >= S:
                continue
            old = before[q]
            if old >= 0 and old not in taken:
                cands = [s for s in range(S) if before[s] >= 0 and before[s] not in a
                         and s not in taken]
                best = min(cands, key=lambda s: (last.get(before[s], 0), s))
                assert q == best
            taken.add(q)
        for e in a:
            last[e] = b


def test_spill_exhaustion_leaves_state_unchanged(m):
    c = make(m, 16, 2, 0)
    assert c.plan([0, 1]) == [(0, 0), (1, 1)]
    snap = (c.slot_expert.clone(), c.expert_slot.clone(), c.resident.clone(),
            c.last_use.clone(), c.counters())
    with pytest.raises(m.AcceptMoEError) as ei:
        c.plan([3, 4, 5])
    assert ei.value.code == m.EINVAL
    assert all(bool((x == y).all()) for x, y in zip(snap[:4], (c.slot_expert, c.expert_slot,
                                                                c.resident, c.last_use)))
    assert c.counters() == snap[4]


@pytest.mark.parametrize("active", [[1, 1], [-1], [16], [3, 99]])
def test_bad_active_lists(m, active):
    c = make(m, 16, 4, 4)
    with pytest.raises(m.AcceptMoEError) as ei:
        c.plan(active)
    assert ei.value.code == m.EINVAL


def test_inconsistent_state_rejected(m):
    c = make(m, 16, 4, 4)
    c.slot_expert[0] = 3  # slot 0 claims expert 3, whose tables say it is nowhere
    with pytest.raises(m.AcceptMoEError) as ei:
        c.plan([1])
    assert ei.value.code == m.EINVAL
    # a warm start whose expert side disagrees with the slot table: the plan
    # would otherwise count the expert as a hit and index last_use by its slot
    for bad_slot in (-1, 7, 2):
        c = make(m, 16, 4, 4)
        c.reset([5, 6])
        c.resident[9] = 1            # resident, but no slot holds expert 9
        c.expert_slot[9] = bad_slot  # -1, a spill slot, or slot 2 (empty)
        before = (c.slot_expert.clone(), c.expert_slot.clone(), c.resident.clone())
        with pytest.raises(m.AcceptMoEError) as ei:
            c.plan([9])
        assert ei.value.code == m.EINVAL
        assert all(a.equal(b) for a, b in zip(before, (c.slot_expert, c.expert_slot,
                                                        c.resident)))
    # a non-resident expert that names a persistent slot
    c = make(m, 16, 4, 4)
    c.reset([5, 6])
    c.expert_slot[2] = 1
    with pytest.raises(m.AcceptMoEError) as ei:
        c.plan([2])
    assert ei.value.code == m.EINVAL
    # a spill slot from the previous block is a valid state
    c = make(m, 16, 1, 2)
    c.plan([1, 2])                   # 2 spills into slot 1
    assert int(c.expert_slot[2]) == 1 and int(c.resident[2]) == 0
    assert c.plan([2]) == [(2, 0)]


def test_cached_block_argument_checks(m):
    # every call below fails validation before it reaches the device
    import ctypes as C
    lib = m.raw()
    shape = m.make_shape(64, 256, 256, 16, 4, 6)  # row-major bf16
    fake = C.c_void_p(0x1000)
    inp = m.Inputs(*([fake.value] * 16))
    out = m.Outputs(*([fake.value] * 8))
    c = make(m, 16, 4, 4)
    desc = m.ExpertCacheDesc(C.addressof(c.state), *([fake.value] * 6))
    rc = lib.verify_block_cached(C.byref(shape), C.byref(inp), None, C.byref(out), None,
                                 fake, 1 << 30, None)
    assert rc == m.EINVAL
    rc = lib.verify_block_cached(C.byref(shape), C.byref(inp), C.byref(desc), C.byref(out),
                                 None, fake, 1 << 30, None)
    assert rc == m.ENOTSUP  # the cache holds packed weights only
    shape.w_layout = m.LAYOUT_PACKED
    shape.E = 32  # the state was made for E = 16
    rc = lib.verify_block_cached(C.byref(shape), C.byref(inp), C.byref(desc), C.byref(out),
                                 None, fake, 1 << 30, None)
    assert rc == m.EINVAL
