"""GPU tests of physical expert offload (verify_block_cached), with the
copies on the call's stream and on a copy stream overlapping the hit experts.

A sequence of seeded blocks runs through verify_block_cached on an expert
cache of a few device slots.  Each block must give bit-identical outputs to
verify_block on the fully resident weights with the cache's resident mask of
that moment (the same kernels read the same weight bytes, only from slots),
and match the oracle's layer with that mask: the selection bit-exact given
the GPU's logits, y within the dtype's tolerance.  The copies must
follow the oracle's LRU model exactly: the fetched experts, spills, hits and
host-to-device bytes, and the device slot table must equal the host state.
"""

import pytest
import torch

import oracle as O
import workloads as W
from gpu_cases import (TOL, check_selection, expert_fn_from, make_weights, max_rel_err, say,
                       shape_of, shared_fn_from, upload_block)
from oracle.cache import LRUExpertCache

pytestmark = pytest.mark.gpu

CASES = [
    # bf16, residency-aware pruning on (reroute budget 3)
    ("gptoss_120b", dict(E=20, k=4, H=448, I=448, N=53, resident_slots=9, reroute=3), 6, 20),
    # bf16, no pruning: the cache only changes where weights come from
    ("qwen3_30b", dict(E=24, k=4, H=320, I=192, N=37), 8, 24),
    # natural routing: every expert eligible, many misses and spills
    ("qwen3_30b", dict(E=24, k=4, H=320, I=192, N=37, flags=1), 4, 24),
    # fp8 weights with block scales and the shared expert
    ("dsv31", dict(E=20, k=3, H=384, I=256, N=40, n_chains=5, chain_len=8), 8, 20),
    # experts with more than 64 rows (row-group work units)
    ("qwen3_30b", dict(E=12, k=4, H=256, I=320, N=300), 4, 12),
]


def warm_set(cfg, b, slots):
    if b.resident is not None:
        return sorted(int(e) for e in b.resident.nonzero()[0])[:slots]
    return list(range(slots))


@pytest.mark.parametrize("overlap", [False, True], ids=["serial", "overlap"])
@pytest.mark.parametrize("name,over,slots,spill", CASES)
def test_cached_block_matches_resident_block(lib, name, over, slots, spill, overlap):
    cfg = W.CONFIGS[name].with_(**over)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b0 = W.make_block(cfg, 0)
    d0 = upload_block(b0)
    layer = lib.VerifyLayer(shape_of(lib, cfg), dict(w_router=d0["w_router"],
                                                     b_router=d0["b_router"], **w), pack=True)
    plain = layer.variant()
    cache = lib.ExpertCache(layer.shape, slots, spill, layer.w["w13"], layer.w["w2"],
                            device="cuda", overlap=overlap)
    warm = warm_set(cfg, b0, slots)
    cache.reset(warm)
    model = LRUExpertCache(slots, spill, warm)
    per_expert = cache.b13 + cache.b2
    total = 0
    fn, shfn = expert_fn_from(cfg, w), shared_fn_from(cfg, w)
    for seed in range(6):
        say(f"cache {name} {over} slots={slots} spill={spill} overlap={overlap} seed {seed}")
        b = W.make_block(cfg, seed)
        d = upload_block(b)
        res_before = cache.resident.clone().cuda()
        ref = plain.run(d["x"], d["parent"], d["depth"], d["commit"], resident=res_before)
        out = layer.run_cached(cache, d["x"], d["parent"], d["depth"], d["commit"])
        torch.cuda.synchronize()
        rep = layer.report
        for key in ("y", "logits_out", "eligible", "topk_idx", "topk_gate", "counts", "stats"):
            assert torch.equal(out[key], ref[key]), f"seed {seed}: {key} differs"
        st = lib.decode_stats(out["stats"])
        # and against the oracle's layer with the cache's resident mask of
        # that moment (selection bit-exact given the GPU's logits)
        mask = res_before.cpu().numpy().astype(bool)
        lg = out["logits_out"].cpu().numpy()
        oref = O.verify_block(
            k=cfg.k, x=W.to_exact_f64(b.x), expert_fn=fn, parent=b.parent, depth=b.depth,
            commit=b.commit, logits_in=lg, resident=mask, min_set=cfg.min_set,
            fixed_budget=cfg.fixed_budget, reroute_budget=cfg.reroute, flags=cfg.flags,
            shared_fn=shfn)
        assert check_selection(out, oref, st, cfg, f"cached seed {seed}")
        err = max_rel_err(out["y"], oref["y"])
        assert err <= TOL[cfg.w], (seed, err)
        U = st["n_active"]
        assert torch.equal(out["active"][:U], ref["active"][:U])  # entries past U are unset
        active = out["active"][:U].cpu().tolist()
        fetches = model.step(active)
        spilled = sum(1 for _, q in fetches if q >= slots)
        assert rep["n_active"] == U
        assert rep["n_fetched"] == len(fetches) and rep["n_spilled"] == spilled
        assert rep["n_hits"] == U - len(fetches)
        assert rep["h2d_bytes"] == len(fetches) * per_expert
        total += rep["h2d_bytes"]
        assert cache.resident_set() == model.resident()
        for e, q in fetches:
            assert int(cache.expert_slot[e]) == q
        assert torch.equal(cache.dev_expert_slot.cpu(), cache.expert_slot)
        assert torch.equal(cache.dev_resident.cpu(), cache.resident)
        say(f"  U={U} fetched {len(fetches)} (spilled {spilled}) hits {U - len(fetches)}")
    cnt = cache.counters()
    assert cnt["h2d_bytes"] == total
    assert (cnt["hits"], cnt["misses"], cnt["spills"]) == (model.hits, model.misses,
                                                           model.spills)


def test_cached_weights_are_the_experts_bytes(lib):
    # after a block, every persistent slot holds exactly its expert's packed bytes
    cfg = W.CONFIGS["qwen3_30b"].with_(E=16, k=4, H=256, I=256, N=32)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 3)
    d = upload_block(b)
    layer = lib.VerifyLayer(shape_of(lib, cfg), dict(w_router=d["w_router"],
                                                     b_router=d["b_router"], **w), pack=True)
    cache = lib.ExpertCache(layer.shape, 5, 16, layer.w["w13"], layer.w["w2"], device="cuda")
    cache.reset([0, 1])
    layer.run_cached(cache, d["x"], d["parent"], d["depth"], d["commit"])
    torch.cuda.synchronize()
    b13, b2 = cache.b13, cache.b2
    for q in range(5):
        e = int(cache.slot_expert[q])
        if e < 0:
            continue
        assert torch.equal(cache.dev_w13[q * b13:(q + 1) * b13],
                           layer.w["w13"].reshape(-1)[e * b13:(e + 1) * b13])
        assert torch.equal(cache.dev_w2[q * b2:(q + 1) * b2],
                           layer.w["w2"].reshape(-1)[e * b2:(e + 1) * b2])
