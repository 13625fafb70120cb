"""GPU parity of the selection path and the permute against the oracle.

Router logits are compared within 1e-4 * max|l_ref| (fp32 accumulation on the
GPU, fp64 in the oracle).  Everything decided from the logits -- eligible
set, top-k indices, statistics -- is then compared bit-exactly by feeding the
GPU's own fp32 logits to the oracle; gates within 1e-6 relative.  A block
whose decision rests on an fp64 near-tie (oracle flag) is counted and
skipped; the seeded workloads have none.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_cases import DT, check_selection, oracle_select, say, shape_of, upload_block

pytestmark = pytest.mark.gpu


def run_select(lib, cfg, b, flags=None, logits_in=None, resident="block"):
    dev = "cuda"
    d = upload_block(b, dev)
    sh = shape_of(lib, cfg)
    if flags is not None:
        sh.flags = flags
    N, E, k = cfg.N, cfg.E, cfg.k
    out = dict(logits_out=torch.empty((N, E), dtype=torch.float32, device=dev),
               eligible=torch.empty(E, dtype=torch.uint8, device=dev),
               topk_idx=torch.empty((N, k), dtype=torch.int32, device=dev),
               topk_gate=torch.empty((N, k), dtype=torch.float32, device=dev),
               stats=lib.new_stats(dev))
    ws = torch.zeros(lib.acceptmoe_select_workspace_size(sh), dtype=torch.uint8, device=dev)
    res = d["resident"] if isinstance(resident, str) else resident
    lin = None if logits_in is None else torch.from_numpy(logits_in).to(dev)
    lib.acceptmoe_select(sh, d["x"], d["w_router"], d["b_router"], lin, d["parent"],
                         d["depth"], d["commit"], res, out["logits_out"], out["eligible"],
                         out["topk_idx"], out["topk_gate"], out["stats"], ws)
    torch.cuda.synchronize()
    return out, lib.decode_stats(out["stats"])


SMALL = [
    ("tiny", {}),
    ("qwen3_30b", dict(E=48, k=6, H=256, N=37)),
    ("gptoss_120b", dict(E=40, k=4, H=320, N=53, resident_slots=15, reroute=5)),
    ("qwen3_235b_b4", dict(E=64, k=8, H=192, N=64)),
    ("dsv31", dict(E=200, k=8, H=384, N=96, n_chains=12, chain_len=8)),
    ("qwen3_30b", dict(E=256, k=16, H=128, N=300)),
    # 16-node router groups in 8-wave work-groups, fused tail: a ragged last
    # group (203 = 12 x 16 + 11), 7 expert tiles over 8 waves
    ("qwen3_30b", dict(E=100, k=6, H=320, N=203)),
    # the same for more than 128 experts from 65 nodes: 10 tiles (two waves
    # take two), last group of 8
    ("dsv31", dict(E=160, k=8, H=256, N=72, n_chains=9, chain_len=8)),
]


@pytest.mark.parametrize("name,over", SMALL)
def test_select_parity_small(lib, name, over):
    cfg = W.CONFIGS[name].with_(**over)
    skipped = 0
    for seed in range(6):
        say(f"select small {name} {over} seed {seed}")
        b = W.make_block(cfg, seed)
        out, st = run_select(lib, cfg, b)
        lg = out["logits_out"].cpu().numpy()
        lref = O.router_logits(W.to_exact_f64(b.x), W.to_exact_f64(b.w_router),
                               None if b.b_router is None else b.b_router.numpy())
        assert np.max(np.abs(lg - lref)) <= 1e-4 * np.max(np.abs(lref))
        ref = oracle_select(cfg, b, logits_in=lg)
        if not check_selection(out, ref, st, cfg, f"{name} seed {seed}"):
            skipped += 1
    assert skipped == 0


FULL = ["tiny", "qwen3_30b", "gptoss_120b", "qwen3_235b", "qwen3_235b_b025", "qwen3_235b_b4",
        "dsv31"]


@pytest.mark.parametrize("name", FULL)
def test_select_parity_full(lib, name):
    cfg = W.CONFIGS[name]
    for seed in range(4 if cfg.N > 64 else 8):
        say(f"select full {name} seed {seed}")
        b = W.make_block(cfg, seed)
        out, st = run_select(lib, cfg, b)
        lg = out["logits_out"].cpu().numpy()
        lref = O.router_logits(W.to_exact_f64(b.x), W.to_exact_f64(b.w_router),
                               None if b.b_router is None else b.b_router.numpy())
        assert np.max(np.abs(lg - lref)) <= 1e-4 * np.max(np.abs(lref))
        ref = oracle_select(cfg, b, logits_in=lg)
        assert check_selection(out, ref, st, cfg, f"{name} seed {seed}")


def test_natural_and_fixed_budget_modes(lib):
    cfg = W.CONFIGS["qwen3_30b"].with_(E=64, H=256, N=40)
    b = W.make_block(cfg, 5)
    out, st = run_select(lib, cfg, b, flags=lib.F_NATURAL)
    lg = out["logits_out"].cpu().numpy()
    ref = oracle_select(cfg, b, logits_in=lg, flags=O.F_NATURAL)
    assert (out["topk_idx"].cpu().numpy() == O.natural_topk(lg, cfg.k)).all()
    assert check_selection(out, ref, st, cfg, "natural")
    for B in (cfg.k, 13, 40, 64):
        c2 = cfg.with_(fixed_budget=B)
        out, st = run_select(lib, c2, b)
        ref = oracle_select(c2, b, logits_in=out["logits_out"].cpu().numpy())
        assert check_selection(out, ref, st, c2, f"budget {B}")
    c3 = cfg.with_(flags=lib.F_NO_RENORM, min_set=20)
    out, st = run_select(lib, c3, b)
    ref = oracle_select(c3, b, logits_in=out["logits_out"].cpu().numpy())
    assert check_selection(out, ref, st, c3, "no renorm + min_set")


def test_logits_in_and_edge_shapes(lib):
    rng = np.random.default_rng(0)
    cases = [
        dict(E=16, k=2, N=1),              # single node: S = its natural top-k
        dict(E=8, k=8, N=5),               # k = E: every expert chosen
        dict(E=1, k=1, N=3),               # one expert
        dict(E=256, k=16, N=4096),         # largest sizes
        dict(E=33, k=3, N=65),             # ragged wave tails
    ]
    for c in cases:
        cfg = W.CONFIGS["qwen3_30b"].with_(H=64, commit=(1.0, 0.6, 0.3), tree="chain", **c)
        N, E = c["N"], c["E"]
        parent = np.full(N, -1, np.int32)
        depth = np.zeros(N, np.int32)
        for i in range(1, N):
            p = int(rng.integers(-1, i))
            if p >= 0 and depth[p] >= 2:
                p = -1
            parent[i] = p
            depth[i] = 0 if p < 0 else depth[p] + 1
        # coarse logits: plenty of exact ties (and -0.0 next to +0.0)
        lg = (rng.integers(-3, 4, (N, E)) * 0.5).astype(np.float32)
        lg[lg == 0] = np.where(rng.random(int((lg == 0).sum())) < 0.5, -0.0, 0.0)
        b = W.make_block(cfg, 0)
        b.parent, b.depth = parent, depth
        say(f"logits_in edge case {c}")
        out, st = run_select(lib, cfg, b, flags=lib.F_LOGITS_IN, logits_in=lg)
        ref = oracle_select(cfg, b, logits_in=lg, flags=0)
        assert (out["logits_out"].cpu().numpy().view(np.uint32) == lg.view(np.uint32)).all()
        # every case is compared: none of them may rest on an fp64 near tie
        assert not ref["near_tie"], f"edge {c}: near tie, pick other inputs"
        assert check_selection(out, ref, st, cfg, f"edge {c}")


def test_device_error_flags(lib):
    cfg = W.CONFIGS["qwen3_30b"].with_(E=32, H=128, N=8)
    b = W.make_block(cfg, 1)
    cases = [
        ("parent later", dict(parent=[-1, 0, 3, 1, 1, 2, 2, 3]), lib.ERR_BAD_TREE),
        ("depth mismatch", dict(depth=[0, 1, 1, 2, 3, 2, 2, 3]), lib.ERR_BAD_TREE),
        ("too deep", dict(depth=[0, 1, 2, 3, 4, 5, 6, 7], parent=[-1, 0, 1, 2, 3, 4, 5, 6]),
         lib.ERR_DEPTH),
    ]
    for name, ch, bit in cases:
        bb = W.make_block(cfg, 1)
        if "parent" in ch:
            bb.parent = np.array(ch["parent"], np.int32)
        if "depth" in ch:
            bb.depth = np.array(ch["depth"], np.int32)
        if name == "parent later":
            bb.depth = np.array([0, 1, 1, 2, 2, 2, 2, 2], np.int32)
        if name == "depth mismatch":
            bb.parent = np.array([-1, 0, 0, 1, 1, 2, 2, 3], np.int32)
        out, st = run_select(lib, cfg, bb)
        assert st["err_flags"] & bit, (name, st)
        assert (out["topk_idx"].cpu().numpy() >= 0).all()
        assert (out["topk_idx"].cpu().numpy() < cfg.E).all()
    bb = W.make_block(cfg, 1)
    bb.commit = np.array([1.0, -0.5, 0.3, 0.2, 0.1, 0.1], np.float32)
    out, st = run_select(lib, cfg, bb)
    assert st["err_flags"] & lib.ERR_COMMIT
    lg = np.zeros((cfg.N, cfg.E), np.float32)
    lg[3, 5] = np.nan
    out, st = run_select(lib, cfg, b, flags=lib.F_LOGITS_IN, logits_in=lg)
    assert st["err_flags"] & lib.ERR_NONFINITE
    ti = out["topk_idx"].cpu().numpy()
    assert ((ti >= 0) & (ti < cfg.E)).all()


@pytest.mark.parametrize("N,k,E", [(1, 1, 1), (64, 8, 128), (37, 3, 7), (4096, 16, 256),
                                   (256, 8, 256), (1000, 2, 5)])
def test_permute_parity(lib, N, k, E):
    rng = np.random.default_rng(N * 31 + k)
    dev = "cuda"
    for trial in range(3):
        if trial == 2:
            idx = np.full((N, k), E - 1, np.int32)           # one expert takes everything
        else:
            idx = rng.integers(0, E, (N, k)).astype(np.int32)
        ti = torch.from_numpy(idx).to(dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sa = torch.empty(N * k, dtype=torch.int32, device=dev)
        ip = torch.empty(N * k, dtype=torch.int32, device=dev)
        active = torch.full((E,), -7, dtype=torch.int32, device=dev)
        na = torch.empty(1, dtype=torch.int32, device=dev)
        lib.moe_route_permute(N, k, E, ti, counts, offsets, sa, ip, active, na)
        torch.cuda.synchronize()
        ref = O.permute(idx, E)
        assert (counts.cpu().numpy() == ref["counts"]).all()
        assert (offsets.cpu().numpy() == ref["offsets"]).all()
        assert (sa.cpu().numpy() == ref["sorted_assign"]).all()
        assert (ip.cpu().numpy() == ref["inv_pos"]).all()
        n = int(na.item())
        assert n == ref["n_active"]
        assert (active.cpu().numpy()[:n] == ref["active"]).all()
        assert (active.cpu().numpy()[n:] == -7).all()


VARIANTS = [
    ("full-softmax demand", 8, 0),
    ("no anchor", 16, 0),
    ("unit commitment", 32, 0),
    ("MoE-Spec B=16", 16 | 32, 16),
    ("MoE-Spec B=24", 16 | 32, 24),
    ("AcceptMoE-B B=16", 0, 16),
    ("full demand, no anchor", 8 | 16, 0),
]


@pytest.mark.parametrize("name,over", [("qwen3_30b", {}), ("gptoss_120b", {}),
                                       ("dsv31", dict(E=64, H=256)),
                                       ("qwen3_30b", dict(E=80, k=4, H=128, N=300))])
@pytest.mark.parametrize("vname,flags,budget", VARIANTS)
def test_selector_variants(lib, name, over, vname, flags, budget):
    """Selector variants (flags on the same kernels) against the oracle with
    the same flags: bit-exact sets, top-k and statistics."""
    cfg = W.CONFIGS[name].with_(fixed_budget=budget, **over)
    for seed in range(3):
        say(f"variant {vname} on {name} {over} seed {seed}")
        b = W.make_block(cfg, seed)
        out, st = run_select(lib, cfg, b, flags=flags)
        lg = out["logits_out"].cpu().numpy()
        ref = oracle_select(cfg, b, logits_in=lg, flags=flags)
        assert check_selection(out, ref, st, cfg, f"{vname} {name} seed {seed}")
        if flags & 16:
            assert st["n_anchor"] == 0
        if budget and not (flags & 16) and cfg.resident_slots == 0:
            assert st["n_eligible"] == max(budget, st["n_anchor"], cfg.k, cfg.min_set)


@pytest.mark.parametrize("N", [40, 300], ids=["tail_topk", "restricted_kernel"])
def test_workspace_misuse_is_flagged_and_repaired(lib, N):
    """A workspace whose arrival counters are not zero (never zero-filled, or
    shared by overlapping calls) must not go unnoticed: the call sets
    ERR_WORKSPACE, keeps every index in range, and leaves the counters at
    zero, so the next call on the same workspace is exact again.  Counters
    set here: a node group's K-slice counter below its slice count (one
    work-group is elected too early), another far above it (none is
    elected), and the restricted kernel's counter."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=32, k=4, H=256, N=N)
    b = W.make_block(cfg, 1)
    d = upload_block(b)
    sh = shape_of(lib, cfg)
    dev = "cuda"
    ws = torch.zeros(lib.acceptmoe_select_workspace_size(sh), dtype=torch.uint8, device=dev)

    def call():
        o = dict(logits_out=torch.empty((N, cfg.E), dtype=torch.float32, device=dev),
                 eligible=torch.empty(cfg.E, dtype=torch.uint8, device=dev),
                 topk_idx=torch.empty((N, cfg.k), dtype=torch.int32, device=dev),
                 topk_gate=torch.empty((N, cfg.k), dtype=torch.float32, device=dev),
                 stats=lib.new_stats(dev))
        lib.acceptmoe_select(sh, d["x"], d["w_router"], d["b_router"], None, d["parent"],
                             d["depth"], d["commit"], None, o["logits_out"], o["eligible"],
                             o["topk_idx"], o["topk_gate"], o["stats"], ws)
        torch.cuda.synchronize()
        return o, lib.decode_stats(o["stats"])

    ref, st0 = call()
    assert st0["err_flags"] == 0
    # workspace layout: counters[2] at byte 0, the node groups' K-slice
    # counters from byte 256 (int index 64)
    c = ws.view(torch.int32)
    c[64 + 0] = 1          # group 0: elected after its first arrival
    c[64 + 1] = 1000       # group 1: never elected
    c[1] = 5               # restricted kernel's arrivals
    torch.cuda.synchronize()
    say(f"workspace misuse N={N}")
    bad, st1 = call()
    assert st1["err_flags"] & lib.ERR_WORKSPACE, st1
    ti = bad["topk_idx"].cpu().numpy()
    assert ((ti >= 0) & (ti < cfg.E)).all()
    assert int(c[64]) == 0 and int(c[65]) == 0 and int(c[1]) == 0 and int(c[0]) == 0
    good, st2 = call()
    assert st2 == st0
    for key in ref:
        assert torch.equal(good[key], ref[key]), key
