"""GPU parity of the whole layer (verify_block) and of the separate entry
points against the oracle.

Selection is made identical by handing the GPU's fp32 logits to the oracle
(the logits themselves are checked within 1e-4 * max|l_ref|); the layer
output y must then be within tol * max|y_ref| of the oracle's fp64 layer:
tol = 1e-4 for fp32, 2e-2 for bf16, 6e-2 for fp8 weights.  Small shapes span
several tiles with ragged tails; every full workload shape is checked on all
tokens (the larger ones also on two tokens against the per-token definition
of the layer).
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_cases import (TOL, check_selection, expert_fn_from, expert_fn_streaming, make_weights,
                       max_rel_err, oracle_select, say, shape_of, shared_fn_from, upload_block)

pytestmark = pytest.mark.gpu


def run_layer(lib, cfg, b, w, flags=None, pack=None):
    d = upload_block(b)
    sh = shape_of(lib, cfg)
    if flags is not None:
        sh.flags = flags
    weights = dict(w_router=d["w_router"], b_router=d["b_router"], **w)
    layer = lib.VerifyLayer(sh, weights, pack=pack)
    out = layer.run(d["x"], d["parent"], d["depth"], d["commit"], resident=d["resident"])
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in out.items()}, lib.decode_stats(out["stats"])


def oracle_layer(cfg, b, w, logits):
    return O.verify_block(
        k=cfg.k, x=W.to_exact_f64(b.x), expert_fn=expert_fn_from(cfg, w), parent=b.parent,
        depth=b.depth, commit=b.commit, logits_in=logits, resident=b.resident,
        min_set=cfg.min_set, fixed_budget=cfg.fixed_budget, reroute_budget=cfg.reroute,
        flags=cfg.flags, shared_fn=shared_fn_from(cfg, w))


SMALL = [
    # fp32 weights: the tiny layer and a ragged multi-tile variant
    ("tiny", {}),
    ("tiny", dict(E=12, k=3, H=192, I=320, N=23, tree="eagle", eagle_steps=3, eagle_width=4)),
    # bf16: ragged token groups, I and H not multiples of 128
    ("qwen3_30b", dict(E=24, k=4, H=320, I=192, N=37)),
    ("gptoss_120b", dict(E=20, k=4, H=448, I=448, N=53, resident_slots=9, reroute=3)),
    ("qwen3_235b_b025", dict(E=32, k=8, H=256, I=384, N=64)),
    # fp8 weights with block scales and the shared expert; chains of 8
    ("dsv31", dict(E=20, k=3, H=384, I=256, N=40, n_chains=5, chain_len=8)),
    ("dsv31", dict(E=48, k=8, H=256, I=512, N=96, n_chains=12, chain_len=8)),
    # more than 256 nodes: the restricted top-k runs as a kernel of its own
    ("qwen3_30b", dict(E=40, k=6, H=192, I=128, N=300)),
    # more work items than two per CU: the expert kernels cut items between
    # work-groups (gate/up, then down; fp8 with the shared expert)
    ("qwen3_30b", dict(E=40, k=8, H=192, I=2112, N=64)),
    ("qwen3_30b", dict(E=40, k=8, H=2112, I=192, N=64)),
    ("dsv31", dict(E=24, k=8, H=256, I=2304, N=64, n_chains=8, chain_len=8)),
    # natural routing over 40 experts: 3-tile items (48 weight rows) in both
    # projections, with a shorter last item per expert (32 and 16 tiles)
    ("qwen3_30b", dict(E=40, k=8, H=256, I=256, N=64, flags=1)),
    # more than 64 rows per expert (up to ~200): each item's row groups run as
    # separate units next to each other
    ("qwen3_30b", dict(E=12, k=4, H=256, I=320, N=300)),
    ("dsv31", dict(E=10, k=3, H=256, I=256, N=200, n_chains=25, chain_len=8)),
    # 256 or more routed rows per expert on average, packed weights: the
    # GEMM tiling (two 64-row items per work-group, 128-row groups), fp8 with
    # the shared expert, bf16 with an odd number of 64-row items per expert
    ("dsv31", dict(E=10, k=3, H=256, I=256, N=1000, n_chains=125, chain_len=8)),
    ("qwen3_30b", dict(E=24, k=4, H=384, I=320, N=1560)),
    # the largest sizes: 4096 nodes (thousands of rows per expert, dozens of
    # 64-row groups each), and 256 experts with top-16
    ("qwen3_30b", dict(E=16, k=8, H=128, I=128, N=4096)),
    ("qwen3_30b", dict(E=256, k=16, H=128, I=128, N=64)),
]


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "rowmajor"])
@pytest.mark.parametrize("name,over", SMALL)
def test_layer_parity_small(lib, name, over, pack):
    cfg = W.CONFIGS[name].with_(**over)
    if pack and cfg.w == "f32":
        pytest.skip("the packed layout is for bf16 / fp8 weights")
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    for seed in range(3):
        say(f"layer small {name} {over} pack={pack} seed {seed}")
        b = W.make_block(cfg, seed)
        out, st = run_layer(lib, cfg, b, w, pack=pack)
        lg = out["logits_out"].cpu().numpy()
        lref = O.router_logits(W.to_exact_f64(b.x), W.to_exact_f64(b.w_router),
                               None if b.b_router is None else b.b_router.numpy())
        assert np.max(np.abs(lg - lref)) <= 1e-4 * np.max(np.abs(lref))
        ref = oracle_layer(cfg, b, w, lg)
        assert check_selection(out, ref, st, cfg, f"{name} seed {seed}")
        assert st["n_active"] == ref["perm"]["n_active"]
        assert (out["counts"].cpu().numpy() == ref["perm"]["counts"]).all()
        err = max_rel_err(out["y"], ref["y"])
        say(f"  U={st['n_active']} |S|={st['n_eligible']} rel err {err:.2e}")
        assert err <= TOL[cfg.w], err


def test_layer_parity_full_tiny_and_qwen3_30b(lib):
    for name in ["tiny", "qwen3_30b"]:
        cfg = W.CONFIGS[name]
        w = make_weights(cfg, device="cuda", gen_device="cpu" if name == "tiny" else "cuda")
        for seed in range(2):
            say(f"layer full {name} seed {seed}")
            b = W.make_block(cfg, seed)
            out, st = run_layer(lib, cfg, b, w)
            ref = oracle_layer(cfg, b, w, out["logits_out"].cpu().numpy())
            assert check_selection(out, ref, st, cfg, f"{name} seed {seed}")
            err = max_rel_err(out["y"], ref["y"])
            say(f"  U={st['n_active']} rel err {err:.2e}")
            assert err <= TOL[cfg.w]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,tokens", [("gptoss_120b", [0, 63]),
                                         ("qwen3_235b_b025", [0, 40]),
                                         ("qwen3_235b", [0, 40]),
                                         ("qwen3_235b_b4", [1, 33]),
                                         ("dsv31", [0, 129])])
def test_layer_parity_full(lib, name, tokens):
    """Full-size layers on every token: y[N, H] against the oracle's grouped
    layer (each active expert evaluated once in fp64, the shared expert
    added for the DeepSeek-shaped layer), max-abs error over the whole output
    within tol * max|y_ref| of the whole output; the selection bit-exact given
    the GPU's logits.  Two tokens are also checked against the per-token
    definition y_i = sum_j g_ij E_sel_ij(x_i) (+ shared) as a cross-check of
    the oracle's grouping."""
    cfg = W.CONFIGS[name]
    say(f"layer full {name}: generating weights")
    w = make_weights(cfg, device="cuda")
    b = W.make_block(cfg, 0)
    out, st = run_layer(lib, cfg, b, w)
    lg = out["logits_out"].cpu().numpy()
    sel = oracle_select(cfg, b, logits_in=lg)
    assert check_selection(out, sel, st, cfg, name)
    active = O.permute(sel["topk_idx"], cfg.E)["active"]
    say(f"  U={st['n_active']} |S|={st['n_eligible']}: oracle layer over {len(active)} experts")
    ref = O.verify_block(
        k=cfg.k, x=W.to_exact_f64(b.x), expert_fn=expert_fn_streaming(cfg, w, active),
        parent=b.parent, depth=b.depth, commit=b.commit, logits_in=lg, resident=b.resident,
        min_set=cfg.min_set, fixed_budget=cfg.fixed_budget, reroute_budget=cfg.reroute,
        flags=cfg.flags, shared_fn=shared_fn_from(cfg, w))
    assert (ref["topk_idx"] == sel["topk_idx"]).all()
    err = max_rel_err(out["y"], ref["y"])
    say(f"  whole-output rel err {err:.2e} (tol {TOL[cfg.w]})")
    assert err <= TOL[cfg.w], err
    fn = expert_fn_from(cfg, w, cache_size=0)
    y_tok = O.token_outputs(W.to_exact_f64(b.x), ref["topk_idx"], ref["topk_gate"], fn,
                            shared_fn=shared_fn_from(cfg, w), tokens=tokens)
    assert np.max(np.abs(y_tok - ref["y"][tokens])) <= 1e-9 * np.max(np.abs(ref["y"]))


@pytest.mark.timeout(900)
def test_layer_parity_full_4096_natural(lib):
    """The large-batch regime at its full size: the Qwen3-30B-shaped layer
    under natural routing (standard speculative decoding) for 512 chains of
    8 tokens, N = 4096 -- ~118 active experts with ~280 routed rows on
    average and thousands for the most routed ones, so every active expert
    runs in the GEMM kernels.  The whole y[4096, 2048] against the oracle's
    grouped layer, the selection bit-exact given the GPU's logits."""
    from workloads.gen import _CHAIN8_COMMIT
    cfg = W.CONFIGS["qwen3_30b"].with_(tree="chains", commit=_CHAIN8_COMMIT, flags=1,
                                       resident_slots=0, shared=False, N=4096,
                                       n_chains=512, chain_len=8)
    say("layer full 4096 natural: generating weights")
    w = make_weights(cfg, device="cuda")
    b = W.make_block(cfg, 0)
    out, st = run_layer(lib, cfg, b, w)
    lg = out["logits_out"].cpu().numpy()
    sel = oracle_select(cfg, b, logits_in=lg)
    assert check_selection(out, sel, st, cfg, "4096 natural")
    assert (out["topk_idx"].cpu().numpy() == O.natural_topk(lg, cfg.k)).all()
    active = O.permute(sel["topk_idx"], cfg.E)["active"]
    rows = np.bincount(sel["topk_idx"].ravel(), minlength=cfg.E)
    say(f"  U={st['n_active']}, most routed rows {rows.max()}: oracle layer")
    assert rows.max() > 256  # the GEMM tiling's regime
    ref = O.verify_block(
        k=cfg.k, x=W.to_exact_f64(b.x), expert_fn=expert_fn_streaming(cfg, w, active),
        parent=b.parent, depth=b.depth, commit=b.commit, logits_in=lg, resident=b.resident,
        min_set=cfg.min_set, fixed_budget=cfg.fixed_budget, reroute_budget=cfg.reroute,
        flags=cfg.flags)
    assert (ref["topk_idx"] == sel["topk_idx"]).all()
    err = max_rel_err(out["y"], ref["y"])
    say(f"  whole-output rel err {err:.2e} (tol {TOL[cfg.w]})")
    assert err <= TOL[cfg.w], err


@pytest.mark.parametrize("pack", [False, True], ids=["rowmajor", "packed"])
def test_separate_entry_points_match_verify_block(lib, pack):
    """acceptmoe_select -> moe_route_permute -> moe_grouped_swiglu (+ shared)
    -> moe_combine reproduces verify_block bit for bit, for either weight
    layout (the grouped call gets the layout verify_block used)."""
    cfg = W.CONFIGS["dsv31"].with_(E=24, k=4, H=256, I=384, N=32, n_chains=4, chain_len=8)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 2)
    out, st = run_layer(lib, cfg, b, w, pack=pack)
    d = upload_block(b)
    dev = "cuda"
    sh = shape_of(lib, cfg)
    N, H, I, E, k = cfg.N, cfg.H, cfg.I, cfg.E, cfg.k
    e_ = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=dev)
    elig, ti, tg = e_(E, dt=torch.uint8), e_(N, k), e_(N, k, dt=torch.float32)
    stats = lib.new_stats(dev)
    ws = torch.zeros(lib.acceptmoe_select_workspace_size(sh), dtype=torch.uint8, device=dev)
    lib.acceptmoe_select(sh, d["x"], d["w_router"], d["b_router"], None, d["parent"],
                         d["depth"], d["commit"], None, None, elig, ti, tg, stats, ws)
    counts, offsets, sa, ip, act, na = e_(E), e_(E + 1), e_(N * k), e_(N * k), e_(E), e_(1)
    lib.moe_route_permute(N, k, E, ti, counts, offsets, sa, ip, act, na)
    layout = lib.LAYOUT_PACKED if pack else lib.LAYOUT_ROWMAJOR
    w13, w2, w13s, w2s = w["w13"], w["w2"], w["w13_shared"][None], w["w2_shared"][None]
    if pack:
        psh = shape_of(lib, cfg, w_layout=lib.LAYOUT_PACKED)
        w13, w2 = lib.pack_experts(psh, w13, w2, E)
        w13s, w2s = lib.pack_experts(psh, w13s, w2s, 1)
    y_perm = e_(N * k, H, dt=torch.float32)
    gws = torch.zeros(lib.moe_grouped_swiglu_workspace_size(N, k, I, 2), dtype=torch.uint8,
                      device=dev)
    lib.moe_grouped_swiglu(N, k, E, H, I, 1, 2, d["x"], w13, w2, w["s13"], w["s2"],
                           offsets, sa, act, na, y_perm, gws, w_layout=layout)
    # shared expert = one-expert grouped call
    so = torch.tensor([0, N], dtype=torch.int32, device=dev)
    ss = torch.arange(N, dtype=torch.int32, device=dev)
    y_sh = e_(N, H, dt=torch.float32)
    sws = torch.zeros(lib.moe_grouped_swiglu_workspace_size(N, 1, I, 2), dtype=torch.uint8,
                      device=dev)
    lib.moe_grouped_swiglu(N, 1, 1, H, I, 1, 2, d["x"], w13s, w2s, w["s13_shared"][None],
                           w["s2_shared"][None], so, ss, torch.zeros(1, dtype=torch.int32, device=dev),
                           torch.ones(1, dtype=torch.int32, device=dev), y_sh, sws,
                           w_layout=layout)
    y = e_(N, H, dt=torch.bfloat16)
    lib.moe_combine(N, k, H, 1, y_perm, ip, tg, y_sh, y)
    torch.cuda.synchronize()
    assert torch.equal(ti, out["topk_idx"]) and torch.equal(tg, out["topk_gate"])
    assert torch.equal(y.view(torch.int16), out["y"].view(torch.int16))


@pytest.mark.parametrize("over", [dict(E=64, H=512, I=256, N=64),
                                  dict(E=40, k=8, H=192, I=2112, N=64)],
                         ids=["whole_items", "split_items"])
def test_determinism(lib, over):
    cfg = W.CONFIGS["qwen3_30b"].with_(**over)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 4)
    o1, s1 = run_layer(lib, cfg, b, w)
    o2, s2 = run_layer(lib, cfg, b, w)
    for key in o1:
        assert torch.equal(o1[key].view(torch.uint8), o2[key].view(torch.uint8)), key
    assert s1 == s2


@pytest.mark.parametrize("pack", [False, True], ids=["rowmajor", "packed"])
def test_grouped_expert_with_more_rows_than_tokens(lib, pack):
    """moe_grouped_swiglu with a grouping in which tokens repeat within an
    expert (100 rows for 64 tokens), with enough work items that the kernels
    cut items between work-groups: every row must match the oracle's grouped
    SwiGLU, the rows past the first 64 included."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=8, k=8, H=256, I=2560, N=64)
    N, k, E, H, I = cfg.N, cfg.k, cfg.E, cfg.H, cfg.I
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 5)
    # the last expert's items are among those cut into pieces
    te = np.array([60, 60, 60, 60, 60, 60, 52, 100])
    assert te.sum() == N * k
    offsets = np.concatenate([[0], np.cumsum(te)]).astype(np.int32)
    sa = np.random.default_rng(7).permutation(N * k).astype(np.int32)
    perm = dict(offsets=offsets, sorted_assign=sa, active=np.arange(E))
    dev = "cuda"
    t32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    layout = lib.LAYOUT_PACKED if pack else lib.LAYOUT_ROWMAJOR
    w13, w2 = w["w13"], w["w2"]
    if pack:
        w13, w2 = lib.pack_experts(shape_of(lib, cfg, w_layout=lib.LAYOUT_PACKED), w13, w2, E)
    y_perm = torch.zeros(N * k, H, dtype=torch.float32, device=dev)
    gws = torch.zeros(lib.moe_grouped_swiglu_workspace_size(N, k, I, 1), dtype=torch.uint8,
                      device=dev)
    x = b.x.to(dev)
    for _ in range(2):  # the second call reuses the workspace the first left
        say(f"grouped repeated-token rows pack={pack}")
        lib.moe_grouped_swiglu(N, k, E, H, I, 1, 1, x, w13, w2, None, None, t32(offsets),
                               t32(sa), t32(np.arange(E)), t32([E]), y_perm, gws,
                               w_layout=layout)
        torch.cuda.synchronize()
        ref = O.grouped_swiglu(W.to_exact_f64(b.x), expert_fn_from(cfg, w), perm, k)
        err = max_rel_err(y_perm, ref)
        say(f"  rel err {err:.2e}")
        assert err <= TOL["bf16"], err


def test_natural_mode_layer(lib):
    """Natural routing (all experts eligible) is the standard MoE layer."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=32, H=256, I=192, N=30, flags=1)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 9)
    out, st = run_layer(lib, cfg, b, w)
    lg = out["logits_out"].cpu().numpy()
    ref = oracle_layer(cfg, b, w, lg)
    assert (out["topk_idx"].cpu().numpy() == O.natural_topk(lg, cfg.k)).all()
    assert st["n_active"] == st["n_natural_union"]
    assert max_rel_err(out["y"], ref["y"]) <= TOL["bf16"]


@pytest.mark.parametrize("vname,flags,budget", [("MoE-Spec B=8", 16 | 32, 8),
                                                ("full-softmax demand", 8, 0)])
def test_selector_variant_layer(lib, vname, flags, budget):
    """A selector variant through the whole layer: same kernels, output
    within tolerance of the oracle's layer with the same flags."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=32, H=256, I=192, N=30, flags=flags,
                                       fixed_budget=budget)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    for seed in range(2):
        say(f"layer variant {vname} seed {seed}")
        b = W.make_block(cfg, seed)
        out, st = run_layer(lib, cfg, b, w)
        ref = oracle_layer(cfg, b, w, out["logits_out"].cpu().numpy())
        assert check_selection(out, ref, st, cfg, f"{vname} seed {seed}")
        assert max_rel_err(out["y"], ref["y"]) <= TOL["bf16"]


@pytest.mark.parametrize("budget", [6, 10, 20], ids=["b6", "b10", "b20"])
def test_work_order_rounds_match_separate_path(lib, budget):
    """verify_block hands the expert kernels the active experts heaviest
    cost class first and deals the work items over the per-CU rounds in a
    snake (on 256 CUs: one round and part of a second, two and part of a
    third, more items than one pass: U = 6, 10, 14 active experts of 64
    gate/up items each);
    the standalone grouped call takes the ascending active list with the
    plain order.  Both must give the same bits, and y must be within the bf16
    tolerance of the oracle."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=32, k=2, H=256, I=2048, N=64, fixed_budget=budget)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 3)
    say(f"work order B={budget}")
    out, st = run_layer(lib, cfg, b, w, pack=True)
    ref = oracle_layer(cfg, b, w, out["logits_out"].cpu().numpy())
    assert check_selection(out, ref, st, cfg, f"work order B={budget}")
    assert max_rel_err(out["y"], ref["y"]) <= TOL["bf16"]
    # the same selection through the separate entry points
    N, H, I, E, k = cfg.N, cfg.H, cfg.I, cfg.E, cfg.k
    dev = "cuda"
    e_ = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=dev)
    ti, tg = out["topk_idx"], out["topk_gate"]
    counts, offsets, sa, ip, act, na = e_(E), e_(E + 1), e_(N * k), e_(N * k), e_(E), e_(1)
    lib.moe_route_permute(N, k, E, ti, counts, offsets, sa, ip, act, na)
    w13, w2 = lib.pack_experts(shape_of(lib, cfg, w_layout=lib.LAYOUT_PACKED), w["w13"], w["w2"], E)
    y_perm = e_(N * k, H, dt=torch.float32)
    gws = torch.zeros(lib.moe_grouped_swiglu_workspace_size(N, k, I, 1), dtype=torch.uint8,
                      device=dev)
    d = upload_block(b)
    lib.moe_grouped_swiglu(N, k, E, H, I, 1, 1, d["x"], w13, w2, None, None, offsets, sa, act,
                           na, y_perm, gws, w_layout=lib.LAYOUT_PACKED)
    y = e_(N, H, dt=torch.bfloat16)
    lib.moe_combine(N, k, H, 1, y_perm, ip, tg, None, y)
    torch.cuda.synchronize()
    u = int(na.item())
    rows = counts.cpu().numpy()[act.cpu().numpy()[:u]]
    say(f"  U={u} rows per active expert {sorted(rows.tolist(), reverse=True)}")
    assert u == st["n_active"] and rows.max() <= 64
    assert torch.equal(y.view(torch.int16), out["y"].view(torch.int16))


def test_gemm_many_units_per_workgroup(lib):
    """Every token routed to all 8 experts (k = E, natural routing): 4096 rows
    per expert in 128-row groups, 3 column tiles per projection -- 768 GEMM
    tiles per kernel, so each work-group runs several in sequence (the ring,
    epilogue staging and output-row table reused across tiles).  y must be
    the same bits as the streaming kernels' (the standalone grouped call)."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=8, k=8, H=1536, I=768, N=4096, flags=1)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 2)
    say("gemm many units per work-group")
    out, st = run_layer(lib, cfg, b, w, pack=True)
    N, H, I, E, k = cfg.N, cfg.H, cfg.I, cfg.E, cfg.k
    assert st["n_active"] == E
    dev = "cuda"
    e_ = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=dev)
    ti, tg = out["topk_idx"], out["topk_gate"]
    counts, offsets, sa, ip, act, na = e_(E), e_(E + 1), e_(N * k), e_(N * k), e_(E), e_(1)
    lib.moe_route_permute(N, k, E, ti, counts, offsets, sa, ip, act, na)
    w13, w2 = lib.pack_experts(shape_of(lib, cfg, w_layout=lib.LAYOUT_PACKED), w["w13"], w["w2"], E)
    y_perm = e_(N * k, H, dt=torch.float32)
    gws = torch.zeros(lib.moe_grouped_swiglu_workspace_size(N, k, I, 1), dtype=torch.uint8,
                      device=dev)
    d = upload_block(b)
    lib.moe_grouped_swiglu(N, k, E, H, I, 1, 1, d["x"], w13, w2, None, None, offsets, sa, act,
                           na, y_perm, gws, w_layout=lib.LAYOUT_PACKED)
    y = e_(N, H, dt=torch.bfloat16)
    lib.moe_combine(N, k, H, 1, y_perm, ip, tg, None, y)
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == N).all()
    assert torch.equal(y.view(torch.int16), out["y"].view(torch.int16))
    assert torch.isfinite(out["y"].float()).all()


@pytest.mark.parametrize("over", [
    # natural routing, ~500 rows per expert: every expert in the GEMM tiles,
    # a partial last column tile (10 gate/up items), K = 320 padded to 384
    dict(E=16, k=8, H=256, I=320, N=1024, flags=1),
    # ~75 rows per expert on average: every active expert in the GEMM tiles,
    # also those with fewer than 64 rows (most row tiles empty)
    dict(E=32, k=4, H=512, I=256, N=600),
    # ~50 rows per expert on average: the experts with more than 64 rows in
    # the GEMM tiles, the others in the streaming kernels
    dict(E=32, k=4, H=512, I=256, N=400),
], ids=["all_large", "all_gemm", "mixed"])
def test_gemm_split_matches_separate_path(lib, over):
    """Blocks whose experts average 32 or more routed rows (packed bf16): the
    experts with many rows (from 64 mean rows on, every active expert) run in
    the GEMM kernels, the others in the streaming kernels.  The standalone
    grouped call runs every expert in the streaming kernels; each output
    element takes the same MFMA sequence in both, so y must be the same bits,
    and within the bf16 tolerance of the oracle."""
    cfg = W.CONFIGS["qwen3_30b"].with_(**over)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    b = W.make_block(cfg, 5)
    say(f"gemm split {over}")
    out, st = run_layer(lib, cfg, b, w, pack=True)
    ref = oracle_layer(cfg, b, w, out["logits_out"].cpu().numpy())
    assert check_selection(out, ref, st, cfg, f"gemm split {over}")
    assert max_rel_err(out["y"], ref["y"]) <= TOL["bf16"]
    N, H, I, E, k = cfg.N, cfg.H, cfg.I, cfg.E, cfg.k
    dev = "cuda"
    e_ = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=dev)
    ti, tg = out["topk_idx"], out["topk_gate"]
    counts, offsets, sa, ip, act, na = e_(E), e_(E + 1), e_(N * k), e_(N * k), e_(E), e_(1)
    lib.moe_route_permute(N, k, E, ti, counts, offsets, sa, ip, act, na)
    w13, w2 = lib.pack_experts(shape_of(lib, cfg, w_layout=lib.LAYOUT_PACKED), w["w13"], w["w2"], E)
    y_perm = e_(N * k, H, dt=torch.float32)
    gws = torch.zeros(lib.moe_grouped_swiglu_workspace_size(N, k, I, 1), dtype=torch.uint8,
                      device=dev)
    d = upload_block(b)
    lib.moe_grouped_swiglu(N, k, E, H, I, 1, 1, d["x"], w13, w2, None, None, offsets, sa, act,
                           na, y_perm, gws, w_layout=lib.LAYOUT_PACKED)
    y = e_(N, H, dt=torch.bfloat16)
    lib.moe_combine(N, k, H, 1, y_perm, ip, tg, None, y)
    torch.cuda.synchronize()
    rows = counts.cpu().numpy()[act.cpu().numpy()[:int(na.item())]]
    say(f"  U={int(na.item())} rows per active expert {sorted(rows.tolist(), reverse=True)}")
    assert rows.max() > 64
    assert torch.equal(y.view(torch.int16), out["y"].view(torch.int16))
