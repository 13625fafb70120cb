"""verify_block_noalloc (the library's own device workspace, for callers that
cannot allocate) against verify_block with a caller workspace: two calls in a
row, the second with a smaller block, must give the same bits as the
existing entry point, and the layer must match the oracle within the bf16
tolerance."""

import pytest
import torch

import workloads as W
from gpu_cases import (TOL, check_selection, make_weights, max_rel_err, oracle_layer_args, say,
                       shape_of, upload_block)
import oracle as O

pytestmark = pytest.mark.gpu

KEYS = ("y", "logits_out", "eligible", "topk_idx", "topk_gate", "counts", "stats")


def outputs_like(lib, cfg, dev="cuda"):
    N, E, k, H = cfg.N, cfg.E, cfg.k, cfg.H
    return dict(y=torch.empty((N, H), dtype=torch.bfloat16, device=dev),
                logits_out=torch.empty((N, E), dtype=torch.float32, device=dev),
                eligible=torch.empty(E, dtype=torch.uint8, device=dev),
                topk_idx=torch.empty((N, k), dtype=torch.int32, device=dev),
                topk_gate=torch.empty((N, k), dtype=torch.float32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                active=torch.empty(E, dtype=torch.int32, device=dev),
                stats=lib.new_stats(dev))


def test_noalloc_matches_verify_block(lib):
    base = W.CONFIGS["qwen3_30b"].with_(E=48, k=8, H=512, I=384)
    w = make_weights(base.with_(N=64), device="cuda", gen_device="cpu")
    for n_nodes, seed in ((64, 0), (23, 1)):  # the second call is a smaller block
        cfg = base.with_(N=n_nodes)
        b = W.make_block(cfg, seed)
        d = upload_block(b)
        sh = shape_of(lib, cfg)
        inputs = dict(x=d["x"], w_router=d["w_router"], b_router=d["b_router"],
                      parent=d["parent"], depth=d["depth"], commit=d["commit"],
                      resident=d["resident"], w13=w["w13"], w2=w["w2"])
        say(f"noalloc N={n_nodes} seed {seed}")
        ref = outputs_like(lib, cfg)
        ws = torch.zeros(lib.acceptmoe_workspace_size(sh), dtype=torch.uint8, device="cuda")
        lib.verify_block(sh, inputs, ref, ws)
        got = outputs_like(lib, cfg)
        lib.verify_block_noalloc(sh, inputs, got)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), f"N={n_nodes}: {key} differs"
        st = lib.decode_stats(got["stats"])
        U = st["n_active"]
        assert torch.equal(got["active"][:U], ref["active"][:U])
        oref = O.verify_block(**oracle_layer_args(cfg, b, w, got["logits_out"].cpu().numpy()))
        assert check_selection(got, oref, st, cfg, f"noalloc N={n_nodes}")
        err = max_rel_err(got["y"], oref["y"])
        say(f"  U={U} rel err {err:.2e}")
        assert err <= TOL[cfg.w]


def test_noalloc_graph_replays(lib):
    """verify_block_noalloc captured in a HIP graph (its counter clear is a
    kernel, not a memset node): every replay, with eager work between the
    replays, gives the bits verify_block gives."""
    cfg = W.CONFIGS["qwen3_30b"].with_(E=48, k=8, H=512, I=384, N=64)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    blocks = [W.make_block(cfg, s) for s in range(2)]
    sh = shape_of(lib, cfg)
    ws = torch.zeros(lib.acceptmoe_workspace_size(sh), dtype=torch.uint8, device="cuda")
    ins, refs, outs = [], [], []
    for b in blocks:
        d = upload_block(b)
        inputs = dict(x=d["x"], w_router=d["w_router"], b_router=d["b_router"],
                      parent=d["parent"], depth=d["depth"], commit=d["commit"],
                      resident=d["resident"], w13=w["w13"], w2=w["w2"])
        ref = outputs_like(lib, cfg)
        lib.verify_block(sh, inputs, ref, ws)
        ins.append(inputs)
        refs.append(ref)
        outs.append(outputs_like(lib, cfg))
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for inputs, o in zip(ins, outs):
            lib.verify_block_noalloc(sh, inputs, o)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graphs = []
    for inputs, o in zip(ins, outs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lib.verify_block_noalloc(sh, inputs, o)
        graphs.append(g)
    torch.cuda.synchronize()
    junk = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        for i, g in enumerate(graphs):
            junk.normal_()
            for key in KEYS:
                outs[i][key].zero_()
            g.replay()
            torch.cuda.synchronize()
            say(f"noalloc graph replay {rep} block {i}")
            for key in KEYS:
                assert torch.equal(outs[i][key], refs[i][key]), f"replay {rep} block {i}: {key}"
