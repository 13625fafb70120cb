"""verify_block_overlap (the shared expert on a side stream while the
selection and the routed experts run) against verify_block: every output bit
for bit, with and without a shared expert, for both weight layouts, and under
HIP-graph capture with repeated replays."""

import pytest
import torch

import workloads as W
from gpu_cases import make_weights, say, shape_of, upload_block

pytestmark = pytest.mark.gpu

KEYS = ("y", "logits_out", "eligible", "topk_idx", "topk_gate", "counts", "stats")

CASES = [
    # fp8 with the shared expert, 40 and 96 nodes (the latter: more than one
    # 64-row group of the shared expert)
    ("dsv31", dict(E=20, k=3, H=384, I=256, N=40, n_chains=5, chain_len=8)),
    ("dsv31", dict(E=48, k=8, H=256, I=512, N=96, n_chains=12, chain_len=8)),
    # more work items than two per CU in the shared expert's gate/up
    ("dsv31", dict(E=24, k=8, H=256, I=2304, N=64, n_chains=8, chain_len=8)),
    # no shared expert: the call is verify_block
    ("qwen3_30b", dict(E=48, k=8, H=512, I=384, N=64)),
    ("gptoss_120b", dict(E=20, k=4, H=448, I=448, N=53, resident_slots=9, reroute=3)),
]


def layers(lib, cfg, w, b, pack=True):
    d = upload_block(b)
    weights = dict(w_router=d["w_router"], b_router=d["b_router"], **w)
    ovl = lib.VerifyLayer(shape_of(lib, cfg), weights, pack=pack, overlap=True)
    ser = ovl.variant()
    ser.set_overlap(False)
    return d, ovl, ser


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "rowmajor"])
@pytest.mark.parametrize("name,over", CASES)
def test_overlap_matches_serial(lib, name, over, pack):
    cfg = W.CONFIGS[name].with_(**over)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    for seed in range(2):
        say(f"overlap {name} {over} pack={pack} seed {seed}")
        b = W.make_block(cfg, seed)
        d, ovl, ser = layers(lib, cfg, w, b, pack=pack)
        args = (d["x"], d["parent"], d["depth"], d["commit"])
        a = {k: v.clone() for k, v in ser.run(*args, resident=d["resident"]).items()}
        o = ovl.run(*args, resident=d["resident"])
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(o[key], a[key]), f"seed {seed}: {key} differs"
        U = lib.decode_stats(o["stats"])["n_active"]
        assert torch.equal(o["active"][:U], a["active"][:U])


def test_overlap_full_dsv31_block(lib):
    cfg = W.CONFIGS["dsv31"]
    w = make_weights(cfg, device="cuda")
    for seed in range(2):
        say(f"overlap full dsv31 seed {seed}")
        b = W.make_block(cfg, seed)
        d, ovl, ser = layers(lib, cfg, w, b)
        args = (d["x"], d["parent"], d["depth"], d["commit"])
        a = {k: v.clone() for k, v in ser.run(*args).items()}
        o = ovl.run(*args)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(o[key], a[key]), f"seed {seed}: {key} differs"


@pytest.mark.parametrize("name,over", [CASES[0], CASES[1]])
def test_overlap_graph_replays(lib, name, over):
    """The overlapped call captured in a HIP graph (the side stream joins the
    capture through the events): every replay, with eager work and
    synchronizations between the replays, reproduces the eager result."""
    cfg = W.CONFIGS[name].with_(**over)
    w = make_weights(cfg, device="cuda", gen_device="cpu")
    blocks = [W.make_block(cfg, s) for s in range(2)]
    d0, ovl, ser = layers(lib, cfg, w, blocks[0])
    ds = [upload_block(b) for b in blocks]
    eager = []
    for d in ds:
        out = ser.run(d["x"], d["parent"], d["depth"], d["commit"], resident=d["resident"])
        eager.append({k: v.clone() for k, v in out.items()})
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for d in ds:
            ovl.run(d["x"], d["parent"], d["depth"], d["commit"], resident=d["resident"])
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for d in ds:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ovl.run(d["x"], d["parent"], d["depth"], d["commit"], resident=d["resident"])
        graphs.append(g)
    torch.cuda.synchronize()
    junk = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        for i, g in enumerate(graphs):
            junk.normal_()  # eager work between the replays
            g.replay()
            torch.cuda.synchronize()
            say(f"graph replay {rep} block {i}")
            for key in KEYS:
                assert torch.equal(ovl.out[key], eager[i][key]), f"replay {rep} block {i}: {key}"
