"""Shared helpers for the GPU parity tests: upload seeded blocks, run the HIP
path through the C ABI, and evaluate the oracle on the same inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
from oracle import acceptmoe as OA
from oracle import fp8 as OF8
import workloads as W

DT = {"f32": 0, "bf16": 1, "fp8": 2}
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}   # max-abs error / max|y_ref|


def say(msg: str):
    print(msg, flush=True)


def shape_of(lib, cfg, **kw):
    return lib.make_shape(cfg.N, cfg.H, cfg.I, cfg.E, cfg.k, cfg.n_depth,
                          act_dtype=DT[cfg.act], w_dtype=DT[cfg.w], min_set=cfg.min_set,
                          fixed_budget=cfg.fixed_budget, reroute_budget=cfg.reroute,
                          flags=cfg.flags, **kw)


def upload_block(b: W.Block, dev="cuda"):
    d = dict(x=b.x.to(dev), w_router=b.w_router.to(dev),
             b_router=None if b.b_router is None else b.b_router.to(dev),
             parent=torch.from_numpy(b.parent).to(dev), depth=torch.from_numpy(b.depth).to(dev),
             commit=torch.from_numpy(b.commit).to(dev),
             resident=None if b.resident is None else torch.from_numpy(b.resident).to(dev))
    return d


def make_weights(cfg, device="cuda", layer=0, gen_device=None):
    """Expert weights on `device` (drawn on gen_device: CPU for small shapes)."""
    gd = gen_device or device
    w = W.expert_weights(cfg, layer=layer, device=gd)
    out = {k: (None if v is None else v.to(device)) for k, v in w.items()}
    if cfg.shared:
        s = W.shared_weights(cfg, layer=layer, device=gd)
        out["w13_shared"] = s["w13"][0].to(device)
        out["w2_shared"] = s["w2"][0].to(device)
        if s["s13"] is not None:
            out["s13_shared"] = s["s13"][0].to(device)
            out["s2_shared"] = s["s2"][0].to(device)
    return out


def _exact_expert(cfg, w, e):
    """One expert's exact fp64 (Wg, Wu, Wd), read back from the device."""
    if cfg.w == "fp8":
        q13 = w["w13"][e].cpu().numpy()
        s13 = w["s13"][e].cpu().numpy()
        return (OF8.dequant_blocks(q13[0], s13[0]), OF8.dequant_blocks(q13[1], s13[1]),
                OF8.dequant_blocks(w["w2"][e].cpu().numpy(), w["s2"][e].cpu().numpy()))
    w13 = W.to_exact_f64(w["w13"][e])
    return (w13[0], w13[1], W.to_exact_f64(w["w2"][e]))


def expert_fn_from(cfg, w, cache_size=48):
    """Oracle accessor reading one expert's exact weights back from the device
    (the last `cache_size` distinct experts are kept)."""
    cache = {}

    def fn(e):
        if e in cache:
            return cache[e]
        val = _exact_expert(cfg, w, e)
        if len(cache) < cache_size:
            cache[e] = val
        return val
    return fn


def expert_fn_streaming(cfg, w, order, threads=8, window=12):
    """Oracle accessor for experts requested once each in `order` (the
    grouped layer's ascending active list): the exact weights of the next
    `window` experts are prepared by a thread pool ahead of the request, and
    dropped once handed out, so a full-size layer costs little host memory.
    The device reads happen here, on the calling thread."""
    import concurrent.futures as cf
    order = [int(e) for e in order]
    pos = {e: i for i, e in enumerate(order)}
    ex = cf.ThreadPoolExecutor(max_workers=threads)
    futs = {}

    def submit(i):
        if i < len(order) and order[i] not in futs:
            e = order[i]
            if cfg.w == "fp8":
                raw = (w["w13"][e].cpu().numpy(), w["s13"][e].cpu().numpy(),
                       w["w2"][e].cpu().numpy(), w["s2"][e].cpu().numpy())
                futs[e] = ex.submit(lambda r: (OF8.dequant_blocks(r[0][0], r[1][0]),
                                               OF8.dequant_blocks(r[0][1], r[1][1]),
                                               OF8.dequant_blocks(r[2], r[3])), raw)
            else:
                raw = (w["w13"][e].cpu(), w["w2"][e].cpu())
                futs[e] = ex.submit(lambda r: (W.to_exact_f64(r[0][0]), W.to_exact_f64(r[0][1]),
                                               W.to_exact_f64(r[1])), raw)

    for i in range(min(window, len(order))):
        submit(i)

    def fn(e):
        e = int(e)
        if e not in pos:
            return _exact_expert(cfg, w, e)
        submit(pos[e])
        val = futs.pop(e).result()
        submit(pos[e] + window)
        if pos[e] == len(order) - 1:
            ex.shutdown(wait=False)
        return val
    return fn


def shared_fn_from(cfg, w):
    if "w13_shared" not in w:
        return None
    if cfg.w == "fp8":
        q13 = w["w13_shared"].cpu().numpy()
        s13 = w["s13_shared"].cpu().numpy()
        val = (OF8.dequant_blocks(q13[0], s13[0]), OF8.dequant_blocks(q13[1], s13[1]),
               OF8.dequant_blocks(w["w2_shared"].cpu().numpy(), w["s2_shared"].cpu().numpy()))
    else:
        w13 = W.to_exact_f64(w["w13_shared"])
        val = (w13[0], w13[1], W.to_exact_f64(w["w2_shared"]))
    return lambda: val


def oracle_select(cfg, b: W.Block, logits_in=None, flags=None, resident="block", **kw):
    res = b.resident if isinstance(resident, str) else resident
    args = dict(k=cfg.k, parent=b.parent, depth=b.depth, commit=b.commit, resident=res,
                min_set=cfg.min_set, fixed_budget=cfg.fixed_budget,
                reroute_budget=cfg.reroute, flags=cfg.flags if flags is None else flags)
    args.update(kw)
    if logits_in is not None:
        args["logits_in"] = logits_in
    else:
        args.update(x=W.to_exact_f64(b.x), w_router=W.to_exact_f64(b.w_router),
                    b_router=None if b.b_router is None else b.b_router.numpy())
    return O.select(**args)


def check_selection(gpu: dict, ref: dict, stats: dict, cfg, ctx=""):
    """Bit-exact comparison of the integer outputs of the selection."""
    if ref["near_tie"]:
        return False
    elig = gpu["eligible"].cpu().numpy().astype(bool)
    assert (elig == ref["eligible"]).all(), f"{ctx}: eligible set differs"
    ti = gpu["topk_idx"].cpu().numpy()
    assert (ti == ref["topk_idx"]).all(), f"{ctx}: topk_idx differs"
    tg = gpu["topk_gate"].cpu().numpy().astype(np.float64)
    rg = ref["topk_gate"].astype(np.float64)
    assert np.max(np.abs(tg - rg) / np.abs(rg)) <= 1e-6, f"{ctx}: gates differ"
    rs = ref["stats"]
    for key in ("n_anchor", "n_selfsize", "n_eligible", "n_pruned", "n_natural_union",
                "n_active", "n_active_nonresident"):
        assert stats[key] == rs[key], f"{ctx}: stats {key} {stats[key]} != {rs[key]}"
    assert stats["err_flags"] == 0
    assert abs(stats["r_eff"] - rs["r_eff"]) <= 1e-12 * max(1.0, rs["r_eff"]), ctx
    return True


def max_rel_err(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref)))


def oracle_layer_args(cfg, b, w, logits, resident="block"):
    """Keyword arguments of oracle.verify_block for a block run with the GPU's
    fp32 logits (the selection is then bit-exact to compare)."""
    return dict(k=cfg.k, x=W.to_exact_f64(b.x), expert_fn=expert_fn_from(cfg, w),
                parent=b.parent, depth=b.depth, commit=b.commit, logits_in=logits,
                resident=b.resident if isinstance(resident, str) else resident,
                min_set=cfg.min_set, fixed_budget=cfg.fixed_budget,
                reroute_budget=cfg.reroute, flags=cfg.flags, shared_fn=shared_fn_from(cfg, w))
