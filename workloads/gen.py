"""Seeded synthetic verification blocks with the shapes of the pages' workloads.

No benchmark data or trained weights exist here; every block is drawn from a
seeded generator with the structure the workloads have:

* draft trees like an EAGLE-3 tree of 5 draft steps, branching up to 10,
  64 nodes, batch 1 [AcceptMoE news §03]; a root plus a short chain for the
  tiny layer; 32 independent 8-token chains for the batched DeepSeek-shaped
  layer;
* per-depth commitment probabilities decaying with depth [AcceptMoE news §02];
* router logits = shared per-expert bias + per-token noise, so demand is skewed
  (set sizes in the range the AcceptMoE article reports, 23-34 experts);
* a 48-slot resident mask drawn from a Zipf(1.1) popularity [AcceptMoE news §03];
* expert weights ~ N(0, 0.02) in the storage dtype; fp8 experts are quantised
  per 128 x 128 block (scale = block amax / 448, E4M3FN round-to-nearest-even).

Host-side draws use ``numpy.random.default_rng([config id, seed, stream])``;
expert weights are drawn with ``torch.Generator`` on the requested device
(CPU for small parity shapes, the GPU for multi-GB layers), seeded per expert.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cid: int
    E: int
    k: int
    H: int
    I: int
    N: int
    act: str            # "f32" | "bf16"
    w: str              # "f32" | "bf16" | "fp8"
    tree: str           # "chain" | "eagle" | "chains"
    commit: tuple
    x_std: float
    wr_std: float       # router weight std (0 -> 1/sqrt(H))
    bias_std: float
    w_std: float = 0.02
    shared: bool = False
    resident_slots: int = 0
    zipf: float = 1.1
    reroute: int = 0
    min_set: int = 0
    fixed_budget: int = 0
    flags: int = 0
    n_chains: int = 0
    chain_len: int = 0
    eagle_steps: int = 5
    eagle_width: int = 10

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def n_depth(self) -> int:
        return len(self.commit)

    def expert_bytes(self) -> int:
        """Weight bytes of one routed expert (w13 + w2), scales excluded."""
        per = {"f32": 4, "bf16": 2, "fp8": 1}[self.w]
        return 3 * self.H * self.I * per

    def scale_bytes(self) -> int:
        if self.w != "fp8":
            return 0
        return 4 * (2 * (self.I // 128) * (self.H // 128) + (self.H // 128) * (self.I // 128))


_EAGLE_COMMIT = (1.0, 0.75, 0.5, 0.33, 0.2, 0.12)
# the batched chains are 8 deep; the two extra depths continue the table's
# decay by a factor 0.6 (a stated assumption)
_CHAIN8_COMMIT = (1.0, 0.75, 0.5, 0.33, 0.2, 0.12, 0.072, 0.0432)

CONFIGS = {
    "tiny": Config("tiny", 0, E=16, k=2, H=64, I=128, N=4, act="f32", w="f32",
                   tree="chain", commit=(1.0, 0.7, 0.45, 0.3), x_std=1 / 8,
                   wr_std=1 / 8, bias_std=0.0),
    "qwen3_30b": Config("qwen3_30b", 1, E=128, k=8, H=2048, I=768, N=64,
                        act="bf16", w="bf16", tree="eagle", commit=_EAGLE_COMMIT,
                        x_std=1.0, wr_std=0.0, bias_std=1.0),
    "gptoss_120b": Config("gptoss_120b", 2, E=128, k=4, H=2880, I=2880, N=64,
                          act="bf16", w="bf16", tree="eagle", commit=_EAGLE_COMMIT,
                          x_std=1.0, wr_std=0.0, bias_std=1.0, resident_slots=48,
                          zipf=1.1, reroute=8),
    "qwen3_235b": Config("qwen3_235b", 3, E=128, k=8, H=4096, I=1536, N=64,
                         act="bf16", w="bf16", tree="eagle", commit=_EAGLE_COMMIT,
                         x_std=1.0, wr_std=0.0, bias_std=1.0),
    "dsv31": Config("dsv31", 4, E=256, k=8, H=7168, I=2048, N=256, act="bf16",
                    w="fp8", tree="chains", commit=_CHAIN8_COMMIT, x_std=1.0,
                    wr_std=0.0, bias_std=0.0, shared=True, n_chains=32, chain_len=8),
}
# demand-concentration sweep of the Qwen3-235B-shaped layer (router bias std)
CONFIGS["qwen3_235b_b025"] = CONFIGS["qwen3_235b"].with_(name="qwen3_235b_b025", cid=5, bias_std=0.25)
CONFIGS["qwen3_235b_b4"] = CONFIGS["qwen3_235b"].with_(name="qwen3_235b_b4", cid=6, bias_std=4.0)


@dataclasses.dataclass
class Block:
    """One verification block's non-weight inputs (exact values, host side)."""
    cfg: Config
    seed: int
    parent: np.ndarray      # int32 [N]
    depth: np.ndarray       # int32 [N]
    commit: np.ndarray      # float32 [n_depth]
    x: torch.Tensor         # [N, H] act dtype (CPU)
    w_router: torch.Tensor  # [E, H] act dtype (CPU)
    b_router: Optional[torch.Tensor]   # [E] float32 or None
    resident: Optional[np.ndarray]     # uint8 [E] or None


def _rng(cfg: Config, seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cfg.cid, int(seed), stream])


def make_tree(cfg: Config, rng: np.random.Generator):
    """Parent pointers (topological, roots = -1) and depths for one block."""
    if cfg.tree == "chain":
        parent = np.arange(-1, cfg.N - 1, dtype=np.int32)
        depth = np.arange(cfg.N, dtype=np.int32)
        return parent, depth
    if cfg.tree == "chains":
        L = cfg.chain_len
        assert cfg.n_chains * L == cfg.N
        parent = np.empty(cfg.N, dtype=np.int32)
        depth = np.empty(cfg.N, dtype=np.int32)
        for c in range(cfg.n_chains):
            for d in range(L):
                parent[c * L + d] = -1 if d == 0 else c * L + d - 1
                depth[c * L + d] = d
        return parent, depth
    assert cfg.tree == "eagle"
    steps, width = cfg.eagle_steps, cfg.eagle_width
    while True:
        par = [-1]
        dep = [0]
        kids = [0]
        for i in range(1, cfg.N):
            cand = [j for j in range(i) if dep[j] < steps and kids[j] < width]
            j = int(cand[rng.integers(len(cand))])
            par.append(j)
            dep.append(dep[j] + 1)
            kids[j] += 1
            kids.append(0)
        if max(dep) == steps or cfg.N <= steps:
            break
    dep = np.array(dep)
    order = np.argsort(dep, kind="stable")
    pos = np.empty_like(order)
    pos[order] = np.arange(len(order))
    parent = np.array([-1 if par[o] < 0 else pos[par[o]] for o in order], dtype=np.int32)
    depth = dep[order].astype(np.int32)
    return parent, depth


def _act_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_block(cfg, seed: int, **overrides) -> Block:
    """Seeded non-weight inputs: tree, commit table, x, router, resident mask."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = cfg.with_(**overrides)
    parent, depth = make_tree(cfg, _rng(cfg, seed, 0))
    rng = _rng(cfg, seed, 1)
    dt = _act_dtype(cfg.act)
    x = torch.from_numpy(rng.normal(0.0, cfg.x_std, (cfg.N, cfg.H)).astype(np.float32)).to(dt)
    wr_std = cfg.wr_std if cfg.wr_std > 0 else 1.0 / math.sqrt(cfg.H)
    # router weights and bias belong to the layer: drawn from a seed-free stream
    lrng = np.random.default_rng([cfg.cid, 7919, cfg.E, cfg.H])
    w_router = torch.from_numpy(lrng.normal(0.0, wr_std, (cfg.E, cfg.H)).astype(np.float32)).to(dt)
    b_router = None
    bias_np = None
    if cfg.bias_std > 0:
        bias_np = lrng.normal(0.0, cfg.bias_std, cfg.E).astype(np.float32)
        b_router = torch.from_numpy(bias_np)
    resident = None
    if cfg.resident_slots > 0:
        rrng = _rng(cfg, seed, 2)
        by_pop = (np.argsort(-bias_np, kind="stable") if bias_np is not None
                  else np.arange(cfg.E))
        ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
        prob = ranks ** (-cfg.zipf)
        prob /= prob.sum()
        picks = rrng.choice(cfg.E, size=min(cfg.resident_slots, cfg.E), replace=False, p=prob)
        resident = np.zeros(cfg.E, dtype=np.uint8)
        resident[by_pop[picks]] = 1
    commit = np.array(cfg.commit, dtype=np.float32)
    return Block(cfg, seed, parent, depth, commit, x, w_router, b_router, resident)


# ------------------------------------------------------------ expert weights --
def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    h = 0
    for v in key:
        h = (h * 1000003 + int(v) + 1) % (2 ** 61 - 1)
    g.manual_seed(h)
    return g


def _quant_fp8_blocks(w: torch.Tensor, block: int = 128):
    """Per-block symmetric E4M3FN quantisation of a [O, In] fp32 matrix."""
    O, In = w.shape
    wb = w.reshape(O // block, block, In // block, block)
    amax = wb.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wb / scale[:, None, :, None]).clamp_(-448.0, 448.0)
    q = q.reshape(O, In).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, scale.to(torch.float32)


def _one_expert(cfg: Config, key, device):
    gen = _gen(device, *key)
    w13 = torch.randn((2, cfg.I, cfg.H), generator=gen, device=device) * cfg.w_std
    w2 = torch.randn((cfg.H, cfg.I), generator=gen, device=device) * cfg.w_std
    return w13, w2


def expert_weights(cfg, layer: int = 0, device="cpu", **overrides) -> dict:
    """Routed expert weights for one layer in the storage dtype.

    Returns {"w13": [E,2,I,H], "w2": [E,H,I]} (+ "s13" [E,2,I/128,H/128],
    "s2" [E,H/128,I/128] fp32 for fp8, where w13/w2 hold uint8 E4M3FN codes).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = cfg.with_(**overrides)
    E, I, H = cfg.E, cfg.I, cfg.H
    if cfg.w == "fp8":
        w13 = torch.empty((E, 2, I, H), dtype=torch.uint8, device=device)
        w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
        s13 = torch.empty((E, 2, I // 128, H // 128), dtype=torch.float32, device=device)
        s2 = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=device)
        for e in range(E):
            a, b = _one_expert(cfg, (cfg.cid, layer, e, E, H, I), device)
            for j in range(2):
                w13[e, j], s13[e, j] = _quant_fp8_blocks(a[j])
            w2[e], s2[e] = _quant_fp8_blocks(b)
        return dict(w13=w13, w2=w2, s13=s13, s2=s2)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[cfg.w]
    w13 = torch.empty((E, 2, I, H), dtype=dt, device=device)
    w2 = torch.empty((E, H, I), dtype=dt, device=device)
    for e in range(E):
        a, b = _one_expert(cfg, (cfg.cid, layer, e, E, H, I), device)
        w13[e] = a.to(dt)
        w2[e] = b.to(dt)
    return dict(w13=w13, w2=w2, s13=None, s2=None)


def shared_weights(cfg, layer: int = 0, device="cpu", **overrides) -> dict:
    """The always-on shared expert (same shapes as one routed expert, E = 1)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = cfg.with_(**overrides)
    one = cfg.with_(E=1, cid=cfg.cid + 1000)
    return expert_weights(one, layer=layer, device=device)


def to_exact_f64(t) -> np.ndarray:
    """Exact fp64 values of a float tensor (bf16/fp32 widen exactly)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()
