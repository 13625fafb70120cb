"""ctypes binding of libacceptmoe.so (the C ABI in include/acceptmoe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels.
Tensors are PyTorch device tensors (torch provides memory and streams); each
wrapper checks dtype, contiguity, device and shape, then passes raw pointers
and the current stream.  The library must be built (``build()`` in
``__graft_entry__`` or ``python moe_speculative_decoding_gemm_amd/build.py``);
importing this module without it raises.
"""

from __future__ import annotations

import ctypes as C
import os
import struct
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libacceptmoe.so")

OK, EINVAL, ENOTSUP, EHIP = 0, -1, -2, -3
F32, BF16, FP8_E4M3FN = 0, 1, 2
F_NATURAL, F_NO_RENORM, F_LOGITS_IN = 1, 2, 4
F_DEMAND_FULL, F_NO_ANCHOR, F_UNIT_COMMIT = 8, 16, 32
LAYOUT_ROWMAJOR, LAYOUT_PACKED = 0, 1
ERR_BAD_TREE, ERR_DEPTH, ERR_NONFINITE, ERR_COMMIT, ERR_WORKSPACE = 1, 2, 4, 8, 16

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8_E4M3FN,
       torch.float8_e4m3fn: FP8_E4M3FN}


class AcceptMoEError(RuntimeError):
    def __init__(self, code: int, fn: str, detail: str):
        super().__init__(f"{fn} failed ({code}): {detail}")
        self.code = code


class Shape(C.Structure):
    _fields_ = [("N", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32),
                ("k", C.c_int32), ("n_depth", C.c_int32), ("min_set", C.c_int32),
                ("fixed_budget", C.c_int32), ("reroute_budget", C.c_int32),
                ("flags", C.c_uint32), ("act_dtype", C.c_int32), ("w_dtype", C.c_int32),
                ("w_layout", C.c_int32)]


class Inputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "x", "w_router", "b_router", "logits_in", "parent", "depth", "commit", "resident",
        "w13", "w2", "s13", "s2", "w13_shared", "w2_shared", "s13_shared", "s2_shared")]


class Outputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "y", "logits_out", "eligible", "topk_idx", "topk_gate", "counts", "active", "stats")]


class Overlap(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("side", "start", "done")]


class CacheState(C.Structure):
    _fields_ = [("E", C.c_int32), ("n_slots", C.c_int32), ("n_spill", C.c_int32),
                ("_pad", C.c_int32), ("slot_expert", C.c_void_p), ("expert_slot", C.c_void_p),
                ("resident", C.c_void_p), ("last_use", C.c_void_p), ("clock", C.c_int64),
                ("hits", C.c_int64), ("misses", C.c_int64), ("spills", C.c_int64),
                ("h2d_bytes", C.c_int64)]


class ExpertCacheDesc(C.Structure):
    _fields_ = [("state", C.c_void_p), ("host_w13", C.c_void_p), ("host_w2", C.c_void_p),
                ("dev_w13", C.c_void_p), ("dev_w2", C.c_void_p),
                ("dev_expert_slot", C.c_void_p), ("dev_resident", C.c_void_p),
                ("copy_stream", C.c_void_p), ("copy_done", C.c_void_p),
                ("dev_lists", C.c_void_p)]


class CacheReport(C.Structure):
    _fields_ = [("n_active", C.c_int32), ("n_hits", C.c_int32), ("n_fetched", C.c_int32),
                ("n_spilled", C.c_int32), ("h2d_bytes", C.c_int64)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


STATS_BYTES = 48
_STATS_FIELDS = ("n_anchor", "n_selfsize", "n_eligible", "n_pruned", "n_active",
                 "n_active_nonresident", "n_natural_union", "err_flags", "r_eff",
                 "demand_total")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python moe_speculative_decoding_gemm_amd/build.py)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    sig = {
        "acceptmoe_select_workspace_size": (sz, [vp]),
        "acceptmoe_select": (C.c_int, [vp] + [vp] * 13 + [vp, sz, vp]),
        "moe_route_permute": (C.c_int, [i32, i32, i32] + [vp] * 7 + [vp]),
        "moe_grouped_swiglu_workspace_size": (sz, [i32, i32, i32, i32]),
        "moe_grouped_swiglu": (C.c_int, [i32] * 8 + [vp] * 10 + [vp, sz, vp]),
        "acceptmoe_packed_size": (sz, [vp, i32, i32]),
        "acceptmoe_pack_experts": (C.c_int, [vp, i32, vp, vp, vp, vp, vp]),
        "moe_combine": (C.c_int, [i32] * 4 + [vp] * 5 + [vp]),
        "acceptmoe_workspace_size": (sz, [vp]),
        "verify_block": (C.c_int, [vp, vp, vp, vp, sz, vp]),
        "verify_block_noalloc": (C.c_int, [vp, vp, vp, vp]),
        "verify_block_overlap": (C.c_int, [vp, vp, vp, vp, vp, sz, vp]),
        "acceptmoe_cache_plan": (C.c_int, [vp, vp, i32, vp, vp, vp]),
        "verify_block_cached": (C.c_int, [vp, vp, vp, vp, vp, vp, sz, vp]),
        "acceptmoe_set_stage_timer": (C.c_int, [i32, vp, vp]),
        "acceptmoe_strerror": (C.c_char_p, [C.c_int]),
        "acceptmoe_last_error": (C.c_char_p, []),
        "acceptmoe_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("acceptmoe_select_workspace_size", "acceptmoe_select", "moe_route_permute",
            "moe_grouped_swiglu_workspace_size", "moe_grouped_swiglu", "moe_combine",
            "acceptmoe_packed_size", "acceptmoe_pack_experts",
            "acceptmoe_workspace_size", "verify_block", "verify_block_noalloc", "verify_block_overlap",
            "acceptmoe_cache_plan",
            "verify_block_cached", "acceptmoe_set_stage_timer",
            "acceptmoe_strerror",
            "acceptmoe_last_error", "acceptmoe_version")


def raw():
    """The ctypes library object (for tests of the bare C ABI)."""
    return _lib


STAGE_NONE, STAGE_SELECT, STAGE_PERMUTE, STAGE_GATEUP, STAGE_DOWN, STAGE_EXPERTS, \
    STAGE_COMBINE, STAGE_FETCH = range(8)


def acceptmoe_set_stage_timer(stage: int, start_event, stop_event):
    """start_event / stop_event: raw hipEvent_t handles (int) or None."""
    _check(_lib.acceptmoe_set_stage_timer(stage, start_event, stop_event),
           "acceptmoe_set_stage_timer")


def version() -> str:
    return _lib.acceptmoe_version().decode()


def _check(rc: int, fn: str):
    if rc != 0:
        raise AcceptMoEError(rc, fn, _lib.acceptmoe_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, dev=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def dtype_code(t: torch.dtype) -> int:
    return _DT[t]


def make_shape(N, H, I, E, k, n_depth, act_dtype=BF16, w_dtype=BF16, min_set=0,
               fixed_budget=0, reroute_budget=0, flags=0, w_layout=LAYOUT_ROWMAJOR) -> Shape:
    return Shape(N, H, I, E, k, n_depth, min_set, fixed_budget, reroute_budget, flags,
                 act_dtype, w_dtype, w_layout)


def decode_stats(t: torch.Tensor) -> dict:
    """acceptmoe_stats from a STATS_BYTES uint8 device (or host) tensor."""
    b = bytes(t.detach().to("cpu").numpy().tobytes())
    vals = struct.unpack("<8i2d", b[:STATS_BYTES])
    return dict(zip(_STATS_FIELDS, vals))


def new_stats(device=None) -> torch.Tensor:
    return torch.zeros(STATS_BYTES, dtype=torch.uint8, device=device or "cuda")


def _act_dt(shape: Shape):
    return torch.float32 if shape.act_dtype == F32 else torch.bfloat16


def _w_dt(shape: Shape):
    return {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3FN: (torch.uint8, torch.float8_e4m3fn)}[shape.w_dtype]


# ----------------------------------------------------------------- select --
def acceptmoe_select_workspace_size(shape: Shape) -> int:
    return int(_lib.acceptmoe_select_workspace_size(C.byref(shape)))


def acceptmoe_select(shape: Shape, x, w_router, b_router, logits_in, parent, depth, commit,
                     resident, logits_out, eligible, topk_idx, topk_gate, stats, ws,
                     stream=None):
    N, H, E, k = shape.N, shape.H, shape.E, shape.k
    adt = _act_dt(shape)
    args = [
        _ptr(x, "x", adt, (N, H)), _ptr(w_router, "w_router", adt, (E, H)),
        _ptr(b_router, "b_router", torch.float32, (E,)),
        _ptr(logits_in, "logits_in", torch.float32, (N, E)),
        _ptr(parent, "parent", torch.int32, (N,)), _ptr(depth, "depth", torch.int32, (N,)),
        _ptr(commit, "commit", torch.float32, (shape.n_depth,)),
        _ptr(resident, "resident", torch.uint8, (E,)),
        _ptr(logits_out, "logits_out", torch.float32, (N, E)),
        _ptr(eligible, "eligible", torch.uint8, (E,)),
        _ptr(topk_idx, "topk_idx", torch.int32, (N, k)),
        _ptr(topk_gate, "topk_gate", torch.float32, (N, k)),
        _ptr(stats, "stats", torch.uint8, (STATS_BYTES,)),
    ]
    wsp = _ptr(ws, "ws", torch.uint8)
    nb = ws.numel() if ws is not None else 0
    _check(_lib.acceptmoe_select(C.byref(shape), *args, wsp, nb, _stream(stream)),
           "acceptmoe_select")


# ---------------------------------------------------------------- permute --
def moe_route_permute(N, k, E, topk_idx, counts, offsets, sorted_assign, inv_pos, active,
                      n_active, stream=None):
    i32 = torch.int32
    _check(_lib.moe_route_permute(
        N, k, E, _ptr(topk_idx, "topk_idx", i32, (N, k)), _ptr(counts, "counts", i32, (E,)),
        _ptr(offsets, "offsets", i32, (E + 1,)),
        _ptr(sorted_assign, "sorted_assign", i32, (N * k,)),
        _ptr(inv_pos, "inv_pos", i32, (N * k,)), _ptr(active, "active", i32, (E,)),
        _ptr(n_active, "n_active", i32, (1,)), _stream(stream)), "moe_route_permute")


# ---------------------------------------------------------------- experts --
def moe_grouped_swiglu_workspace_size(N, k, I, w_dtype) -> int:
    return int(_lib.moe_grouped_swiglu_workspace_size(N, k, I, w_dtype))


def moe_grouped_swiglu(N, k, E, H, I, act_dtype, w_dtype, x, w13, w2, s13, s2, offsets,
                       sorted_assign, active, n_active, y_perm, ws, stream=None,
                       w_layout=LAYOUT_ROWMAJOR):
    adt = torch.float32 if act_dtype == F32 else torch.bfloat16
    wdt = {F32: torch.float32, BF16: torch.bfloat16,
           FP8_E4M3FN: (torch.uint8, torch.float8_e4m3fn)}[w_dtype]
    i32 = torch.int32
    fp8 = w_dtype == FP8_E4M3FN
    packed = w_layout == LAYOUT_PACKED
    _check(_lib.moe_grouped_swiglu(
        N, k, E, H, I, act_dtype, w_dtype, w_layout, _ptr(x, "x", adt, (N, H)),
        _ptr(w13, "w13", torch.uint8 if packed else wdt, None if packed else (E, 2, I, H)),
        _ptr(w2, "w2", torch.uint8 if packed else wdt, None if packed else (E, H, I)),
        _ptr(s13, "s13", torch.float32, (E, 2, I // 128, H // 128) if fp8 else None),
        _ptr(s2, "s2", torch.float32, (E, H // 128, I // 128) if fp8 else None),
        _ptr(offsets, "offsets", i32, (E + 1,)),
        _ptr(sorted_assign, "sorted_assign", i32, (N * k,)),
        _ptr(active, "active", i32, (E,)), _ptr(n_active, "n_active", i32, (1,)),
        _ptr(y_perm, "y_perm", torch.float32, (N * k, H)), _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0, _stream(stream)), "moe_grouped_swiglu")


def moe_combine(N, k, H, act_dtype, y_perm, inv_pos, topk_gate, y_shared, y, stream=None):
    adt = torch.float32 if act_dtype == F32 else torch.bfloat16
    _check(_lib.moe_combine(
        N, k, H, act_dtype, _ptr(y_perm, "y_perm", torch.float32, (N * k, H)),
        _ptr(inv_pos, "inv_pos", torch.int32, (N * k,)),
        _ptr(topk_gate, "topk_gate", torch.float32, (N, k)),
        _ptr(y_shared, "y_shared", torch.float32, (N, H)), _ptr(y, "y", adt, (N, H)),
        _stream(stream)), "moe_combine")


# ----------------------------------------------------------------- packing --
def acceptmoe_packed_size(shape: Shape, which: int, n_experts: int) -> int:
    return int(_lib.acceptmoe_packed_size(C.byref(shape), which, n_experts))


def acceptmoe_pack_experts(shape: Shape, n_experts: int, w13, w2, w13_packed, w2_packed,
                           stream=None):
    wdt = {BF16: torch.bfloat16, FP8_E4M3FN: (torch.uint8, torch.float8_e4m3fn)}.get(shape.w_dtype)
    H, I = shape.H, shape.I
    _check(_lib.acceptmoe_pack_experts(
        C.byref(shape), n_experts, _ptr(w13, "w13", wdt, (n_experts, 2, I, H)),
        _ptr(w2, "w2", wdt, (n_experts, H, I)),
        _ptr(w13_packed, "w13_packed", torch.uint8, (acceptmoe_packed_size(shape, 0, n_experts),)),
        _ptr(w2_packed, "w2_packed", torch.uint8, (acceptmoe_packed_size(shape, 1, n_experts),)),
        _stream(stream)), "acceptmoe_pack_experts")


def pack_experts(shape: Shape, w13, w2, n_experts: int, stream=None):
    """Allocate (torch) and fill the packed copies of w13 / w2."""
    dev = w13.device
    p13 = torch.empty(acceptmoe_packed_size(shape, 0, n_experts), dtype=torch.uint8, device=dev)
    p2 = torch.empty(acceptmoe_packed_size(shape, 1, n_experts), dtype=torch.uint8, device=dev)
    acceptmoe_pack_experts(shape, n_experts, w13.contiguous(), w2.contiguous(), p13, p2, stream)
    return p13, p2


# ------------------------------------------------------------ whole block --
def acceptmoe_workspace_size(shape: Shape) -> int:
    return int(_lib.acceptmoe_workspace_size(C.byref(shape)))


def _block_args(shape: Shape, inputs: dict, outputs: dict):
    N, H, I, E, k = shape.N, shape.H, shape.I, shape.E, shape.k
    adt = _act_dt(shape)
    packed = shape.w_layout == LAYOUT_PACKED
    wdt = torch.uint8 if packed else _w_dt(shape)
    fp8 = shape.w_dtype == FP8_E4M3FN
    g = inputs.get
    inp = Inputs(
        _ptr(g("x"), "x", adt, (N, H)), _ptr(g("w_router"), "w_router", adt, (E, H)),
        _ptr(g("b_router"), "b_router", torch.float32, (E,)),
        _ptr(g("logits_in"), "logits_in", torch.float32, (N, E)),
        _ptr(g("parent"), "parent", torch.int32, (N,)),
        _ptr(g("depth"), "depth", torch.int32, (N,)),
        _ptr(g("commit"), "commit", torch.float32, (shape.n_depth,)),
        _ptr(g("resident"), "resident", torch.uint8, (E,)),
        _ptr(g("w13"), "w13", wdt, None if packed else (E, 2, I, H)),
        _ptr(g("w2"), "w2", wdt, None if packed else (E, H, I)),
        _ptr(g("s13"), "s13", torch.float32, (E, 2, I // 128, H // 128) if fp8 else None),
        _ptr(g("s2"), "s2", torch.float32, (E, H // 128, I // 128) if fp8 else None),
        _ptr(g("w13_shared"), "w13_shared", wdt, None if packed else (2, I, H)),
        _ptr(g("w2_shared"), "w2_shared", wdt, None if packed else (H, I)),
        _ptr(g("s13_shared"), "s13_shared", torch.float32, (2, I // 128, H // 128) if fp8 else None),
        _ptr(g("s2_shared"), "s2_shared", torch.float32, (H // 128, I // 128) if fp8 else None))
    o = outputs.get
    out = Outputs(
        _ptr(o("y"), "y", adt, (N, H)), _ptr(o("logits_out"), "logits_out", torch.float32, (N, E)),
        _ptr(o("eligible"), "eligible", torch.uint8, (E,)),
        _ptr(o("topk_idx"), "topk_idx", torch.int32, (N, k)),
        _ptr(o("topk_gate"), "topk_gate", torch.float32, (N, k)),
        _ptr(o("counts"), "counts", torch.int32, (E,)),
        _ptr(o("active"), "active", torch.int32, (E,)),
        _ptr(o("stats"), "stats", torch.uint8, (STATS_BYTES,)))
    return inp, out


def verify_block(shape: Shape, inputs: dict, outputs: dict, ws, stream=None):
    """inputs/outputs: dicts keyed like acceptmoe_inputs / acceptmoe_outputs."""
    inp, out = _block_args(shape, inputs, outputs)
    _check(_lib.verify_block(C.byref(shape), C.byref(inp), C.byref(out),
                             _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0,
                             _stream(stream)), "verify_block")


def verify_block_overlap(shape: Shape, inputs: dict, outputs: dict, overlap: "Overlap", ws,
                         stream=None):
    """verify_block with the shared expert on the side stream of `overlap`
    while the selection and the routed experts run (same outputs)."""
    inp, out = _block_args(shape, inputs, outputs)
    _check(_lib.verify_block_overlap(C.byref(shape), C.byref(inp), C.byref(out),
                                     C.byref(overlap), _ptr(ws, "ws", torch.uint8),
                                     ws.numel() if ws is not None else 0, _stream(stream)),
           "verify_block_overlap")


NOALLOC_WORKSPACE_BYTES = 16 << 20  # the library's own workspace of verify_block_noalloc


def verify_block_noalloc(shape: Shape, inputs: dict, outputs: dict, stream=None):
    """verify_block with the library's own device workspace (no ws argument,
    no allocation); calls on one GPU must not overlap in time."""
    inp, out = _block_args(shape, inputs, outputs)
    _check(_lib.verify_block_noalloc(C.byref(shape), C.byref(inp), C.byref(out),
                                     _stream(stream)), "verify_block_noalloc")


def acceptmoe_cache_plan(state: CacheState, active) -> list:
    """Host-only fetch plan for one block's ascending active expert ids (a
    sequence of ints); updates `state` and returns [(expert, slot), ...]."""
    act = (C.c_int32 * max(1, len(active)))(*[int(a) for a in active])
    fe = (C.c_int32 * max(1, len(active)))()
    fs = (C.c_int32 * max(1, len(active)))()
    nf = C.c_int32(0)
    _check(_lib.acceptmoe_cache_plan(C.byref(state), act, len(active), fe, fs, C.byref(nf)),
           "acceptmoe_cache_plan")
    return [(fe[i], fs[i]) for i in range(nf.value)]


def verify_block_cached(shape: Shape, inputs: dict, cache: ExpertCacheDesc, outputs: dict, ws,
                        stream=None) -> dict:
    """verify_block with the routed experts from `cache` (in inputs, w13 / w2 /
    resident are not used).  Synchronizes the stream once; returns the call's
    report as a dict."""
    inp, out = _block_args(shape, inputs, outputs)
    report = CacheReport()
    _check(_lib.verify_block_cached(C.byref(shape), C.byref(inp), C.byref(cache), C.byref(out),
                                    C.byref(report), _ptr(ws, "ws", torch.uint8),
                                    ws.numel() if ws is not None else 0, _stream(stream)),
           "verify_block_cached")
    return report.as_dict()
