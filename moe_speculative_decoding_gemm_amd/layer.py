"""A verify-block MoE layer bound to device weights: owns its workspace and
output buffers (allocated once through torch) and calls ``verify_block``."""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L


class VerifyLayer:
    """One MoE layer's weights plus reusable buffers for ``verify_block``.

    weights: dict with w_router [E,H], b_router [E] or None, w13 [E,2,I,H],
    w2 [E,H,I], optional s13/s2 (FP8), optional w13_shared/w2_shared
    (+ s13_shared/s2_shared).  All device tensors, row-major.  With pack=True
    (the default for BF16 / FP8 weights) the expert weights are reordered
    once into the packed layout the kernels stream fastest; the row-major
    tensors are then not referenced.  With overlap=True (the default for a
    layer with a shared expert and BF16 / FP8 weights) run() calls
    verify_block_overlap on a side stream of the layer's own (default
    priority) and two events; overlap=False calls verify_block.  Both give the
    same bits.
    """

    def __init__(self, shape: L.Shape, weights: dict, device=None, debug_outputs: bool = True,
                 pack: Optional[bool] = None, overlap: Optional[bool] = None):
        if pack is None:
            pack = shape.w_dtype != L.F32
        self.shape = L.Shape.from_buffer_copy(shape)
        self.shape.w_layout = L.LAYOUT_PACKED if pack else L.LAYOUT_ROWMAJOR
        shape = self.shape
        self.w = dict(weights)
        dev = torch.device(device or weights["w13"].device)
        if pack:
            E = shape.E
            self.w["w13"], self.w["w2"] = L.pack_experts(shape, weights["w13"], weights["w2"], E)
            if weights.get("w13_shared") is not None:
                p13, p2 = L.pack_experts(shape, weights["w13_shared"][None],
                                         weights["w2_shared"][None], 1)
                self.w["w13_shared"], self.w["w2_shared"] = p13, p2
        self.device = dev
        if overlap is None:
            overlap = shape.w_dtype != L.F32 and weights.get("w13_shared") is not None
        self.set_overlap(overlap)
        N, H, E, k = shape.N, shape.H, shape.E, shape.k
        adt = torch.float32 if shape.act_dtype == L.F32 else torch.bfloat16
        nbytes = L.acceptmoe_workspace_size(shape)
        if nbytes == 0:
            raise L.AcceptMoEError(L.EINVAL, "acceptmoe_workspace_size",
                                   L.raw().acceptmoe_last_error().decode())
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.out = {"y": torch.empty((N, H), dtype=adt, device=dev)}
        if debug_outputs:
            self.out.update(
                logits_out=torch.empty((N, E), dtype=torch.float32, device=dev),
                eligible=torch.empty(E, dtype=torch.uint8, device=dev),
                topk_idx=torch.empty((N, k), dtype=torch.int32, device=dev),
                topk_gate=torch.empty((N, k), dtype=torch.float32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                active=torch.empty(E, dtype=torch.int32, device=dev),
                stats=torch.zeros(L.STATS_BYTES, dtype=torch.uint8, device=dev))

    def set_overlap(self, on: bool):
        """Use verify_block_overlap (on) or verify_block (off) in run()."""
        self.ovl = None
        if on:
            if getattr(self, "_side", None) is None:
                self._side = torch.cuda.Stream(device=self.device)
                self._events = [torch.cuda.Event() for _ in range(2)]
                for ev in self._events:  # creates the event handles
                    ev.record(self._side)
                torch.cuda.synchronize(self.device)
            self.ovl = L.Overlap(self._side.cuda_stream,
                                 *[ev.cuda_event for ev in self._events])

    def variant(self, **fields) -> "VerifyLayer":
        """A layer on the same (already packed) weights whose shape differs in
        the fields given (N, n_depth, flags, fixed_budget, min_set,
        reroute_budget), with its own workspace and output buffers."""
        allowed = {"N", "n_depth", "flags", "fixed_budget", "min_set", "reroute_budget"}
        bad = set(fields) - allowed
        if bad:
            raise ValueError(f"variant() changes only {sorted(allowed)}, not {sorted(bad)}")
        v = object.__new__(VerifyLayer)
        v.shape = L.Shape.from_buffer_copy(self.shape)
        for key, val in fields.items():
            setattr(v.shape, key, val)
        v.w = self.w
        v.device = self.device
        v._side = getattr(self, "_side", None)
        v._events = getattr(self, "_events", None)
        v.ovl = self.ovl
        nbytes = L.acceptmoe_workspace_size(v.shape)
        if nbytes == 0:
            raise L.AcceptMoEError(L.EINVAL, "acceptmoe_workspace_size",
                                   L.raw().acceptmoe_last_error().decode())
        v.ws = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        N = v.shape.N
        v.out = {}
        for key, t in self.out.items():
            shp = list(t.shape)
            if key in ("y", "logits_out", "topk_idx", "topk_gate"):
                shp[0] = N
            v.out[key] = torch.empty(shp, dtype=t.dtype, device=self.device)
        if "stats" in v.out:
            v.out["stats"].zero_()
        return v

    def run(self, x, parent, depth, commit, resident: Optional[torch.Tensor] = None,
            logits_in: Optional[torch.Tensor] = None, stream=None) -> dict:
        inputs = dict(self.w)
        inputs.update(x=x, parent=parent, depth=depth, commit=commit, resident=resident,
                      logits_in=logits_in)
        if self.ovl is not None:
            L.verify_block_overlap(self.shape, inputs, self.out, self.ovl, self.ws, stream=stream)
        else:
            L.verify_block(self.shape, inputs, self.out, self.ws, stream=stream)
        return self.out

    def run_cached(self, cache, x, parent, depth, commit,
                   logits_in: Optional[torch.Tensor] = None, stream=None) -> dict:
        """The block with the routed experts' weights from an ExpertCache
        (the cache's resident mask drives residency-aware pruning).  Returns
        the outputs; the call's cache report is in ``self.report``."""
        inputs = dict(self.w)
        inputs.update(x=x, parent=parent, depth=depth, commit=commit, resident=None,
                      logits_in=logits_in, w13=None, w2=None)
        self.report = L.verify_block_cached(self.shape, inputs, cache.desc, self.out, self.ws,
                                            stream=stream)
        return self.out
