"""Per-layer expert cache for physical expert offload (``verify_block_cached``).

Every routed expert's packed weights live in host memory (pinned, so that
the copies are asynchronous DMA); ``n_slots`` persistent device slots hold
the resident experts and ``n_spill`` more slots take one block's overflow.
The replacement policy and the copies run in the C library
(``acceptmoe_cache_plan``, ``verify_block_cached``); this class only owns the
buffers and the host-side state tables.
"""

from __future__ import annotations

import ctypes as C
from typing import Iterable, Optional

import torch

from . import _lib as L


class ExpertCache:
    """Host store + device slots + state of one layer's expert cache.

    shape: the layer's (packed-layout) shape.  w13_packed / w2_packed: packed
    weights of all E experts (``pack_experts``), on the device or the host;
    they are copied into a host store.  device=None builds the host state only
    (for the plan on a machine without a GPU).
    """

    def __init__(self, shape: L.Shape, n_slots: int, n_spill: int,
                 w13_packed: Optional[torch.Tensor] = None,
                 w2_packed: Optional[torch.Tensor] = None, device=None, overlap: bool = False):
        E = shape.E
        self.E, self.n_slots, self.n_spill = E, n_slots, n_spill
        pin = device is not None
        i32, u8, i64 = torch.int32, torch.uint8, torch.int64
        self.slot_expert = torch.full((max(n_slots, 1),), -1, dtype=i32, pin_memory=pin)
        self.expert_slot = torch.full((E,), -1, dtype=i32, pin_memory=pin)
        self.resident = torch.zeros(E, dtype=u8, pin_memory=pin)
        self.last_use = torch.zeros(max(n_slots, 1), dtype=i64, pin_memory=pin)
        self.state = L.CacheState(E, n_slots, n_spill, 0, self.slot_expert.data_ptr(),
                                  self.expert_slot.data_ptr(), self.resident.data_ptr(),
                                  self.last_use.data_ptr(), 0, 0, 0, 0, 0)
        self.device = torch.device(device) if device is not None else None
        self.desc = None
        if device is None:
            return
        p = L.Shape.from_buffer_copy(shape)
        p.w_layout = L.LAYOUT_PACKED
        self.b13 = L.acceptmoe_packed_size(p, 0, 1)
        self.b2 = L.acceptmoe_packed_size(p, 1, 1)
        if w13_packed.numel() != E * self.b13 or w2_packed.numel() != E * self.b2:
            raise ValueError("packed weights do not match the shape")
        self.host_w13 = torch.empty(E * self.b13, dtype=u8, pin_memory=True)
        self.host_w2 = torch.empty(E * self.b2, dtype=u8, pin_memory=True)
        self.host_w13.copy_(w13_packed.reshape(-1))
        self.host_w2.copy_(w2_packed.reshape(-1))
        ns = n_slots + n_spill
        dev = self.device
        self.dev_w13 = torch.zeros(max(ns, 1) * self.b13, dtype=u8, device=dev)
        self.dev_w2 = torch.zeros(max(ns, 1) * self.b2, dtype=u8, device=dev)
        self.dev_expert_slot = torch.full((E,), -1, dtype=i32, device=dev)
        self.dev_resident = torch.zeros(E, dtype=u8, device=dev)
        self.desc = L.ExpertCacheDesc(
            C.addressof(self.state), self.host_w13.data_ptr(), self.host_w2.data_ptr(),
            self.dev_w13.data_ptr(), self.dev_w2.data_ptr(), self.dev_expert_slot.data_ptr(),
            self.dev_resident.data_ptr(), None, None, None)
        self.set_overlap(overlap)

    def set_overlap(self, on: bool):
        """Copy the missing experts on a stream of their own (default
        priority) while the hit experts run, each missing expert computed as
        soon as its copy has landed; or copy them on the call's stream."""
        if on and getattr(self, "copy_stream", None) is None:
            self.copy_stream = torch.cuda.Stream(device=self.device)
            self.copy_done = torch.cuda.Event()
            self.copy_done.record(self.copy_stream)  # creates the event handle
            self.dev_lists = torch.zeros(2 * self.E + 3, dtype=torch.int32, device=self.device)
            torch.cuda.synchronize(self.device)
        if on:
            self.desc.copy_stream = self.copy_stream.cuda_stream
            self.desc.copy_done = self.copy_done.cuda_event
            self.desc.dev_lists = self.dev_lists.data_ptr()
        else:
            self.desc.copy_stream = self.desc.copy_done = self.desc.dev_lists = None

    def reset(self, experts: Iterable[int] = ()):
        """Empty the cache, then place `experts` in slots 0, 1, ... (a warm
        start: their weights are copied now, outside any timed block)."""
        experts = [int(e) for e in experts]
        if len(experts) > self.n_slots or len(set(experts)) != len(experts):
            raise ValueError("warm-start experts must be distinct and fit the slots")
        if self.device is not None:
            torch.cuda.synchronize(self.device)  # no copy of an earlier call still reads them
        self.slot_expert.fill_(-1)
        self.expert_slot.fill_(-1)
        self.resident.zero_()
        self.last_use.zero_()
        for q, e in enumerate(experts):
            self.slot_expert[q] = e
            self.expert_slot[e] = q
            self.resident[e] = 1
        st = self.state
        st.clock = st.hits = st.misses = st.spills = st.h2d_bytes = 0
        if self.device is not None:
            for q, e in enumerate(experts):
                self.dev_w13[q * self.b13:(q + 1) * self.b13].copy_(
                    self.host_w13[e * self.b13:(e + 1) * self.b13])
                self.dev_w2[q * self.b2:(q + 1) * self.b2].copy_(
                    self.host_w2[e * self.b2:(e + 1) * self.b2])
            self.dev_expert_slot.copy_(self.expert_slot)
            self.dev_resident.copy_(self.resident)
            torch.cuda.synchronize(self.device)

    def plan(self, active: Iterable[int]) -> list:
        """Host-only plan for one block's ascending active experts."""
        return L.acceptmoe_cache_plan(self.state, list(active))

    def counters(self) -> dict:
        st = self.state
        return {"clock": st.clock, "hits": st.hits, "misses": st.misses, "spills": st.spills,
                "h2d_bytes": st.h2d_bytes}

    def resident_set(self) -> set:
        return {int(e) for e in torch.nonzero(self.resident).flatten().tolist()}
