"""Oracle of the expert cache used under physical expert offload.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`): never imported by the product
path; shares no code with the HIP library.

[AcceptMoE news §02]: an expert already on the GPU runs directly; one that is
not must be loaded from CPU memory first.  [AcceptMoE news §03]: 48 expert
slots per layer; reported are host-to-device expert bytes and the expert-cache
hit rate.  The pages name no replacement policy.  Reading taken here (listed
in DESIGN.md): least recently used, where "use" is a block in which the
expert is active, an expert active in the current block is never evicted,
empty slots are filled first (lowest slot first), ties between equally old
slots go to the lowest slot, misses are placed in ascending expert order, and
a miss that finds no slot goes to a one-block spill slot (loaded again on its
next use).

Pinned by ``tests/test_cache_cpu.py``: a hand-traced sequence, invariants,
and agreement with brute-force recomputation of "least recently used" from
the full history of blocks.
"""

from __future__ import annotations


class LRUExpertCache:
    """Slots 0..n_slots-1 persistent, spill slots n_slots.. for one block."""

    def __init__(self, n_slots: int, n_spill: int, warm=()):
        self.n_slots, self.n_spill = n_slots, n_spill
        self.holder = [None] * n_slots       # expert in each persistent slot
        self.stamp = [0] * n_slots           # block number of the slot's last use
        for q, e in enumerate(warm):
            self.holder[q] = int(e)
        self.block = 0
        self.hits = self.misses = self.spills = 0

    def resident(self) -> set:
        return {e for e in self.holder if e is not None}

    def slot_of(self, e: int):
        return self.holder.index(e) if e in self.holder else None

    def step(self, active):
        """One block: returns the fetches [(expert, slot), ...] in order, or
        raises ValueError (state unchanged) when the spill slots run out."""
        active = sorted(int(e) for e in active)
        if len(set(active)) != len(active):
            raise ValueError("repeated expert")
        act = set(active)
        missing = [e for e in active if e not in self.resident()]
        usable = sum(1 for e in self.holder if e is None or e not in act)
        if len(missing) - usable > self.n_spill:
            raise ValueError("not enough spill slots")
        self.block += 1
        for e in active:
            q = self.slot_of(e)
            if q is not None:
                self.stamp[q] = self.block
                self.hits += 1
        fetches = []
        spilled = 0
        for e in missing:
            empty = [q for q in range(self.n_slots) if self.holder[q] is None]
            if empty:
                q = empty[0]
            else:
                free = [q for q in range(self.n_slots) if self.holder[q] not in act]
                q = min(free, key=lambda s: (self.stamp[s], s)) if free else None
            if q is None:
                q = self.n_slots + spilled
                spilled += 1
            else:
                self.holder[q] = e
                self.stamp[q] = self.block
            fetches.append((e, q))
        self.misses += len(fetches)
        self.spills += spilled
        return fetches
