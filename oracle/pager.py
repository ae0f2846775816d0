"""CPU model of the expert slot arena (expert paging), test infrastructure.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code with the GPU library and
never imports it.

What it models comes from the HelloSun/ling30tiny model card: its introduction
describes experts that are not active staying off the compute device while a
bounded arena holds the experts the router currently selects, and its table of
RAM-limit measurements (RAM 上限實測) reports the arena as a number of slots and a
hot rate.  The pages give no replacement policy; this model takes these readings:

  R18  one slot holds one routed expert (gate, up and down); per call the distinct
       experts the routing selects are looked up; an expert already resident is a
       hit, the others are misses and are copied into slots; victims are the slots
       whose expert the call does not need, least recently used first (a slot's
       stamp is the number of the last call that used it; slots never used have
       stamp 0 and go first), ties to the lower slot; the misses, in ascending
       expert order, take the victims in that order.  hot rate = hits / lookups.
       Shared experts are not paged (every token uses them).

The arena must hold at least as many slots as one call can need, so no expert a
call needs is evicted during that call.
"""
from __future__ import annotations

import numpy as np


class SlotArena:
    """Residency tables and counters of one layer's arena of `num_slots` slots over
    `num_experts` routed experts."""

    def __init__(self, num_experts: int, num_slots: int):
        self.E, self.N = num_experts, num_slots
        self.key_slot = np.full(num_experts, -1, dtype=np.int64)
        self.slot_key = np.full(num_slots, -1, dtype=np.int64)
        self.stamp = np.zeros(num_slots, dtype=np.int64)
        self.calls = 0
        self.refs = 0        # routed (token, slot) references
        self.lookups = 0     # distinct experts needed, summed over calls
        self.hits = 0
        self.misses = 0

    def step(self, ids):
        """One call with routed ids [T, k].  Returns (slot ids [T, k], copies [(expert,
        slot)] in the order the misses take their victims)."""
        ids = np.asarray(ids, dtype=np.int64)
        need = np.unique(ids)
        if need.size > self.N:
            raise ValueError("the arena holds fewer slots than one call needs")
        clock = self.calls + 1
        hit = need[self.key_slot[need] >= 0]
        miss = need[self.key_slot[need] < 0]
        needed_slots = set(self.key_slot[hit].tolist())
        cand = [s for s in range(self.N) if s not in needed_slots]
        cand.sort(key=lambda s: (self.stamp[s], s))
        copies = []
        for e, s in zip(miss.tolist(), cand[:miss.size]):
            old = self.slot_key[s]
            if old >= 0:
                self.key_slot[old] = -1
            self.slot_key[s] = e
            self.key_slot[e] = s
            copies.append((e, s))
        self.stamp[self.key_slot[need]] = clock
        self.calls = clock
        self.refs += ids.size
        self.lookups += need.size
        self.hits += hit.size
        self.misses += miss.size
        return self.key_slot[ids], copies

    def hot_rate(self) -> float:
        return self.hits / self.lookups if self.lookups else 0.0
