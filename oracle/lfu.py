"""Oracle: bounded slot pool with LFU + recency eviction (simulation).

The pages ("How it works"; relationship-to-TurboFieldfare section) say hot
experts are cached in a bounded slot pool and evicted by LFU plus recency,
with measured hit rates of 43-70 %.  They give no formula.  Reading:

  * every selection of expert e (one per (token, rank)) adds 1 to count[e],
    and stamps last[e] = step; counts are cumulative over the run;
  * a step needs the distinct experts it selected, taken in first-appearance
    order of the rank-ordered selection list;
  * a needed expert already resident is a hit; otherwise it is loaded into the
    lowest-numbered free slot, or, when none is free, into the slot of the
    resident expert not needed this step with the smallest
    (count, last, expert id) — least frequent, then least recent, then lowest id;
  * hit rate = hits / (hits + misses) over distinct needed experts.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


class SlotPoolSim:
    def __init__(self, E: int, n_slots: int):
        self.E = E
        self.n_slots = n_slots
        self.count = [0] * E
        self.last = [-1] * E
        self.slot_of = [-1] * E
        self.holder = [-1] * n_slots
        self.step = 0
        self.hits = 0
        self.misses = 0

    def plan(self, selected: Sequence[int]) -> List[Tuple[int, int, int]]:
        """Account one step's selections; return loads as (expert, slot, evicted)."""
        need = []
        seen = set()
        for e in selected:
            e = int(e)
            self.count[e] += 1
            self.last[e] = self.step
            if e not in seen:
                seen.add(e)
                need.append(e)
        if len(need) > self.n_slots:
            raise ValueError("pool too small for one step's demand")
        loads = []
        for e in need:
            if self.slot_of[e] >= 0:
                self.hits += 1
                continue
            self.misses += 1
            free = [s for s in range(self.n_slots) if self.holder[s] < 0]
            if free:
                slot, victim = free[0], -1
            else:
                cands = [v for v in range(self.E) if self.slot_of[v] >= 0 and v not in seen]
                victim = min(cands, key=lambda v: (self.count[v], self.last[v], v))
                slot = self.slot_of[victim]
                self.slot_of[victim] = -1
            self.holder[slot] = e
            self.slot_of[e] = slot
            loads.append((e, slot, victim))
        self.step += 1
        return loads

    @property
    def hit_rate(self) -> float:
        n = self.hits + self.misses
        return self.hits / n if n else 0.0
