"""Expert-slot cache policy (oracle).

The FreeToken supported-models guide (section "expert bank & LRU slot cache")
describes a GPU pool of expert slots managed with an LRU policy that records,
for every (layer, expert), the most recent step in which it was active; misses
are fetched from a pinned host bank over PCIe (section "MoE strategies",
offload).  Its "minimum cache constraint" section says too small a cache is
refused outright.  The pages fix no tie-breaks; the plainest deterministic
reading, taken here, is:

  state   owner[s] = (layer, expert) or empty, recency[s], a step clock that
          advances once per (layer-)step
  step    needed  = experts with count > 0, ascending
          if |needed| > S: refuse (capacity error), state unchanged
          misses  = needed that are not resident, ascending
          each miss takes the lowest-index empty slot, else the resident slot
          whose owner is not needed now with the smallest (recency, slot)
          every needed slot's recency := clock; clock += 1

Outputs per step: the slot of every needed expert, the (expert, slot) fills in
order, hit and miss counts.

Resize (README feature list, elastic VRAM: the pool changes size while the
engine runs, no reload).  The pages give no rule for what a smaller pool
keeps; the reading taken is LRU order: keep the min(new S, resident count)
residents with the latest recency (ties: lower slot), drop the rest, and place
the kept ones, in ascending order of their old slot, into slots 0, 1, ...;
recencies and the clock are unchanged.

Parity: pinned by a hand-worked trace (tests/golden), by the textbook LRU
stack-distance rule on single-expert steps, by a textbook recency-list LRU
whose capacity changes between steps, and by invariants.
"""
from __future__ import annotations

import numpy as np


class CapacityError(RuntimeError):
    pass


class LruSlots:
    def __init__(self, S: int):
        if S < 1:
            raise ValueError("S >= 1")
        self.S = S
        self.owner = [None] * S           # (layer, expert) or None
        self.recency = [-1] * S
        self.where = {}                   # (layer, expert) -> slot
        self.clock = 0

    def step(self, layer: int, counts) -> dict:
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        if len(needed) > self.S:
            raise CapacityError(f"{len(needed)} experts needed, {self.S} slots")
        need_keys = {(layer, e) for e in needed}
        misses = [e for e in needed if (layer, e) not in self.where]
        fills = []
        for e in misses:
            empty = [s for s in range(self.S) if self.owner[s] is None]
            if empty:
                s = empty[0]
            else:
                cands = [s for s in range(self.S) if self.owner[s] not in need_keys]
                s = min(cands, key=lambda q: (self.recency[q], q))
                del self.where[self.owner[s]]
            self.owner[s] = (layer, e)
            self.where[(layer, e)] = s
            fills.append((e, s))
        for e in needed:
            self.recency[self.where[(layer, e)]] = self.clock
        self.clock += 1
        return {
            "needed": needed,
            "slot_of": {e: self.where[(layer, e)] for e in needed},
            "fills": fills,
            "hits": len(needed) - len(misses),
            "misses": len(misses),
        }

    def resize(self, new_S: int) -> list:
        """New pool size; returns the (old slot, new slot) of every kept resident."""
        if new_S < 1:
            raise ValueError("S >= 1")
        resident = [s for s in range(self.S) if self.owner[s] is not None]
        by_recency = sorted(resident, key=lambda q: (-self.recency[q], q))
        kept = sorted(by_recency[:new_S])
        owner = [None] * new_S
        recency = [-1] * new_S
        moves = []
        for p, q in enumerate(kept):
            owner[p], recency[p] = self.owner[q], self.recency[q]
            moves.append((q, p))
        self.S, self.owner, self.recency = new_S, owner, recency
        self.where = {key: p for p, key in enumerate(owner) if key is not None}
        return moves

    def slot_table(self, layer: int, E: int) -> np.ndarray:
        """Slot of every expert of `layer` that is resident, -1 otherwise."""
        t = np.full(E, -1, dtype=np.int32)
        for (l, e), s in self.where.items():
            if l == layer:
                t[e] = s
        return t
