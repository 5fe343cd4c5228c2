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

Waves (a step that needs more experts than the pool holds; README feature
list, "full-layer double-buffered prefill streaming"; the feature article's
two-buffer mechanism: one buffer is computed on while the next is filled).
The pages give no rule; the reading taken is: when |needed| > S the step runs
in waves of at most floor(S/2) experts (two staging sets) — the experts
already resident first, then the others, each class ascending — and each wave
is one step of the policy above (one clock tick).  A wave's slots then carry
the newest recency, and the next wave never lacks older victims (it needs at
most floor(S/2) slots besides them), so its fills never evict an expert the
wave before it reads: wave w+1 can be copied while wave w computes.  With
S = 1 the waves hold one expert each and follow one another.  A step with
|needed| <= S is a single wave (the step above).

Hybrid execution (guide, "MoE strategies": in a hybrid step part of the misses
is fetched over PCIe and the rest computed on the CPU, at the same time; the
cpu strategy computes every miss on the CPU; "expert bank & LRU slot cache":
the cache keeps each (layer, expert)'s most recent active step so that the
per-layer fetch cap takes the most active misses first).  Reading taken:
every (layer, expert) remembers the step it was last needed in, resident or
not; a hybrid step fetches n_fetch = ceil(q * misses) of its misses (q the
fetch fraction: 1 = offload, 0 = cpu; at most max_fetch when that is >= 0),
the misses ordered by last active step, latest first (never active last; ties
lower expert first); the rest run on the CPU and take no slot.  The fetched
misses and the hits form the GPU step (waves as above; a step with no GPU
expert still advances the clock); CPU experts' last active step is that
step's clock.

Parity: pinned by hand-worked traces (tests/golden), by the textbook LRU
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
        self.last_active = {}             # (layer, expert) -> last step it was needed

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
            self.last_active[(layer, e)] = self.clock
        self.clock += 1
        return {
            "needed": needed,
            "slot_of": {e: self.where[(layer, e)] for e in needed},
            "fills": fills,
            "hits": len(needed) - len(misses),
            "misses": len(misses),
        }

    def waves(self, layer: int, counts) -> list:
        """The experts of one step, split into the waves described above."""
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        if len(needed) <= self.S:
            return [needed] if needed else []
        size = max(1, self.S // 2)
        order = ([e for e in needed if (layer, e) in self.where]
                 + [e for e in needed if (layer, e) not in self.where])
        return [order[i:i + size] for i in range(0, len(order), size)]

    def step_waves(self, layer: int, counts) -> list:
        """One step in waves: the per-wave results of step(), in wave order."""
        counts = np.asarray(counts)
        out = []
        for wave in self.waves(layer, counts):
            cw = np.zeros_like(counts)
            cw[wave] = counts[wave]
            out.append(self.step(layer, cw))
        return out

    def split_hybrid(self, layer: int, counts, fetch_fraction: float, max_fetch: int = -1):
        """(fetched misses, CPU misses) of one hybrid step, each in the order taken."""
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        misses = [e for e in needed if (layer, e) not in self.where]
        order = sorted(misses, key=lambda e: (-self.last_active.get((layer, e), -1), e))
        n_fetch = int(np.ceil(fetch_fraction * len(misses)))
        if max_fetch >= 0:
            n_fetch = min(n_fetch, max_fetch)
        return order[:n_fetch], order[n_fetch:]

    def step_hybrid(self, layer: int, counts, fetch_fraction: float, max_fetch: int = -1) -> dict:
        counts = np.asarray(counts)
        fetch, cpu = self.split_hybrid(layer, counts, fetch_fraction, max_fetch)
        gpu_counts = counts.copy()
        gpu_counts[cpu] = 0
        if np.any(gpu_counts > 0):
            waves = self.step_waves(layer, gpu_counts)
        else:
            waves = []
            self.clock += 1
        for e in cpu:
            self.last_active[(layer, e)] = self.clock - 1
        return {"fetch": fetch, "cpu": sorted(cpu), "waves": waves,
                "fills": [f for r in waves for f in r["fills"]],
                "hits": sum(r["hits"] for r in waves)}

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
