"""Pins of the oracle's LRU slot policy (CPU only)."""
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import lru


def _trace():
    rows = []
    with open(os.path.join(GOLDEN, "lru_trace.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = [p.strip() for p in line.split("|")]
            layer = int(parts[0])
            needed = [int(v) for v in parts[1].split()]
            if parts[2] == "CAPACITY":
                rows.append((layer, needed, None))
            else:
                fills = [tuple(int(v) for v in fs.split(":")) for fs in parts[2].split()]
                rows.append((layer, needed, (fills, int(parts[3]), int(parts[4]))))
    return rows


def test_hand_worked_trace():
    c = lru.LruSlots(3)
    for layer, needed, exp in _trace():
        counts = np.zeros(8, np.int32)
        counts[needed] = 1
        if exp is None:
            with pytest.raises(lru.CapacityError):
                c.step(layer, counts)
            continue
        r = c.step(layer, counts)
        assert (r["fills"], r["hits"], r["misses"]) == exp, (layer, needed)


def _stack_distance_hits(seq, S):
    """Textbook LRU: an access hits iff fewer than S distinct other keys were
    touched since its previous access (the LRU stack property)."""
    hits = []
    for i, key in enumerate(seq):
        prev = max((j for j in range(i) if seq[j] == key), default=None)
        if prev is None:
            hits.append(False)
        else:
            hits.append(len(set(seq[prev + 1:i]) - {key}) < S)
    return hits


@pytest.mark.parametrize("seed", range(8))
def test_single_expert_steps_reduce_to_textbook_lru(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 6))
    seq = [(int(rng.integers(0, 2)), int(rng.integers(0, 9))) for _ in range(200)]
    c = lru.LruSlots(S)
    got = []
    for layer, e in seq:
        counts = np.zeros(9, np.int32)
        counts[e] = 3
        got.append(c.step(layer, counts)["hits"] == 1)
    assert got == _stack_distance_hits(seq, S)


@pytest.mark.parametrize("seed", range(6))
def test_invariants_random_multi_expert(seed):
    rng = np.random.default_rng(100 + seed)
    E, S = 32, 12
    c = lru.LruSlots(S)
    for step in range(150):
        layer = int(rng.integers(0, 3))
        n = int(rng.integers(0, S + 3))
        counts = np.zeros(E, np.int32)
        counts[rng.permutation(E)[:n]] = rng.integers(1, 5, size=n)
        needed = list(np.nonzero(counts)[0])
        before = dict(c.where)
        if len(needed) > S:
            with pytest.raises(lru.CapacityError):
                c.step(layer, counts)
            assert c.where == before
            continue
        r = c.step(layer, counts)
        assert len(c.where) <= S
        slots = [r["slot_of"][e] for e in needed]
        assert len(set(slots)) == len(slots)            # distinct slots
        for e in needed:                                # needed resident after fill
            assert c.where[(layer, e)] == r["slot_of"][e]
        for key, s in before.items():                   # hits keep their slot
            if key[0] == layer and key[1] in needed:
                assert r["slot_of"][key[1]] == s
        assert r["hits"] + r["misses"] == len(needed)
        tab = c.slot_table(layer, E)
        assert all(tab[e] == r["slot_of"][e] for e in needed)


def test_compulsory_misses_only_when_everything_fits():
    c = lru.LruSlots(10)
    rng = np.random.default_rng(1)
    seen, misses = set(), 0
    for _ in range(50):
        counts = np.zeros(10, np.int32)
        counts[rng.permutation(10)[:4]] = 1
        r = c.step(0, counts)
        misses += r["misses"]
        seen |= set(r["needed"])
    assert misses == len(seen)
