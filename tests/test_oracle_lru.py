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


def test_resize_hand_worked():
    """S = 4, one layer: experts 1, 2, 3, 4 fill slots 0..3 at steps 0..3, expert 2
    is used again at step 4.  Shrinking to 2 keeps the two most recently used
    (expert 2 in slot 1, step 4; expert 4 in slot 3, step 3), packed in slot
    order; growing to 3 keeps both where they are; the next miss takes slot 2."""
    c = lru.LruSlots(4)
    for e in (1, 2, 3, 4, 2):
        counts = np.zeros(8, np.int32)
        counts[e] = 1
        c.step(0, counts)
    assert c.resize(2) == [(1, 0), (3, 1)]
    assert c.slot_table(0, 8).tolist() == [-1, -1, 0, -1, 1, -1, -1, -1]
    assert c.resize(3) == [(0, 0), (1, 1)]
    counts = np.zeros(8, np.int32)
    counts[[2, 5]] = 1
    r = c.step(0, counts)
    assert r["fills"] == [(5, 2)] and r["hits"] == 1


def _textbook_lru_hits(seq, caps):
    """Textbook LRU as a recency list (most recent first) whose capacity is
    caps[i] when access i is made: a key is cached iff it is among the first
    `capacity` entries; a capacity change truncates the list."""
    stack, hits = [], []
    for key, cap in zip(seq, caps):
        del stack[cap:]
        hits.append(key in stack)
        if key in stack:
            stack.remove(key)
        stack.insert(0, key)
        del stack[cap:]
    return hits


@pytest.mark.parametrize("seed", range(8))
def test_resize_single_expert_steps_match_textbook_lru(seed):
    rng = np.random.default_rng(50 + seed)
    seq = [(int(rng.integers(0, 3)), int(rng.integers(0, 10))) for _ in range(300)]
    caps, cap = [], int(rng.integers(1, 8))
    for i in range(len(seq)):
        if i and rng.random() < 0.05:
            cap = int(rng.integers(1, 12))
        caps.append(cap)
    c = lru.LruSlots(caps[0])
    got = []
    for (layer, e), cap in zip(seq, caps):
        if cap != c.S:
            c.resize(cap)
        counts = np.zeros(10, np.int32)
        counts[e] = 2
        got.append(c.step(layer, counts)["hits"] == 1)
    assert got == _textbook_lru_hits(seq, caps)


@pytest.mark.parametrize("seed", range(4))
def test_resize_invariants_multi_expert(seed):
    rng = np.random.default_rng(300 + seed)
    E = 24
    c = lru.LruSlots(10)
    for step in range(200):
        if rng.random() < 0.1:
            new_S = int(rng.integers(1, 16))
            before = {key: (s, c.recency[s]) for key, s in c.where.items()}
            moves = c.resize(new_S)
            kept = {c.owner[p] for p in range(len(moves))}
            assert len(moves) == min(new_S, len(before)) == len(c.where)
            assert [p for _, p in moves] == list(range(len(moves)))
            assert [q for q, _ in moves] == sorted(q for q, _ in moves)
            for q, p in moves:                          # bytes follow their owner
                assert before[c.owner[p]][0] == q
            if kept:                                    # nothing dropped is more recent
                worst = min(before[k][1] for k in kept)
                assert all(r <= worst for k, (s, r) in before.items() if k not in kept)
            continue
        layer = int(rng.integers(0, 2))
        n = int(rng.integers(0, c.S + 1))
        counts = np.zeros(E, np.int32)
        counts[rng.permutation(E)[:n]] = 1
        r = c.step(layer, counts)
        assert len(set(r["slot_of"].values())) == n and all(0 <= s < c.S for s in r["slot_of"].values())


# ---- waves (a step needing more experts than the pool holds) --------------
def _wave_trace():
    rows = []
    with open(os.path.join(GOLDEN, "lru_waves_trace.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            S, layer, needed, waves, fills = [p.strip() for p in line.split("|")]
            waves = [[int(v) for v in w.split()] for w in waves.split(";")]
            fills = [[] if fw.strip() == "-" else
                     [tuple(int(v) for v in f_.split(":")) for f_ in fw.split()]
                     for fw in fills.split(";")]
            rows.append((int(S), int(layer), [int(v) for v in needed.split()], waves, fills))
    return rows


def test_waves_hand_worked_trace():
    caches = {}
    for S, layer, needed, waves, fills in _wave_trace():
        c = caches.setdefault(S, lru.LruSlots(S))
        counts = np.zeros(8, np.int32)
        counts[needed] = 1 + np.arange(len(needed))
        assert c.waves(layer, counts) == waves, (S, needed)
        res = c.step_waves(layer, counts)
        assert [r["fills"] for r in res] == fills, (S, needed)
        assert [r["needed"] for r in res] == waves


@pytest.mark.parametrize("seed", range(12))
def test_waves_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    S, E = int(rng.integers(1, 12)), int(rng.integers(8, 40))
    c = lru.LruSlots(S)
    for t in range(60):
        layer = int(rng.integers(0, 2))
        counts = (rng.random(E) < rng.uniform(0.05, 0.8)) * rng.integers(1, 9, E)
        needed = [int(e) for e in np.nonzero(counts)[0]]
        resident = {e for e in needed if (layer, e) in c.where}
        if len(needed) <= S:
            ref = lru.LruSlots(S)
            ref.owner, ref.recency = list(c.owner), list(c.recency)
            ref.where, ref.clock = dict(c.where), c.clock
            one = ref.step(layer, counts)
        waves = c.waves(layer, counts)
        res = c.step_waves(layer, counts)
        assert sorted(e for w in waves for e in w) == needed
        if len(needed) > S:
            assert all(len(w) <= max(1, S // 2) for w in waves)
        else:
            assert len(res) == (1 if needed else 0)
            if needed:
                assert res[0]["fills"] == one["fills"]
        flat = [e for w in waves for e in w]
        n_res = sum(1 for e in flat if e in resident)
        if len(needed) > S:
            assert set(flat[:n_res]) == resident             # resident experts first
        prev = set()
        for w, r in zip(waves, res):
            assert r["needed"] == sorted(w)
            if S >= 2:                                        # never evicts the wave before
                assert not {s for _, s in r["fills"]} & prev
            assert sorted(r["slot_of"]) == sorted(w)
            assert len(set(r["slot_of"].values())) == len(w)
            prev = set(r["slot_of"].values())
        for e in waves[-1] if waves else []:
            assert (layer, e) in c.where


# ---- hybrid steps (part of the misses on the CPU) -------------------------
def test_hybrid_hand_worked_trace():
    c = lru.LruSlots(4)
    with open(os.path.join(GOLDEN, "lru_hybrid_trace.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 5
    for line in rows:
        needed, q, mf, fills, cpu, hits = [p.strip() for p in line.split("|")]
        counts = np.zeros(8, np.int32)
        counts[[int(v) for v in needed.split()]] = 3
        r = c.step_hybrid(0, counts, float(q), int(mf))
        exp_f = [] if fills == "-" else [tuple(int(v) for v in x.split(":")) for x in fills.split()]
        exp_c = [] if cpu == "-" else [int(v) for v in cpu.split()]
        assert (r["fills"], r["cpu"], r["hits"]) == (exp_f, exp_c, int(hits)), line


@pytest.mark.parametrize("seed", range(6))
def test_hybrid_invariants_and_extremes(seed):
    rng = np.random.default_rng(700 + seed)
    S, E = int(rng.integers(2, 10)), int(rng.integers(8, 30))
    a, b, c = lru.LruSlots(S), lru.LruSlots(S), lru.LruSlots(S)
    for t in range(50):
        counts = ((rng.random(E) < 0.4) * rng.integers(1, 4, E)).astype(np.int32)
        needed = set(np.nonzero(counts)[0].tolist())
        # q = 1 with no cap is the offload step (waves included)
        ra = a.step_hybrid(0, counts, 1.0)
        rb = b.step_waves(0, counts)
        assert ra["cpu"] == [] and ra["fills"] == [f for r in rb for f in r["fills"]]
        # any q: CPU experts are misses, take no slot, fetched + cpu = misses
        misses = {e for e in needed if (0, e) not in c.where}
        q = float(rng.choice([0.0, 0.3, 0.5, 1.0]))
        c0 = c.clock
        rc = c.step_hybrid(0, counts, q, int(rng.integers(-1, 4)))
        assert set(rc["cpu"]) | set(rc["fetch"]) == misses
        assert not set(rc["cpu"]) & set(rc["fetch"])
        assert all((0, e) not in c.where for e in rc["cpu"])
        assert {e for e, _ in rc["fills"]} == set(rc["fetch"])
        for e in needed:
            assert c0 <= c.last_active[(0, e)] <= c.clock - 1
        for e in rc["cpu"]:
            assert c.last_active[(0, e)] == c.clock - 1
