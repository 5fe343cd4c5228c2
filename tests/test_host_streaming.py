"""Host logic of the streamed cache path (no GPU): wave planning, fill-group
splits, and the LRU policy run wave by wave through the library's host-only
cache handle, checked against the oracle LRU applied to the same waves.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from moe_expert_ffn_router_amd.layer import plan_waves, split_groups
from oracle import lru as OL

import moe_expert_ffn_router_amd as moe


def test_plan_waves_partition_and_order():
    rng = np.random.default_rng(3)
    for _ in range(200):
        E = int(rng.integers(1, 64))
        S = int(rng.integers(1, 20))
        counts = rng.integers(0, 3, size=E) * (rng.random(E) < 0.6)
        resident = np.where(rng.random(E) < 0.3, rng.integers(0, S, size=E), -1)
        waves = plan_waves(counts, S, resident)
        flat = [e for w in waves for e in w]
        needed = [e for e in range(E) if counts[e] > 0]
        assert sorted(flat) == needed and len(flat) == len(set(flat))
        assert all(1 <= len(w) <= S for w in waves)
        assert all(len(w) == S for w in waves[:-1])
        # resident experts come first, each class ascending
        res = [e for e in needed if resident[e] >= 0]
        non = [e for e in needed if resident[e] < 0]
        assert flat == res + non
    assert plan_waves(np.zeros(8), 4) == []
    assert plan_waves(np.array([0, 2, 0, 1, 5]), 8) == [[1, 3, 4]]


def test_split_groups():
    for n in range(0, 40):
        for g in range(1, 17):
            parts = split_groups(n, g)
            assert len(parts) == g and parts[0][0] == 0 and parts[-1][1] == n
            assert all(a[1] == b[0] for a, b in zip(parts, parts[1:]))
            sizes = [b - a for a, b in parts]
            assert max(sizes) - min(sizes) <= 1


def test_waves_through_host_only_cache_match_oracle():
    """A step needing more experts than slots fails as one lookup and succeeds
    wave by wave; every wave's misses and slots equal the oracle LRU's."""
    E, S, L = 24, 5, 2
    cache = moe.ExpertCache(L, E, S, 256)  # host metadata only
    ora = OL.LruSlots(S)
    rng = np.random.default_rng(11)
    resident = {l: None for l in range(L)}
    for step in range(30):
        layer = step % L
        counts = (rng.random(E) < 0.5).astype(np.int32) * rng.integers(1, 4, size=E)
        if int((counts > 0).sum()) > S:
            with pytest.raises(moe.MoeError) as e:
                cache.expert_cache_lookup(layer, torch.from_numpy(counts.astype(np.int32)))
            assert e.value.status == moe.MOE_ERR_CAPACITY
        for wave in plan_waves(counts, S, resident[layer]):
            cw = np.zeros(E, dtype=np.int32)
            cw[wave] = counts[wave]
            me, ms, nm, nh, row = cache.expert_cache_lookup(layer, torch.from_numpy(cw))
            r = ora.step(layer, cw)
            assert list(zip(me.tolist(), ms.tolist())) == r["fills"]
            assert (nh, nm) == (r["hits"], r["misses"])
            assert np.array_equal(row.numpy(), ora.slot_table(layer, E))
            resident[layer] = row.numpy()
    cache.close()
