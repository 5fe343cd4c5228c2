"""Host logic of the streamed cache path (no GPU): the library's wave planner
(expert_cache_plan, host-only handles) against the oracle LRU's waves, step by
step: the same waves, the same fills wave by wave, the same slot table; a step
too large for one lookup is refused by expert_cache_lookup but planned in waves.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lru as OL

import moe_expert_ffn_router_amd as moe


@pytest.mark.parametrize("seed", range(10))
def test_plan_matches_oracle_waves(seed):
    rng = np.random.default_rng(300 + seed)
    E, S, L = int(rng.integers(6, 64)), int(rng.integers(1, 14)), int(rng.integers(1, 4))
    cache = moe.ExpertCache(L, E, S, 256)          # host metadata only
    ora = OL.LruSlots(S)
    for step in range(80):
        layer = int(rng.integers(0, L))
        counts = ((rng.random(E) < rng.uniform(0.05, 0.9)) * rng.integers(1, 5, E)).astype(np.int32)
        got = cache.expert_cache_plan(layer, torch.from_numpy(counts))
        waves = ora.waves(layer, counts)
        res = ora.step_waves(layer, counts)
        assert got["waves"] == [sorted(w) for w in waves], step
        assert got["fills"] == [r["fills"] for r in res], step
        assert got["hits"] == sum(r["hits"] for r in res)
        row = cache.expert_cache_row(layer).numpy()
        assert np.array_equal(row, ora.slot_table(layer, E))
    cache.close()


def test_single_lookup_refuses_what_waves_plan():
    E, S = 24, 5
    cache = moe.ExpertCache(1, E, S, 256)
    counts = np.zeros(E, np.int32)
    counts[:9] = 1
    with pytest.raises(moe.MoeError) as e:
        cache.expert_cache_lookup(0, torch.from_numpy(counts))
    assert e.value.status == moe.MOE_ERR_CAPACITY
    got = cache.expert_cache_plan(0, torch.from_numpy(counts))
    assert got["n_waves"] == 5 and all(len(w) <= 2 for w in got["waves"])   # floor(5/2)
    assert got["misses"] == 9
    cache.close()


def test_streamed_argument_checks_before_any_device_work():
    cache = moe.ExpertCache(1, 16, 4, 256)          # no pool: refused, nothing enqueued
    W = moe.experts("mxfp4", 16, 256, 128, 0, 256)
    counts = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(moe.MoeError) as e:
        cache.moe_expert_ffn_streamed(0, W, None, 4, 2, counts, None, None, None, 2,
                                      torch.zeros(16, dtype=torch.uint8), side=0, compute=0)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG
    cache.close()


@pytest.mark.parametrize("seed", range(8))
def test_hybrid_plan_matches_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    E, S, L = int(rng.integers(6, 48)), int(rng.integers(1, 12)), int(rng.integers(1, 3))
    cache = moe.ExpertCache(L, E, S, 256)
    ora = OL.LruSlots(S)
    for step in range(60):
        layer = int(rng.integers(0, L))
        counts = ((rng.random(E) < rng.uniform(0.05, 0.7)) * rng.integers(1, 5, E)).astype(np.int32)
        q = float(rng.choice([0.0, 0.25, 0.5, 0.7, 1.0]))
        mf = int(rng.integers(-1, 5))
        got = cache.expert_cache_plan_hybrid(layer, torch.from_numpy(counts), q, mf)
        ref = ora.step_hybrid(layer, counts, q, mf)
        assert got["cpu"] == ref["cpu"], step
        assert got["fills"] == [r["fills"] for r in ref["waves"]], step
        assert got["hits"] == ref["hits"]
        assert np.array_equal(cache.expert_cache_row(layer).numpy(), ora.slot_table(layer, E))
    cache.close()
