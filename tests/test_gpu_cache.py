"""GPU tests of the expert-slot cache path (slot-table indirection + LRU fills).

* cache-state invariance: with experts served from a small HBM pool refilled
  from a pinned host bank, the layer output is bit-identical to the run with
  every expert resident;
* the fills made by expert_cache_lookup/fill equal the oracle LRU's;
* after the fills, each resident slot holds exactly its bank record;
* outputs match the oracle within tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_cases import TOL, bf16_to_np, flush, rel_err
from oracle import layer as OLY
from oracle import lru as OL
from oracle import route as OR
from oracle import permute as OP

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")


def _touched(wl, b):
    ids, _ = OR.route(synth.make_logits(wl, b), wl.k)
    return len(np.unique(ids))


def _run_cache_workload(wl: synth.Workload, S: int, n_batches: int, n_layers: int = 1,
                        gen_device="cpu", check_tokens=None):
    lay = synth.record_layout(wl.fmt, wl.H, wl.I)
    stride = lay["stride"]
    # pinned bank of every (layer, expert) record
    bank = torch.empty((n_layers * wl.E, stride), dtype=torch.uint8, pin_memory=True)
    dev_sets = []
    for L in range(n_layers):
        recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, layer=L,
                                         device=gen_device)
        bank[L * wl.E:(L + 1) * wl.E].copy_(recs.cpu())
        dev_sets.append(recs.to(DEV))
        del recs
    pool = torch.empty((S, stride), dtype=torch.uint8, device=DEV)
    table = torch.full((n_layers * wl.E,), -1, dtype=torch.int32, device=DEV)
    cache = moe.ExpertCache(n_layers, wl.E, S, stride, pool, bank, table)
    ora = OL.LruSlots(S)
    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride)
    pool_W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, pool, stride)
    side = torch.cuda.Stream()
    for b in range(n_batches):
        L = b % n_layers
        lg = torch.from_numpy(synth.make_logits(wl, b)).to(DEV)
        x = torch.from_numpy(synth.make_x(wl, b).view(np.int16)).to(DEV).view(torch.bfloat16)
        y_c, info = layer.forward_cached(lg, x, L, cache, pool_W, table, side=side)
        y_c = y_c.clone()
        torch.cuda.synchronize()
        # the oracle's LRU decision for the same counts
        ids, _ = OR.route(synth.make_logits(wl, b), wl.k)
        counts, *_ = OP.permute(ids, wl.E)
        r = ora.step(L, counts)
        assert info["fills"] == r["fills"], (b, info["fills"][:5], r["fills"][:5])
        assert (info["hits"], info["misses"]) == (r["hits"], r["misses"])
        assert np.array_equal(table[L * wl.E:(L + 1) * wl.E].cpu().numpy(), ora.slot_table(L, wl.E))
        # all-resident run through the same separate calls (same kernels, same bits)
        W_r = layer.weights(dev_sets[L])
        layer.route_permute(lg)
        layer.expert_ffn(W_r, x, wl.T)
        layer.combine(wl.T, False)
        y_r = layer.y[:wl.T].clone()
        torch.cuda.synchronize()
        assert torch.equal(y_c.view(torch.int16), y_r.view(torch.int16)), f"batch {b}"
        flush(f"   batch {b} layer {L}: hits {r['hits']} misses {r['misses']}")
        if check_tokens is not None and b == 0:
            ex = OLY.ExpertSet(wl.fmt, wl.H, wl.I, lambda e: dev_sets[0][e].cpu().numpy())
            out = OLY.forward_tokens(synth.make_logits(wl, 0), synth.make_x(wl, 0), wl.k, ex,
                                     check_tokens)
            err = rel_err(bf16_to_np(y_c[check_tokens]), out["y"])
            flush(f"   oracle rel err {err:.2e}")
            assert err <= TOL
    torch.cuda.synchronize()
    # every resident slot holds its bank record
    tab = table.cpu().numpy()
    pool_h = pool.cpu()
    for key, s in ora.where.items():
        L, e = key
        assert tab[L * wl.E + e] == s
        assert torch.equal(pool_h[s], bank[L * wl.E + e]), (key, s)
    st = cache.stats()
    assert st["bytes_filled"] == st["misses"] * stride
    cache.close()
    return st


def test_cache_small_two_layers_invariance():
    wl = synth.Workload("cache_small", T=96, H=512, E=32, I=256, k=4, fmt="fp8_b128", seed=44,
                        zipf=1.2, domains=6, batches=12)
    S = max(_touched(wl, b) for b in range(12)) + 3
    assert S < wl.E
    flush(f"[cache-small] S={S}")
    st = _run_cache_workload(wl, S, 12, n_layers=2, check_tokens=[0, 50, 95])
    assert st["misses"] > 0 and st["hits"] > 0


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "bf16"])
def test_cache_other_formats(fmt):
    wl = synth.Workload("cache_fmt", T=64, H=256, E=16, I=128, k=2, fmt=fmt, seed=45, zipf=1.0,
                        domains=3, batches=6)
    S = max(_touched(wl, b) for b in range(6)) + 1
    flush(f"[cache-fmt] {fmt} S={S}")
    _run_cache_workload(wl, S, 6)


def test_cache_capacity_error_leaves_state():
    wl = synth.Workload("cache_cap", T=64, H=256, E=16, I=128, k=4, fmt="mxfp4", seed=46)
    stride = synth.record_layout(wl.fmt, wl.H, wl.I)["stride"]
    bank = torch.zeros((wl.E, stride), dtype=torch.uint8, pin_memory=True)
    pool = torch.zeros((4, stride), dtype=torch.uint8, device=DEV)
    table = torch.full((wl.E,), -1, dtype=torch.int32, device=DEV)
    cache = moe.ExpertCache(1, wl.E, 4, stride, pool, bank, table)
    counts = torch.zeros(wl.E, dtype=torch.int32)
    counts[:5] = 1
    with pytest.raises(moe.MoeError) as e:
        cache.expert_cache_lookup(0, counts)
    assert e.value.status == moe.MOE_ERR_CAPACITY
    counts[4] = 0
    me, ms, nm, nh, row = cache.expert_cache_lookup(0, counts)
    assert nm == 4 and ms.tolist() == [0, 1, 2, 3]
    # a fill list that is not the pending one is refused
    with pytest.raises(moe.MoeError):
        cache.expert_cache_fill(0, torch.tensor([7], dtype=torch.int32),
                                torch.tensor([0], dtype=torch.int32))
    cache.expert_cache_fill(0, me, ms)
    torch.cuda.synchronize()
    assert table.cpu().tolist()[:4] == [0, 1, 2, 3]
    cache.close()


def test_cache_full_size_fp8_pool():
    """The fp8 LRU-pool workload at full size (E=512, S=160) for a few batches."""
    wl = synth.WORKLOADS["fp8_lru_pool"]
    flush(f"[cache-full] {wl.name}")
    _run_cache_workload(wl, wl.pool_slots, 3, gen_device="cuda", check_tokens=[0, 2047])
