"""GPU tests of the expert-slot cache path (slot-table indirection + LRU fills).

* cache-state invariance: with experts served from a small HBM pool refilled
  from a pinned host bank, the layer output is bit-identical to the run with
  every expert resident;
* the fills made by expert_cache_lookup/fill equal the oracle LRU's;
* after the fills, each resident slot holds exactly its bank record;
* outputs match the oracle within tolerance;
* several layers sharing one pool across run-time resizes of the pool.
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


# ---------------------------------------------------------------------------
# streamed path: FFN behind grouped fills, waves when a step needs > S experts
# ---------------------------------------------------------------------------
def _pool_set(wl, S, gen_device="cpu"):
    stride = synth.record_layout(wl.fmt, wl.H, wl.I)["stride"]
    recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, device=gen_device)
    bank = torch.empty((wl.E, stride), dtype=torch.uint8, pin_memory=True)
    bank.copy_(recs.cpu())
    pool = torch.empty((S, stride), dtype=torch.uint8, device=DEV)
    table = torch.full((wl.E,), -1, dtype=torch.int32, device=DEV)
    cache = moe.ExpertCache(1, wl.E, S, stride, pool, bank, table)
    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride)
    pool_W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, pool, stride)
    return dict(stride=stride, dev=recs.to(DEV), bank=bank, pool=pool, table=table, cache=cache,
                layer=layer, pool_W=pool_W)


def _batch(wl, b):
    lg = torch.from_numpy(synth.make_logits(wl, b)).to(DEV)
    x = torch.from_numpy(synth.make_x(wl, b).view(np.int16)).to(DEV).view(torch.bfloat16)
    return lg, x


@pytest.mark.parametrize("fmt,groups", [("fp8_b128", 3), ("mxfp4", 1), ("nvfp4", 4),
                                        ("bf16", 2)])
def test_streamed_matches_cached(fmt, groups):
    """With every step within the pool, the streamed path makes the same fills
    and gives bit-identical outputs to the one-fill path."""
    wl = synth.Workload("stream_eq", T=96, H=512, E=32, I=256, k=4, fmt=fmt, seed=47, zipf=1.2,
                        domains=6, batches=8)
    S = max(_touched(wl, b) for b in range(8)) + 2
    flush(f"[stream-eq] {fmt} S={S} groups={groups}")
    a, s = _pool_set(wl, S), _pool_set(wl, S)
    side_a, side_s = torch.cuda.Stream(), torch.cuda.Stream()
    for b in range(8):
        lg, x = _batch(wl, b)
        y_a, ia = a["layer"].forward_cached(lg, x, 0, a["cache"], a["pool_W"], a["table"],
                                            side=side_a)
        y_s, is_ = s["layer"].forward_streamed(lg, x, 0, s["cache"], s["pool_W"], s["table"],
                                               side=side_s, groups=groups)
        torch.cuda.synchronize()
        assert is_["waves"] == 1 and is_["fills"] == ia["fills"]
        assert (is_["hits"], is_["misses"]) == (ia["hits"], ia["misses"])
        assert torch.equal(y_a.view(torch.int16), y_s.view(torch.int16)), f"batch {b}"
    assert torch.equal(a["table"], s["table"])
    for d in (a, s):
        d["cache"].close()


@pytest.mark.parametrize("fmt", ["fp8_b128", "mxfp4"])
def test_streamed_waves_exceed_pool(fmt):
    """A pool smaller than one step's experts: the streamed path runs the step
    in waves of at most S/2 (two staging sets, each wave's copies overlapping the
    wave before); fills follow the oracle's waves, every slot holds its bank
    record, y is bit-identical to the all-resident run and matches the oracle."""
    wl = synth.Workload("stream_waves", T=96, H=512, E=32, I=256, k=4, fmt=fmt, seed=48, zipf=1.0,
                        domains=3, batches=6)
    S = 6
    d = _pool_set(wl, S)
    ora = OL.LruSlots(S)
    side = torch.cuda.Stream()
    for b in range(6):
        lg, x = _batch(wl, b)
        y_s, info = d["layer"].forward_streamed(lg, x, 0, d["cache"], d["pool_W"], d["table"],
                                                side=side, groups=2)
        y_s = y_s.clone()
        torch.cuda.synchronize()
        ids, _ = OR.route(synth.make_logits(wl, b), wl.k)
        counts, *_ = OP.permute(ids, wl.E)
        assert int((counts > 0).sum()) > S
        res = ora.step_waves(0, counts)
        fills = [f for r in res for f in r["fills"]]
        assert all(len(r["needed"]) <= S // 2 for r in res)     # two staging sets
        assert info["waves"] == len(res) and info["fills"] == fills, b
        # all-resident run through the same separate calls
        lay = d["layer"]
        lay.route_permute(lg)
        lay.expert_ffn(lay.weights(d["dev"]), x, wl.T)
        lay.combine(wl.T, False)
        y_r = lay.y[:wl.T].clone()
        torch.cuda.synchronize()
        assert torch.equal(y_s.view(torch.int16), y_r.view(torch.int16)), f"batch {b}"
        if b == 0:
            ex = OLY.ExpertSet(wl.fmt, wl.H, wl.I, lambda e: d["bank"][e].numpy())
            toks = [0, 7, 50, wl.T - 1]
            out = OLY.forward_tokens(synth.make_logits(wl, b), synth.make_x(wl, b), wl.k, ex, toks)
            assert rel_err(bf16_to_np(y_s[toks]), out["y"]) <= TOL
        flush(f"   batch {b}: waves {info['waves']} hits {info['hits']} misses {info['misses']}")
    tab = d["table"].cpu().numpy()
    pool_h = d["pool"].cpu()
    for (L, e), s in ora.where.items():
        assert tab[e] == s and torch.equal(pool_h[s], d["bank"][e]), (e, s)
    d["cache"].close()


def test_shared_pool_layers_with_resizes():
    """Three layers share one pool (keys (layer, expert)); the pool shrinks in
    place, grows in place and moves into a new, larger allocation between
    steps.  After each resize every kept slot holds its bank record and every
    layer's slot-table row is the oracle's; the streamed path's fills follow the
    oracle LRU (waves where a step needs more experts than the pool holds) and
    y is bit-identical to the all-resident run."""
    wl = synth.Workload("pool_resize", T=48, H=512, E=32, I=256, k=2, fmt="mxfp4", seed=51,
                        zipf=1.3, domains=2, batches=12)
    L, S0, S_cap = 2, 24, 40
    stride = synth.record_layout(wl.fmt, wl.H, wl.I)["stride"]
    bank = torch.empty((L * wl.E, stride), dtype=torch.uint8, pin_memory=True)
    dev_sets = []
    for li in range(L):
        recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, layer=li)
        bank[li * wl.E:(li + 1) * wl.E].copy_(recs)
        dev_sets.append(recs.to(DEV))
    pool = torch.zeros((S_cap, stride), dtype=torch.uint8, device=DEV)  # room to grow in place
    table = torch.full((L * wl.E,), -1, dtype=torch.int32, device=DEV)
    cache = moe.ExpertCache(L, wl.E, S0, stride, pool, bank, table)
    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride)
    pool_W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, pool, stride)
    ora = OL.LruSlots(S0)
    side = torch.cuda.Stream()
    plan = {4: ("shrink", 9), 8: ("grow", 30), 12: ("move", 48), 16: ("shrink", 16)}
    flush(f"[pool-resize] L={L} S0={S0}")
    hits_after_resize = 0

    def check_pool(tag, whole_table):
        tab = table.cpu().numpy()
        pool_h = pool.cpu()
        if whole_table:  # a resize rewrites every row; fills publish only their own layer's
            for li in range(L):
                assert np.array_equal(tab[li * wl.E:(li + 1) * wl.E],
                                      ora.slot_table(li, wl.E)), tag
        for (li, e), s in ora.where.items():
            assert tab[li * wl.E + e] == s, (tag, li, e)
            assert torch.equal(pool_h[s], bank[li * wl.E + e]), (tag, li, e, s)

    for step in range(20):
        if step in plan:
            kind, new_S = plan[step]
            if kind == "move":
                pool = torch.zeros((new_S, stride), dtype=torch.uint8, device=DEV)
                moves = cache.moe_cache_resize(new_S, pool, side=side)
                pool_W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, pool, stride)
            else:
                moves = cache.moe_cache_resize(new_S, side=side)
            exp = ora.resize(new_S)
            assert list(zip(*(t.tolist() for t in moves))) == exp, step
            check_pool(f"after {kind} to {new_S}", True)
            flush(f"   step {step}: {kind} to {new_S}, kept {len(exp)}")
        li = step % L
        b = step % wl.batches
        lg, x = _batch(wl, b)
        ids, _ = OR.route(synth.make_logits(wl, b), wl.k)
        counts, *_ = OP.permute(ids, wl.E)
        fills = [f for r in ora.step_waves(li, counts) for f in r["fills"]]
        y_s, info = layer.forward_streamed(lg, x, li, cache, pool_W, table, side=side, groups=2)
        y_s = y_s.clone()
        torch.cuda.synchronize()
        assert info["fills"] == fills, step
        if step >= min(plan):
            hits_after_resize += info["hits"]
        layer.route_permute(lg)
        layer.expert_ffn(layer.weights(dev_sets[li]), x, wl.T)
        layer.combine(wl.T, False)
        y_r = layer.y[:wl.T].clone()
        torch.cuda.synchronize()
        assert torch.equal(y_s.view(torch.int16), y_r.view(torch.int16)), step
        flush(f"   step {step} layer {li}: waves {info['waves']} hits {info['hits']} "
              f"misses {info['misses']}")
    check_pool("end", False)
    assert hits_after_resize > 0
    cache.close()


def test_fill_groups_argument_checks():
    wl = synth.Workload("stream_args", T=64, H=256, E=16, I=128, k=4, fmt="mxfp4", seed=49)
    d = _pool_set(wl, 4)
    cache = d["cache"]
    counts = torch.zeros(wl.E, dtype=torch.int32)
    counts[:3] = 1
    me, ms, nm, nh, _ = cache.expert_cache_lookup(0, counts)
    assert nm == 3
    for bad in (0, 4, 17):  # 1..min(16, n_miss) only
        with pytest.raises(moe.MoeError):
            cache.expert_cache_fill_groups(0, me, ms, bad)
    with pytest.raises(moe.MoeError):
        cache.expert_cache_wait_group(16)
    cache.expert_cache_fill_groups(0, me, ms, 3)
    for g in range(3):
        cache.expert_cache_wait_group(g)
    torch.cuda.synchronize()
    assert d["table"].cpu().tolist()[:3] == ms.tolist()
    for i, e in enumerate(me.tolist()):
        assert torch.equal(d["pool"][ms[i]].cpu(), d["bank"][e])
    cache.close()


# ---------------------------------------------------------------------------
# hybrid: part of each step's misses computed on the CPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,q,max_fetch,S", [("mxfp4", 0.5, -1, 10), ("nvfp4", 0.3, 2, 12),
                                               ("fp8_b128", 0.0, -1, 8), ("bf16", 0.6, -1, 6)])
def test_hybrid_matches_oracle(fmt, q, max_fetch, S):
    """Hybrid steps: the CPU experts and the fills follow the oracle's hybrid policy (the
    most recently active misses fetched, the rest on the CPU, waves when the GPU share
    exceeds the pool); GPU experts' y_perm rows are bit-identical to the all-resident
    run's, the CPU experts' rows and y match the oracle within tolerance."""
    wl = synth.Workload("hybrid", T=64, H=512, E=24, I=256, k=4, fmt=fmt, seed=52, zipf=1.0,
                        domains=3, batches=6)
    flush(f"[hybrid] {fmt} q={q} max_fetch={max_fetch} S={S}")
    d = _pool_set(wl, S)
    ora = OL.LruSlots(S)
    cpu_pool = moe.CpuPool(4)
    side = torch.cuda.Stream()
    lay = d["layer"]
    ref_layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, d["stride"])
    n_cpu_total = 0
    for b in range(6):
        lg, x = _batch(wl, b)
        y_h, info = lay.forward_hybrid(lg, x, 0, d["cache"], d["pool_W"], d["table"], cpu_pool,
                                       q, max_fetch, side=side, groups=2)
        y_h = y_h.clone()
        yp = lay.y_perm[:wl.T * wl.k].clone()
        torch.cuda.synchronize()
        ids, w = OR.route(synth.make_logits(wl, b), wl.k)
        counts, offsets, sidx, inv = OP.permute(ids, wl.E)
        r = ora.step_hybrid(0, counts, q, max_fetch)
        assert info["cpu"] == r["cpu"] and info["fills"] == r["fills"], b
        assert info["hits"] == r["hits"]
        n_cpu_total += len(r["cpu"])
        # all-resident run: GPU experts' rows bit-identical
        ref_layer.route_permute(lg)
        ref_layer.expert_ffn(ref_layer.weights(d["dev"]), x, wl.T)
        ref_yp = ref_layer.y_perm[:wl.T * wl.k].clone()
        torch.cuda.synchronize()
        cpu_rows = np.zeros(wl.T * wl.k, bool)
        for e in r["cpu"]:
            cpu_rows[offsets[e]:offsets[e + 1]] = True
        g = torch.from_numpy(~cpu_rows).to(DEV)
        assert torch.equal(yp[g].view(torch.int16), ref_yp[g].view(torch.int16)), b
        # the CPU rows and the output against the oracle
        ex = OLY.ExpertSet(wl.fmt, wl.H, wl.I, lambda e: d["bank"][e].numpy())
        ref = OLY.forward(synth.make_logits(wl, b), synth.make_x(wl, b), wl.k, ex)
        if cpu_rows.any():
            assert rel_err(bf16_to_np(yp)[cpu_rows], ref["y_perm"][cpu_rows]) <= TOL
        assert rel_err(bf16_to_np(y_h), ref["y"]) <= TOL
        flush(f"   batch {b}: cpu {len(r['cpu'])} fetched {len(r['fetch'])} hits {r['hits']}")
    assert n_cpu_total > 0 or q == 1.0
    tab = d["table"].cpu().numpy()
    pool_h = d["pool"].cpu()
    for (L, e), s in ora.where.items():
        assert tab[e] == s and torch.equal(pool_h[s], d["bank"][e]), (e, s)
    cpu_pool.close()
    d["cache"].close()


def test_bench_bw_profile():
    """moe_bench_bw: both rates positive, the recommendation follows the threshold, and
    the fetch fraction is h2d / (h2d + cpu)."""
    wl = synth.Workload("bw", T=8, H=2048, E=16, I=512, k=8, fmt="mxfp4", seed=53)
    d = _pool_set(wl, 8)
    pool = moe.CpuPool(4)
    bank_W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, d["bank"].data_ptr(), d["stride"])
    p = moe.moe_bench_bw(pool, bank_W, d["pool"], 8, 2.0)
    assert p["h2d_bytes_per_s"] > 0 and p["cpu_bytes_per_s"] > 0
    assert p["hybrid_recommended"] == int(p["cpu_bytes_per_s"] >= 2.0 * p["h2d_bytes_per_s"])
    assert abs(p["fetch_fraction"] - p["h2d_bytes_per_s"] /
               (p["h2d_bytes_per_s"] + p["cpu_bytes_per_s"])) < 1e-12
    flush(f"   h2d {p['h2d_bytes_per_s'] / 1e9:.1f} GB/s, cpu {p['cpu_bytes_per_s'] / 1e9:.1f} GB/s")
    pool.close()
    d["cache"].close()
