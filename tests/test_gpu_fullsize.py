"""GPU parity at full workload size, in the launch configuration the benchmark times.

* prefill_nvfp4 (T=4096, E=256, Zipf-skewed): every output element of y and of
  y_perm against the full oracle forward;
* large_prefill_mxfp4 (T=16384, H=7168, E=256, I=2048, + shared expert) and the
  FP8 pool workload (T=2048, H=4096, E=512, I=1024): stratified rows — every
  touched expert is checked on the first, middle and last row of each 128-row
  block of its segment (so every m-tile of every expert, including the ragged
  tails and the hottest segments, is compared), plus the layer output y of a
  spread of tokens; routing, counts, offsets and both permutations bit-exact for
  the whole batch.  The shared expert's output is checked on rows spanning its
  row tiles.
* the FP8 pool workload through the expert cache (160 slots), streamed fills:
  y of batch 0 and batch 1 against the oracle on the same stratified tokens and
  bit-identical to the all-resident run.

The oracle works one expert at a time (decode its record, evaluate the FFN for
the chosen rows), in a thread pool: numpy releases the interpreter lock inside
the decode and the products, and one decoded large expert is 350 MB of float64.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from gpu_cases import TOL, Case, bf16_to_np, flush, rel_err
from oracle import combine as OC
from oracle import ffn as OFF
from oracle import formats as OF
from oracle import layer as OL
from oracle import permute as OP
from oracle import route as OR

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def stratified_rows(offsets, E: int, block: int = 128):
    """(expert, permuted rows) for every touched expert: the first, middle and last row
    of each `block`-row piece of its segment."""
    plan = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        n = hi - lo
        if n <= 0:
            continue
        rel = set()
        for m in range(0, n, block):
            rel.update({m, min(n - 1, m + block // 2), min(n - 1, m + block - 1)})
        plan.append((e, sorted(lo + r for r in rel)))
    return plan


def oracle_by_expert(fmt, H, I, rec_of, x_bits, k, ids, w, sorted_idx, plan, tokens,
                     shared_rec=None, shared_I=0, shared_rows=()):
    """Oracle values, one decoded expert at a time:
      rows   {p: FFN_e(x[token(p)])} for the planned permuted rows,
      y      the layer output of `tokens` (combine of their k expert outputs, + shared),
      shared {t: shared FFN(x_t)} for shared_rows."""
    x = OF.bf16_value(np.asarray(x_bits))
    tokens = np.asarray(tokens, dtype=np.int64)
    sidx = np.asarray(sorted_idx)
    want = {}                                     # expert -> [(i, j)] of the token sample
    for i, t in enumerate(tokens):
        for j in range(k):
            want.setdefault(int(ids[t, j]), []).append((i, j))
    rows_of = dict(plan)
    experts = sorted(set(rows_of) | set(want))

    def work(e):
        Wg, Wu, Wd = OF.decode_record(rec_of(e), fmt, H, I)
        rows = rows_of.get(e, [])
        out_rows = {}
        if rows:
            vals = OFF.swiglu(x[sidx[rows] // k], Wg, Wu, Wd)
            out_rows = dict(zip(rows, vals))
        toks = want.get(e, [])
        out_tok = {}
        if toks:
            vals = OFF.swiglu(x[tokens[[i for i, _ in toks]]], Wg, Wu, Wd)
            out_tok = dict(zip(toks, vals))
        return out_rows, out_tok

    rows_ref, contrib = {}, {}
    done = 0
    with ThreadPoolExecutor(THREADS) as ex:
        for r, c in ex.map(work, experts):
            rows_ref.update(r)
            contrib.update(c)
            done += 1
            if done % 32 == 0:
                flush(f"   oracle: {done}/{len(experts)} experts")
    shared_ref = {}
    ys = None
    if shared_rec is not None:
        Wg, Wu, Wd = OF.decode_record(shared_rec, "bf16", H, shared_I)
        sel = sorted(set(int(t) for t in shared_rows) | set(int(t) for t in tokens))
        vals = OFF.swiglu(x[sel], Wg, Wu, Wd)
        shared_ref = dict(zip(sel, vals))
        ys = np.stack([shared_ref[int(t)] for t in tokens])
    n = len(tokens)
    mini = np.stack([contrib[(i, j)] for i in range(n) for j in range(k)])
    y = OC.combine(mini, np.arange(n * k), w[tokens], n, k, ys)
    return rows_ref, y, shared_ref


def sample_tokens(T: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.choice(T, n, replace=False)]))


def _run_layer(case: Case):
    wl = case.wl
    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, case.stride, shared_I=wl.shared_I,
                         shared_stride=case.shared.shape[1] if case.shared is not None else 0)
    W = layer.weights(case.records)
    Ws = None
    if case.shared is not None:
        Ws = moe.experts("bf16", 1, wl.H, wl.shared_I, case.shared, case.shared.shape[1])
    y = layer.forward(case.logits, case.x, W, Ws)
    torch.cuda.synchronize()
    return layer, y


def _check_routing(layer, wl, logits_np):
    A = wl.T * wl.k
    ref_ids, ref_w = OR.route(logits_np, wl.k)
    counts, offsets, sidx, inv = OP.permute(ref_ids, wl.E)
    assert np.array_equal(layer.ids[:A].cpu().numpy().reshape(wl.T, wl.k), ref_ids)
    assert np.max(np.abs(layer.w[:A].cpu().numpy().reshape(wl.T, wl.k) - ref_w)) <= 1e-5
    for name, buf, ref in (("counts", layer.counts[:wl.E], counts),
                           ("offsets", layer.offsets[:wl.E + 1], offsets),
                           ("sorted_idx", layer.sorted_idx[:A], sidx),
                           ("inv_idx", layer.inv_idx[:A], inv)):
        assert np.array_equal(buf.cpu().numpy(), ref), name
    return ref_ids, ref_w, counts, offsets, sidx


def test_prefill_nvfp4_every_element():
    """T=4096 NVFP4 prefill: all of y and y_perm against the full oracle forward."""
    wl = synth.WORKLOADS["prefill_nvfp4"]
    flush(f"[full] {wl.name}: every element")
    case = Case(wl, gen_device="cuda")
    layer, y = _run_layer(case)
    _check_routing(layer, wl, case.logits_np)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    e_perm = rel_err(bf16_to_np(layer.y_perm[:wl.T * wl.k]), ref["y_perm"])
    e_y = rel_err(bf16_to_np(y), ref["y"])
    flush(f"   y_perm rel err {e_perm:.2e}, y rel err {e_y:.2e} "
          f"({wl.T} tokens, {int((ref['counts'] > 0).sum())} experts)")
    assert e_perm <= TOL and e_y <= TOL


def test_large_prefill_stratified():
    """T=16384, H=7168, I=2048 MXFP4 + bf16 shared expert: every 128-row block of every
    touched expert, a spread of tokens' y, and the shared expert's rows."""
    wl = synth.WORKLOADS["large_prefill_mxfp4"]
    flush(f"[full] {wl.name}: stratified rows")
    case = Case(wl, gen_device="cuda")
    layer, y = _run_layer(case)
    ids, w, counts, offsets, sidx = _check_routing(layer, wl, case.logits_np)
    plan = stratified_rows(offsets, wl.E)
    tokens = sample_tokens(wl.T, 28, 5)
    shared_rows = sorted({r for m in range(0, wl.T, 256) for r in (m, m + 127, m + 255)}
                         | {wl.T - 1})
    flush(f"   {len(plan)} experts, {sum(len(r) for _, r in plan)} rows, "
          f"{len(tokens)} tokens, {len(shared_rows)} shared rows")
    rows_ref, y_ref, sh_ref = oracle_by_expert(
        wl.fmt, wl.H, wl.I, case.rec_host, case.x_np, wl.k, ids, w, sidx, plan, tokens,
        shared_rec=case.shared[0].cpu().numpy(), shared_I=wl.shared_I, shared_rows=shared_rows)
    rows = sorted(rows_ref)
    got = bf16_to_np(layer.y_perm[torch.tensor(rows, device=DEV)])
    e_rows = rel_err(got, np.stack([rows_ref[p] for p in rows]))
    e_y = rel_err(bf16_to_np(y[torch.tensor(tokens, device=DEV)]), y_ref)
    srows = sorted(sh_ref)
    e_sh = rel_err(bf16_to_np(layer.y_shared[torch.tensor(srows, device=DEV)]),
                   np.stack([sh_ref[t] for t in srows]))
    flush(f"   y_perm rows rel err {e_rows:.2e}, y rel err {e_y:.2e}, shared {e_sh:.2e}")
    assert e_rows <= TOL and e_y <= TOL and e_sh <= TOL


def _fp8_oracle(wl, logits_np, x_np, rec_of):
    ids, w = OR.route(logits_np, wl.k)
    counts, offsets, sidx, inv = OP.permute(ids, wl.E)
    plan = stratified_rows(offsets, wl.E)
    tokens = sample_tokens(wl.T, 24, 4)
    rows_ref, y_ref, _ = oracle_by_expert(wl.fmt, wl.H, wl.I, rec_of, x_np, wl.k, ids, w, sidx,
                                          plan, tokens)
    return rows_ref, y_ref, tokens, len(plan)


def test_fp8_pool_resident_and_streamed_stratified():
    """FP8 pool workload (T=2048, H=4096, E=512, I=1024), batches 0 and 1: all experts
    resident, and through the 160-slot pool with streamed fills; stratified oracle rows and
    tokens; the pool path bit-identical to the resident one."""
    wl = synth.WORKLOADS["fp8_lru_pool"]
    flush(f"[full] {wl.name}: resident and streamed, stratified rows")
    stride = synth.record_layout(wl.fmt, wl.H, wl.I)["stride"]
    recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, device=DEV)
    bank = torch.empty((wl.E, stride), dtype=torch.uint8, pin_memory=True)
    bank.copy_(recs.cpu())
    pool = torch.empty((wl.pool_slots, stride), dtype=torch.uint8, device=DEV)
    table = torch.full((wl.E,), -1, dtype=torch.int32, device=DEV)
    cache = moe.ExpertCache(1, wl.E, wl.pool_slots, stride, pool, bank, table)
    res = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride)
    stm = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride)
    pool_W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, pool, stride)
    side = torch.cuda.Stream()
    host = {}

    def rec_of(e):
        if e not in host:
            host[e] = bank[e].numpy()
        return host[e]

    for b in range(2):
        lg_np, x_np = synth.make_logits(wl, b), synth.make_x(wl, b)
        lg = torch.from_numpy(lg_np).to(DEV)
        x = torch.from_numpy(x_np.view(np.int16)).to(DEV).view(torch.bfloat16)
        y_r = res.forward(lg, x, res.weights(recs)).clone()
        torch.cuda.synchronize()
        _check_routing(res, wl, lg_np)
        y_s, info = stm.forward_streamed(lg, x, 0, cache, pool_W, table, side=side, groups=8)
        torch.cuda.synchronize()
        assert torch.equal(y_s.view(torch.int16), y_r.view(torch.int16)), f"batch {b}"
        rows_ref, y_ref, tokens, n_e = _fp8_oracle(wl, lg_np, x_np, rec_of)
        rows = sorted(rows_ref)
        e_rows = rel_err(bf16_to_np(res.y_perm[torch.tensor(rows, device=DEV)]),
                         np.stack([rows_ref[p] for p in rows]))
        tk = torch.tensor(tokens, device=DEV)
        e_y = rel_err(bf16_to_np(y_r[tk]), y_ref)
        e_ys = rel_err(bf16_to_np(y_s[tk]), y_ref)
        flush(f"   batch {b}: {n_e} experts, misses {info['misses']} hits {info['hits']}; "
              f"y_perm rows rel err {e_rows:.2e}, y rel err {e_y:.2e}, streamed y {e_ys:.2e}")
        assert e_rows <= TOL and e_y <= TOL and e_ys <= TOL
    cache.close()
