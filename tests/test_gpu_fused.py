"""GPU tests of the single-launch decode layer (moe_layer_decode).

* bit-identical to the separate calls (route_permute + decode FFN + combine)
  in every weight format, and within tolerance of the oracle;
* repeated calls on one workspace (the kernel must leave its counters at 0);
* slot-table indirection;
* replays of a captured graph, checked against eager results every time.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_cases import TOL, Case, bf16_to_np, flush, rel_err
from oracle import layer as OL

pytestmark = pytest.mark.gpu

# The single-launch decode layer these tests cover used in-kernel waits of one
# workgroup on completion counters written by others.  Its first GPU run
# (test_fused_bit_identical_to_separate_calls[bf16]) did not finish; the cause
# was not established, the design was removed, and moe_layer_decode no longer
# exists.  The tests stay, skipped, until a single-launch design without
# inter-workgroup waits replaces it.
pytest.skip("single-launch decode layer removed after a hang on its first run (cause not "
            "established); see the design notes", allow_module_level=True)

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")

DEC = {f: synth.Workload(f"dec_{f}", T=8, H=512, E=64, I=256, k=8, fmt=f, seed=60 + i)
       for i, f in enumerate(synth.FORMATS)}


def _single_launch(layer, logits, x, W, slot=None):
    """The removed single-launch layer call (its entry point no longer exists)."""
    raise NotImplementedError("the single-launch decode layer was removed; see the module note")


def _layer(case):
    wl = case.wl
    return moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, case.stride)


def _separate(layer, case, logits, x):
    W = layer.weights(case.records)
    layer.route_permute(logits)
    layer.expert_ffn(W, x, logits.shape[0], variant="decode")
    layer.combine(logits.shape[0], False)
    torch.cuda.synchronize()
    return {n: getattr(layer, n).clone() for n in ("ids", "w", "counts", "offsets", "sorted_idx",
                                                  "inv_idx", "y")}


def _fused(layer, case, logits, x, slot=None, base=None):
    W = layer.weights(case.records if base is None else base)
    _single_launch(layer, logits, x, W, slot)
    torch.cuda.synchronize()
    return {n: getattr(layer, n).clone() for n in ("ids", "w", "counts", "offsets", "sorted_idx",
                                                  "inv_idx", "y")}


def _same(r1, r2, T, k, E):
    A = T * k
    sl = {"ids": A, "w": A, "counts": E, "offsets": E + 1, "sorted_idx": A, "inv_idx": A}
    for n, m in sl.items():
        assert torch.equal(r1[n][:m], r2[n][:m]), n
    assert torch.equal(r1["y"][:T].view(torch.int16), r2["y"][:T].view(torch.int16)), "y"


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_fused_bit_identical_to_separate_calls(fmt):
    wl = DEC[fmt]
    flush(f"[fused] {fmt}")
    case = Case(wl)
    layer = _layer(case)
    sep = _separate(layer, case, case.logits, case.x)
    fus = _fused(layer, case, case.logits, case.x)
    _same(sep, fus, wl.T, wl.k, wl.E)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    err = rel_err(bf16_to_np(fus["y"][:wl.T]), ref["y"])
    flush(f"   rel err vs oracle {err:.2e}")
    assert err <= TOL


def test_fused_repeated_calls_and_batch_sizes():
    """Counters reset at exit: many calls in a row, varying T, all match."""
    wl = synth.WORKLOADS["decode_mxfp4"]
    flush("[fused-repeat] decode_mxfp4")
    case = Case(wl, gen_device="cuda")
    layer = _layer(case)
    for b, T in enumerate([8, 8, 1, 5, 8, 3, 8, 2]):
        lg = torch.from_numpy(synth.make_logits(wl, 100 + b)).to(DEV)[:T]
        x = torch.from_numpy(synth.make_x(wl, 100 + b).view(np.int16)).to(DEV).view(torch.bfloat16)[:T]
        sep = _separate(layer, case, lg, x)
        fus = _fused(layer, case, lg, x)
        _same(sep, fus, T, wl.k, wl.E)
    # (the removed design also checked that its in-workspace counters were reset)


def test_fused_slot_table():
    wl = DEC["mxfp4"]
    case = Case(wl)
    layer = _layer(case)
    rng = np.random.default_rng(3)
    perm = rng.permutation(wl.E)                      # expert e lives in pool slot perm[e]
    pool = torch.empty_like(case.records)
    pool[torch.from_numpy(perm).to(DEV)] = case.records
    slot = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    direct = _fused(layer, case, case.logits, case.x)
    via = _fused(layer, case, case.logits, case.x, slot=slot, base=pool)
    _same(direct, via, wl.T, wl.k, wl.E)


def test_fused_graph_replays_match_eager():
    wl = synth.WORKLOADS["decode_mxfp4"]
    flush("[fused-graph]")
    case = Case(wl, gen_device="cuda")
    layer = _layer(case)
    W = layer.weights(case.records)
    batches = []
    for b in range(3):
        lg = torch.from_numpy(synth.make_logits(wl, 200 + b)).to(DEV)
        x = torch.from_numpy(synth.make_x(wl, 200 + b).view(np.int16)).to(DEV).view(torch.bfloat16)
        batches.append((lg, x))
    outs = [torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=DEV) for _ in batches]
    eager = []
    for lg, x in batches:
        eager.append(_single_launch(layer, lg, x, W).clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (lg, x), o in zip(batches, outs):
            _single_launch(layer, lg, x, W)
            o.copy_(layer.y[:wl.T])
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"
        # eager work between replays
        _single_launch(layer, batches[0][0], batches[0][1], W)
        torch.cuda.synchronize()
