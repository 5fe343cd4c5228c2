"""GPU tests of the two-launch decode layer (moe_forward_decode).

* bit-identical to the separate calls (route_permute + decode FFN + combine)
  in every weight format, and within tolerance of the oracle;
* repeated calls with varying batch sizes on one workspace;
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

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")

DEC = {f: synth.Workload(f"dec_{f}", T=8, H=512, E=64, I=256, k=8, fmt=f, seed=70 + i)
       for i, f in enumerate(synth.FORMATS)}
OUTS = ("ids", "w", "counts", "offsets", "sorted_idx", "inv_idx", "y")


def _layer(case):
    wl = case.wl
    return moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, case.stride)


def _separate(layer, W, logits, x):
    T = logits.shape[0]
    layer.route_permute(logits)
    layer.expert_ffn(W, x, T, variant="decode")
    layer.combine(T, False)
    torch.cuda.synchronize()
    return {n: getattr(layer, n).clone() for n in OUTS}


def _decode(layer, W, logits, x, slot=None):
    layer.forward_decode(logits, x, W, slot)
    torch.cuda.synchronize()
    return {n: getattr(layer, n).clone() for n in OUTS}


def _same(r1, r2, T, k, E):
    A = T * k
    sl = {"ids": A, "w": A, "counts": E, "offsets": E + 1, "sorted_idx": A, "inv_idx": A}
    for n, m in sl.items():
        assert torch.equal(r1[n][:m], r2[n][:m]), n
    assert torch.equal(r1["y"][:T].view(torch.int16), r2["y"][:T].view(torch.int16)), "y"


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_decode_layer_bit_identical_to_separate_calls(fmt):
    wl = DEC[fmt]
    flush(f"[decode-layer] {fmt}")
    case = Case(wl)
    layer = _layer(case)
    assert layer.decode_ws is not None
    W = layer.weights(case.records)
    sep = _separate(layer, W, case.logits, case.x)
    dec = _decode(layer, W, case.logits, case.x)
    _same(sep, dec, wl.T, wl.k, wl.E)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    err = rel_err(bf16_to_np(dec["y"][:wl.T]), ref["y"])
    flush(f"   rel err vs oracle {err:.2e}")
    assert err <= TOL


def test_decode_layer_full_workload_and_varying_batch():
    wl = synth.WORKLOADS["decode_mxfp4"]
    flush("[decode-layer] decode_mxfp4, varying T")
    case = Case(wl, gen_device="cuda")
    layer = _layer(case)
    W = layer.weights(case.records)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    dec = _decode(layer, W, case.logits, case.x)
    err = rel_err(bf16_to_np(dec["y"][:wl.T]), ref["y"])
    flush(f"   full batch rel err vs oracle {err:.2e}")
    assert err <= TOL
    for b, T in enumerate([8, 1, 5, 8, 3, 2]):
        lg = torch.from_numpy(synth.make_logits(wl, 100 + b)).to(DEV)[:T].contiguous()
        x = torch.from_numpy(synth.make_x(wl, 100 + b).view(np.int16)).to(DEV).view(torch.bfloat16)
        x = x[:T].contiguous()
        _same(_separate(layer, W, lg, x), _decode(layer, W, lg, x), T, wl.k, wl.E)


def test_decode_layer_slot_table():
    wl = DEC["nvfp4"]
    case = Case(wl)
    layer = _layer(case)
    rng = np.random.default_rng(5)
    perm = rng.permutation(wl.E)                    # expert e lives in pool slot perm[e]
    pool = torch.empty_like(case.records)
    pool[torch.from_numpy(perm).to(DEV)] = case.records
    slot = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    direct = _decode(layer, layer.weights(case.records), case.logits, case.x)
    via = _decode(layer, layer.weights(pool), case.logits, case.x, slot=slot)
    _same(direct, via, wl.T, wl.k, wl.E)


def test_decode_layer_graph_replays_match_eager():
    wl = synth.WORKLOADS["decode_mxfp4"]
    flush("[decode-layer-graph]")
    case = Case(wl, gen_device="cuda")
    layer = _layer(case)
    W = layer.weights(case.records)
    batches = []
    for b in range(3):
        lg = torch.from_numpy(synth.make_logits(wl, 200 + b)).to(DEV)
        x = torch.from_numpy(synth.make_x(wl, 200 + b).view(np.int16)).to(DEV).view(torch.bfloat16)
        batches.append((lg, x))
    outs = [torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=DEV) for _ in batches]
    eager = [layer.forward_decode(lg, x, W).clone() for lg, x in batches]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (lg, x), o in zip(batches, outs):
            layer.forward_decode(lg, x, W)
            o.copy_(layer.y[:wl.T])
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"
        layer.forward_decode(batches[1][0], batches[1][1], W)  # eager work between replays
        torch.cuda.synchronize()


def test_decode_layer_limits():
    assert moe.moe_forward_decode_supported(2048, 512, 8, 8)
    assert not moe.moe_forward_decode_supported(2048, 512, 65, 1)
    assert not moe.moe_forward_decode_supported(7168, 2048, 8, 8)
