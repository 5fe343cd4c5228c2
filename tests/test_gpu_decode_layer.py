"""GPU tests of the decode layer (moe_forward_decode).

* routing outputs (ids, weights, counts, offsets, sorted_idx, inv_idx) are
  bit-identical to the separate calls, y is within tolerance of the oracle
  and of the separate-call path, in every weight format;
* every supported K chunking (H and I of 512 .. 2048), both down-projection
  forms (token-major for small T, tile-major + combine above it) and k not a
  multiple of the 4 waves; the MXFP4 one-stream path at every H/128 chunk
  count and with two rounds of units;
* repeated calls with varying batch sizes on one workspace and
  bit-repeatable results;
* slot-table indirection;
* replays of a captured graph, checked against eager results every time,
  also for several layers chained in one graph.
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

DEC = {f: synth.Workload(f"dec_{f}", T=8, H=512, E=64, I=512, k=8, fmt=f, seed=70 + i)
       for i, f in enumerate(synth.FORMATS)}
ROUTING = ("ids", "w", "counts", "offsets", "sorted_idx", "inv_idx")


def _layer(case):
    wl = case.wl
    return moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, case.stride)


def _grab(layer):
    return {n: getattr(layer, n).clone() for n in ROUTING + ("y",)}


def _separate(layer, W, logits, x):
    T = logits.shape[0]
    layer.route_permute(logits)
    layer.expert_ffn(W, x, T, variant="decode")
    layer.combine(T, False)
    torch.cuda.synchronize()
    return _grab(layer)


def _decode(layer, W, logits, x, slot=None):
    layer.forward_decode(logits, x, W, slot)
    torch.cuda.synchronize()
    return _grab(layer)


def _same_routing(r1, r2, T, k, E):
    A = T * k
    sl = {"ids": A, "w": A, "counts": E, "offsets": E + 1, "sorted_idx": A, "inv_idx": A}
    for n, m in sl.items():
        assert torch.equal(r1[n][:m], r2[n][:m]), n


def _same_bits(r1, r2, T):
    assert torch.equal(r1["y"][:T].view(torch.int16), r2["y"][:T].view(torch.int16)), "y"


def _check_case(wl, seed_note="", gen_device="cpu"):
    case = Case(wl, gen_device=gen_device)
    layer = _layer(case)
    assert layer.decode_ws is not None
    W = layer.weights(case.records)
    sep = _separate(layer, W, case.logits, case.x)
    dec = _decode(layer, W, case.logits, case.x)
    _same_routing(sep, dec, wl.T, wl.k, wl.E)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    err = rel_err(bf16_to_np(dec["y"][:wl.T]), ref["y"])
    dif = rel_err(bf16_to_np(dec["y"][:wl.T]), bf16_to_np(sep["y"][:wl.T]))
    flush(f"   {seed_note}rel err vs oracle {err:.2e}, vs separate calls {dif:.2e}")
    assert err <= TOL
    assert dif <= 1e-2
    again = _decode(layer, W, case.logits, case.x)
    _same_bits(dec, again, wl.T)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_decode_layer_matches_oracle_and_separate_calls(fmt):
    flush(f"[decode-layer] {fmt}")
    _check_case(DEC[fmt])


# MXFP4 shapes that take the one-stream path (T*k*(I/128) a multiple of 256,
# E <= 256): every H/128 chunk count, two rounds of units (T = 16, or I = 1024),
# and the full decode workload's expert count
@pytest.mark.parametrize("H,I,T,k,E", [(1024, 512, 8, 8, 64), (1536, 512, 8, 8, 64),
                                       (2048, 512, 16, 8, 256), (512, 1024, 8, 8, 128),
                                       (2048, 512, 8, 8, 256)])
def test_decode_layer_one_stream_shapes(H, I, T, k, E):
    flush(f"[decode-one-stream] H={H} I={I} T={T} k={k} E={E}")
    assert (T * k * (I // 128)) % 256 == 0
    wl = synth.Workload(f"dec_fu_{H}_{I}_{T}", T=T, H=H, E=E, I=I, k=k, fmt="mxfp4",
                        seed=90 + H // 512 + T)
    _check_case(wl)


def test_one_stream_batch_inside_a_larger_workspace():
    """A layer sized for 12 tokens runs an 8-token batch on the one-stream path (its
    partials need more workspace than 12 tokens on the two-kernel path), then 12
    and 3 tokens on the same workspace, each matching the oracle."""
    wl = synth.Workload("dec_ws12", T=12, H=512, E=64, I=512, k=8, fmt="mxfp4", seed=97)
    flush("[decode-ws] T_max=12")
    case = Case(wl)
    layer = _layer(case)
    W = layer.weights(case.records)
    ex = case.oracle_experts()
    for T in (8, 12, 3, 8):
        lg = case.logits[:T].contiguous()
        x = case.x[:T].contiguous()
        d = _decode(layer, W, lg, x)
        ref = OL.forward(case.logits_np[:T], case.x_np[:T], wl.k, ex)
        assert rel_err(bf16_to_np(d["y"][:T]), ref["y"]) <= TOL, T


@pytest.mark.parametrize("H,I,T,k", [(1024, 1536, 6, 4), (2048, 2048, 6, 4), (1536, 1024, 6, 4),
                                     (512, 512, 16, 13), (512, 1024, 32, 4), (2048, 512, 24, 8)])
def test_decode_layer_chunkings(H, I, T, k):
    """Every K chunking; T <= 16 takes the token-major down, larger T the tile-major one."""
    wl = synth.Workload(f"dec_chunk_{H}_{I}", T=T, H=H, E=32, I=I, k=k, fmt="mxfp4", seed=H + I + T)
    flush(f"[decode-layer] H={H} I={I} T={T} k={k}")
    _check_case(wl, f"H={H} I={I} T={T} k={k}: ")


@pytest.mark.parametrize("fmt,T,k", [("nvfp4", 4, 16), ("mxfp4", 4, 16), ("bf16", 20, 8),
                                      ("fp8_b128", 20, 8)])
def test_decode_layer_largest_expert_count(fmt, T, k):
    """E = 1024: the token-major kernels' sixteen logits per lane (T <= 16, k = 16)
    and the tile-major tile table over 1024 experts (T = 20)."""
    wl = synth.Workload(f"dec_e1024_{fmt}", T=T, H=512, E=1024, I=512, k=k, fmt=fmt, seed=T + k + 400)
    flush(f"[decode-layer] E=1024 {fmt} T={T} k={k}")
    _check_case(wl, f"E=1024 T={T} k={k}: ", gen_device="cuda")


def test_decode_layer_full_workload_and_varying_batch():
    wl = synth.WORKLOADS["decode_mxfp4"]
    flush("[decode-layer] decode_mxfp4, varying T")
    case = Case(wl, gen_device="cuda")
    layer = _layer(case)
    W = layer.weights(case.records)
    ex = case.oracle_experts()
    ref = OL.forward(case.logits_np, case.x_np, wl.k, ex)
    dec = _decode(layer, W, case.logits, case.x)
    err = rel_err(bf16_to_np(dec["y"][:wl.T]), ref["y"])
    flush(f"   full batch rel err vs oracle {err:.2e}")
    assert err <= TOL
    for b, T in enumerate([8, 1, 5, 8, 3, 2]):
        lg_np = synth.make_logits(wl, 100 + b)[:T]
        x_np = synth.make_x(wl, 100 + b)[:T]
        lg = torch.from_numpy(np.ascontiguousarray(lg_np)).to(DEV)
        x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV).view(torch.bfloat16)
        sep = _separate(layer, W, lg, x)
        d1 = _decode(layer, W, lg, x)
        d2 = _decode(layer, W, lg, x)
        _same_routing(sep, d1, T, wl.k, wl.E)
        _same_bits(d1, d2, T)
        r = OL.forward(lg_np, x_np, wl.k, ex)
        err = rel_err(bf16_to_np(d1["y"][:T]), r["y"])
        assert err <= TOL, (T, err)


def test_decode_layer_routing_ties():
    """Logits with many exact ties: the token-major kernels route each token
    themselves and must keep the lowest-index tie-break."""
    wl = synth.Workload("dec_ties", T=8, H=512, E=256, I=512, k=8, fmt="mxfp4", seed=77)
    flush("[decode-layer] ties")
    case = Case(wl)
    rng = np.random.default_rng(9)
    lg_np = (rng.integers(-2, 3, size=(wl.T, wl.E)) * 0.5).astype(np.float32)
    lg = torch.from_numpy(lg_np).to(DEV)
    layer = _layer(case)
    W = layer.weights(case.records)
    sep = _separate(layer, W, lg, case.x)
    dec = _decode(layer, W, lg, case.x)
    _same_routing(sep, dec, wl.T, wl.k, wl.E)
    ref = OL.forward(lg_np, case.x_np, wl.k, case.oracle_experts())
    assert np.array_equal(dec["ids"][:wl.T * wl.k].cpu().numpy().reshape(wl.T, wl.k), ref["ids"])
    assert rel_err(bf16_to_np(dec["y"][:wl.T]), ref["y"]) <= TOL


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])   # mxfp4: the one-stream path
def test_decode_layer_slot_table(fmt):
    wl = DEC[fmt]
    flush(f"[decode-layer] slot table {fmt}")
    case = Case(wl)
    layer = _layer(case)
    rng = np.random.default_rng(5)
    perm = rng.permutation(wl.E)                    # expert e lives in pool slot perm[e]
    pool = torch.empty_like(case.records)
    pool[torch.from_numpy(perm).to(DEV)] = case.records
    slot = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    direct = _decode(layer, layer.weights(case.records), case.logits, case.x)
    via = _decode(layer, layer.weights(pool), case.logits, case.x, slot=slot)
    _same_routing(direct, via, wl.T, wl.k, wl.E)
    _same_bits(direct, via, wl.T)


@pytest.mark.parametrize("T,E", [(8, 256), (16, 256), (16, 16)])
def test_decode_layer_every_token_same_experts(T, E):
    """Every token routes to the same k experts (identical logits rows): on the
    one-stream path each unit then serves all T tokens (the most rows one unit
    takes) and only k * I/128 units have work."""
    wl = synth.Workload(f"dec_same_{T}_{E}", T=T, H=2048, E=E, I=512, k=8, fmt="mxfp4",
                        seed=300 + T + E)
    flush(f"[decode-layer] same experts T={T} E={E}")
    case = Case(wl, gen_device="cuda")
    row = np.random.default_rng(T + E).standard_normal(wl.E).astype(np.float32)
    lg_np = np.repeat(row[None, :], wl.T, axis=0)
    lg = torch.from_numpy(lg_np).to(DEV)
    layer = _layer(case)
    W = layer.weights(case.records)
    sep = _separate(layer, W, lg, case.x)
    dec = _decode(layer, W, lg, case.x)
    _same_routing(sep, dec, wl.T, wl.k, wl.E)
    ref = OL.forward(lg_np, case.x_np, wl.k, case.oracle_experts())
    err = rel_err(bf16_to_np(dec["y"][:wl.T]), ref["y"])
    flush(f"   rel err vs oracle {err:.2e}")
    assert err <= TOL
    assert rel_err(bf16_to_np(dec["y"][:wl.T]), bf16_to_np(sep["y"][:wl.T])) <= 1e-2


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


def test_chained_layers_in_one_graph():
    """Several decode layers chained (each layer's y is the next one's x), captured
    once: every replay reproduces the eager chain bit for bit, and each layer's
    output matches the oracle given the bf16 input that layer actually received."""
    wl = DEC["mxfp4"]
    L = 4
    flush("[decode-chain-graph] L=%d" % L)
    layers, Ws, logits = [], [], []
    for li in range(L):
        recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, layer=li,
                                         device="cuda").to(DEV)
        lay = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, recs.shape[1])
        layers.append((lay, recs))
        Ws.append(lay.weights(recs))
        logits.append(torch.from_numpy(synth.make_logits(wl, 300 + li)).to(DEV))
    x0 = torch.from_numpy(synth.make_x(wl, 300).view(np.int16)).to(DEV).view(torch.bfloat16)

    def chain():
        x = x0
        for (lay, _), W, lg in zip(layers, Ws, logits):
            x = lay.forward_decode(lg, x, W)
        return x

    ins, outs = [x0.clone()], []
    x = x0
    for (lay, _), W, lg in zip(layers, Ws, logits):
        x = lay.forward_decode(lg, x, W)
        torch.cuda.synchronize()
        outs.append(x.clone())
        ins.append(x.clone())
    eager = outs[-1]

    # per layer against the oracle, on the input that layer saw
    for li, (lay, recs) in enumerate(layers):
        rec_np = recs.cpu().numpy()
        ex = OL.ExpertSet(wl.fmt, wl.H, wl.I, lambda e, r=rec_np: r[e])
        xin = ins[li].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = OL.forward(logits[li].cpu().numpy(), xin, wl.k, ex)
        assert rel_err(bf16_to_np(outs[li]), ref["y"]) <= TOL, f"layer {li}"

    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out.copy_(chain())
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        layers[1][0].forward_decode(logits[0], x0, Ws[1])  # eager work between replays
        torch.cuda.synchronize()


def test_decode_layer_limits():
    assert moe.moe_forward_decode_supported(2048, 512, 8, 8)
    assert moe.moe_forward_decode_supported(512, 2048, 64, 4)
    assert not moe.moe_forward_decode_supported(2048, 512, 65, 1)
    assert not moe.moe_forward_decode_supported(2048, 256, 8, 8)
    assert not moe.moe_forward_decode_supported(7168, 2048, 8, 8)
