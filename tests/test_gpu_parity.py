"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar: routing ids, counts, offsets, sorted / inverse indices bit-exact; routing
weights within 1e-5; bf16 outputs within 2e-2 * max|oracle| (decoded weights
are exact, so the error comes only from bf16 rounding of h, y_perm and y and
fp32 summation order).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_cases import TOL, Case, bf16_to_np, flush, rel_err
from oracle import combine as OC
from oracle import formats as OF
from oracle import layer as OL
from oracle import permute as OP
from oracle import route as OR

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")


def _i32(n):
    return torch.empty(max(n, 1), dtype=torch.int32, device=DEV)


# --------------------------------------------------------------------------
# weight decoders: every code on the device equals the oracle's value
# --------------------------------------------------------------------------
def _all_code_record(fmt, H, I, rng):
    lay = synth.record_layout(fmt, H, I)
    rec = np.zeros(lay["stride"], np.uint8)
    for name, (off, n) in lay["sections"].items():
        if name in ("w13", "w2"):
            if fmt == "fp8_b128":
                rec[off:off + n] = np.arange(n) % 256            # every E4M3 code incl. NaN
            elif fmt == "bf16":
                v = (rng.standard_normal(n // 2) * 0.02).astype(np.float32)
                rec[off:off + n] = torch.from_numpy(v).to(torch.bfloat16).view(torch.uint8).numpy()
            else:
                rec[off:off + n] = rng.integers(0, 256, n)       # every E2M1 pair
        elif name in ("w13s", "w2s"):
            if fmt == "mxfp4":
                rec[off:off + n] = rng.integers(20, 231, n)      # 2^-107 .. 2^103
            elif fmt == "nvfp4":
                rec[off:off + n] = np.arange(n) % 0x7F           # every finite E4M3 >= 0
            else:
                rec[off:off + n] = np.frombuffer(
                    np.exp2(rng.integers(-12, 4, n // 4)).astype(np.float32).tobytes(), np.uint8)
        elif name == "ts":
            rec[off:off + n] = np.frombuffer(np.array([0.37, 1.5e-3, 2.0], np.float32).tobytes(),
                                             np.uint8)
    return rec


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_device_decode_every_code(fmt):
    H, I = 256, 128
    flush(f"[decode] fmt={fmt}")
    rng = np.random.default_rng(1)
    rec = _all_code_record(fmt, H, I, rng)
    base = torch.from_numpy(rec).to(DEV)
    W = moe.experts(fmt, 1, H, I, base, len(rec))
    w13 = torch.empty((2 * I, H), dtype=torch.float32, device=DEV)
    w2 = torch.empty((H, I), dtype=torch.float32, device=DEV)
    moe.moe_dequant_expert(W, 0, w13, w2)
    torch.cuda.synchronize()
    g, u, d = OF.decode_record(rec, fmt, H, I)
    ref13 = np.concatenate([g, u]).astype(np.float32)
    for got, ref in ((w13.cpu().numpy(), ref13), (w2.cpu().numpy(), d.astype(np.float32))):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan]), np.argwhere(got != ref)[:5]


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------
def _route_gpu(lg_np, k, renorm=True):
    T, E = lg_np.shape
    lg = torch.from_numpy(np.ascontiguousarray(lg_np)).to(DEV)
    ids = _i32(T * k)
    w = torch.empty(max(T * k, 1), dtype=torch.float32, device=DEV)
    moe.moe_route(lg, k, ids, w, renorm)
    torch.cuda.synchronize()
    return ids[:T * k].cpu().numpy().reshape(T, k), w[:T * k].cpu().numpy().reshape(T, k)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_route_full_size(name):
    wl = synth.WORKLOADS[name]
    flush(f"[route] {name} T={wl.T} E={wl.E} k={wl.k}")
    lg = synth.make_logits(wl)
    ids, w = _route_gpu(lg, wl.k)
    oid, ow = OR.route(lg, wl.k)
    assert np.array_equal(ids, oid)
    assert np.max(np.abs(w - ow)) <= 1e-5


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 3), (33, 64, 16), (7, 1024, 16), (130, 1000, 5),
                                   (64, 65, 2), (9, 129, 8), (3, 512, 1)])
def test_route_edge_shapes_and_ties(T, E, k):
    flush(f"[route-edge] T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 1000 + E)
    lg = (rng.integers(-3, 4, size=(T, E)) * 0.25).astype(np.float32)   # many exact ties
    lg[0, :min(E, 4)] = np.array([0.0, -0.0, 0.0, -0.0], np.float32)[:min(E, 4)]
    for renorm in (True, False):
        ids, w = _route_gpu(lg, k, renorm)
        oid, ow = OR.route(lg, k, renorm)
        assert np.array_equal(ids, oid)
        assert np.max(np.abs(w - ow)) <= 1e-5


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------
def _permute_gpu(ids_np, E):
    T, k = ids_np.shape
    A = T * k
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(DEV)
    counts, offsets, sidx, inv = _i32(E), _i32(E + 1), _i32(A), _i32(A)
    ws = torch.empty(moe.moe_permute_workspace(T, k, E), dtype=torch.uint8, device=DEV)
    moe.moe_permute(ids, T, k, E, counts, offsets, sidx, inv, ws)
    torch.cuda.synchronize()
    return (counts.cpu().numpy()[:E], offsets.cpu().numpy()[:E + 1], sidx.cpu().numpy()[:A],
            inv.cpu().numpy()[:A])


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_permute_full_size(name):
    wl = synth.WORKLOADS[name]
    flush(f"[permute] {name}")
    oid, _ = OR.route(synth.make_logits(wl), wl.k)
    got = _permute_gpu(oid, wl.E)
    ref = OP.permute(oid, wl.E)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (128, 8, 8), (129, 8, 8), (1000, 2, 1), (1025, 1, 1),
                                   (3000, 1024, 16), (777, 37, 5), (4096, 300, 1)])
def test_permute_edge_shapes(T, E, k):
    flush(f"[permute-edge] T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E + k)
    p = rng.zipf(1.3, size=E * 4)
    ids = np.stack([rng.permutation(E)[:k] if rng.random() < 0.5 else
                    np.argsort(-(rng.random(E) + (p[:E] > 2)))[:k] for _ in range(T)])
    got = _permute_gpu(ids.astype(np.int32), E)
    for g, r in zip(got, OP.permute(ids, E)):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (8, 256, 8), (64, 8, 2), (64, 1024, 4), (32, 512, 8),
                                   (17, 100, 16), (65, 256, 2), (100, 64, 8)])
def test_route_permute_fused(T, E, k):
    """moe_route_permute (one workgroup when T <= 64 and T*k <= 256) == oracle."""
    flush(f"[route-permute] T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, ::3] = np.round(lg[:, ::3])                      # exact ties
    lg_d = torch.from_numpy(lg).to(DEV)
    A = T * k
    ids, w = _i32(A), torch.empty(A, dtype=torch.float32, device=DEV)
    counts, offsets, sidx, inv = _i32(E), _i32(E + 1), _i32(A), _i32(A)
    ws = torch.empty(max(moe.moe_permute_workspace(T, k, E), 256), dtype=torch.uint8, device=DEV)
    moe.moe_route_permute(lg_d, k, ids, w, counts, offsets, sidx, inv, ws)
    torch.cuda.synchronize()
    oid, ow = OR.route(lg, k)
    assert np.array_equal(ids.cpu().numpy().reshape(T, k), oid)
    assert np.max(np.abs(w.cpu().numpy().reshape(T, k) - ow)) <= 1e-5
    for g, r in zip((counts[:E], offsets[:E + 1], sidx[:A], inv[:A]), OP.permute(oid, E)):
        assert np.array_equal(g.cpu().numpy(), r)


def test_permute_all_to_one_expert():
    ids = np.zeros((5000, 1), np.int32)
    got = _permute_gpu(ids, 3)
    for g, r in zip(got, OP.permute(ids, 3)):
        assert np.array_equal(g, r)


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,H,shared", [(1, 1, 8, False), (37, 8, 2048, True), (300, 2, 256, False)])
def test_combine(T, k, H, shared):
    flush(f"[combine] T={T} k={k} H={H}")
    rng = np.random.default_rng(T)
    E = max(k, 9)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, _, inv = OP.permute(ids, E)
    yp = torch.randn(T * k, H, device=DEV).to(torch.bfloat16)
    w = torch.rand(T * k, device=DEV)
    ys = torch.randn(T, H, device=DEV).to(torch.bfloat16) if shared else None
    y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(yp, torch.from_numpy(inv).to(DEV), w, T, k, H, ys, y)
    torch.cuda.synchronize()
    ref = OC.combine(bf16_to_np(yp), inv, w.cpu().numpy().astype(np.float64), T, k,
                     bf16_to_np(ys) if shared else None)
    got = bf16_to_np(y)
    # one bf16 rounding of an fp32 sum
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
def _run_layer(case: Case, variant="auto", T=None):
    wl = case.wl
    T = wl.T if T is None else T
    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, T, case.stride, shared_I=wl.shared_I,
                         shared_stride=case.shared.shape[1] if case.shared is not None else 0)
    W = layer.weights(case.records)
    Ws = None
    if case.shared is not None:
        Ws = moe.experts("bf16", 1, wl.H, wl.shared_I, case.shared, case.shared.shape[1])
    y = layer.forward(case.logits[:T], case.x[:T], W, Ws, variant=variant)
    torch.cuda.synchronize()
    return layer, y


SMALL = {
    # several m-tiles, several column blocks and a ragged tail in every format
    f: synth.Workload(f"small_{f}", T=150, H=384, E=6, I=256, k=2, fmt=f, seed=40 + i, zipf=0.7)
    for i, f in enumerate(synth.FORMATS)
}


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("variant", ["decode", "prefill"])
def test_layer_small_all_formats(fmt, variant):
    wl = SMALL[fmt]
    flush(f"[layer-small] fmt={fmt} variant={variant}")
    case = Case(wl)
    layer, y = _run_layer(case, variant)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    assert np.array_equal(layer.ids[:wl.T * wl.k].cpu().numpy().reshape(wl.T, wl.k), ref["ids"])
    assert np.array_equal(layer.sorted_idx[:wl.T * wl.k].cpu().numpy(), ref["sorted_idx"])
    yp = bf16_to_np(layer.y_perm[:wl.T * wl.k])
    assert rel_err(yp, ref["y_perm"]) <= TOL
    err = rel_err(bf16_to_np(y), ref["y"])
    flush(f"   rel err {err:.2e}")
    assert err <= TOL


# Shapes the pipelined prefill GEMMs take (H and I multiples of 256; MXFP4 and
# FP8 through the block-scaled kernels, BF16 and NVFP4 through the bf16 ones):
# 64-row tiles with ragged tails, several column blocks, every format; 1200
# tokens over 16 experts give ~48 tiles, several super-tile groups of 8;
# H = I = 256 is the shortest K loop (two chunks); 600 experts with ~2 rows
# each make the grid's tile bound far looser than the tiles with rows.
PIPE = [(f, T, E, H, I) for f in synth.FORMATS
        for (T, E, H, I) in ((300, 4, 512, 768), (170, 12, 512, 768), (1200, 16, 512, 768),
                             (200, 4, 256, 256), (600, 600, 256, 256))]


@pytest.mark.parametrize("fmt,T,E,H,I", PIPE)
def test_layer_prefill_pipe(fmt, T, E, H, I):
    wl = synth.Workload(f"pipe_{fmt}_{T}", T=T, H=H, E=E, I=I, k=2, fmt=fmt,
                        seed=90 + T + E, zipf=0.8)
    flush(f"[layer-pipe] fmt={fmt} T={T} E={E} H={H} I={I} A/E={T * 2 / E:.0f}")
    case = Case(wl)
    layer, y = _run_layer(case, "prefill")
    y = y.clone()
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    assert np.array_equal(layer.sorted_idx[:wl.T * wl.k].cpu().numpy(), ref["sorted_idx"])
    assert rel_err(bf16_to_np(layer.y_perm[:wl.T * wl.k]), ref["y_perm"]) <= TOL
    err = rel_err(bf16_to_np(y), ref["y"])
    _, y_dec = _run_layer(case, "decode")
    dif = rel_err(bf16_to_np(y), bf16_to_np(y_dec))
    flush(f"   rel err {err:.2e}, vs decode kernels {dif:.2e}")
    assert err <= TOL and dif <= 1e-2


# Per-expert row counts on both sides of every 16-row subtile and 64 / 128-row
# tile boundary (and an expert with no rows), one expert per token (k = 1):
# the prefill kernels skip the subtiles past an expert's rows.
BOUNDARY_COUNTS = [1, 15, 16, 17, 0, 63, 64, 65, 127, 128, 129, 2, 300]


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_layer_prefill_row_boundaries(fmt):
    E, H, I = len(BOUNDARY_COUNTS), 512, 768
    T = sum(BOUNDARY_COUNTS)
    wl = synth.Workload(f"bound_{fmt}", T=T, H=H, E=E, I=I, k=1, fmt=fmt, seed=150)
    flush(f"[layer-bounds] fmt={fmt} T={T} E={E}")
    case = Case(wl)
    rng = np.random.default_rng(151)
    expert = np.repeat(np.arange(E), BOUNDARY_COUNTS)
    rng.shuffle(expert)
    lg = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    lg[np.arange(T), expert] = 4.0
    case.logits_np = lg
    case.logits = torch.from_numpy(lg).to(DEV)
    layer, y = _run_layer(case, "prefill")
    y = y.clone()
    assert np.array_equal(layer.counts[:E].cpu().numpy(), np.array(BOUNDARY_COUNTS))
    ref = OL.forward(lg, case.x_np, wl.k, case.oracle_experts())
    e_perm = rel_err(bf16_to_np(layer.y_perm[:T]), ref["y_perm"])
    err = rel_err(bf16_to_np(y), ref["y"])
    flush(f"   rel err y_perm {e_perm:.2e}, y {err:.2e}")
    assert e_perm <= TOL and err <= TOL
    # every row on its own: a wrong or skipped subtile shows in its rows even when
    # the largest row dominates the relative error
    yp = bf16_to_np(layer.y_perm[:T])
    row_err = np.max(np.abs(yp - ref["y_perm"]), axis=1) / np.max(np.abs(ref["y_perm"]), axis=1)
    assert np.all(row_err <= TOL), int(np.argmax(row_err))


# The ends of the supported range: the largest expert count with the largest k
# (the tile search holds sixteen experts per lane), the largest hidden and
# intermediate sizes, and k = E (every token picks every expert).
EXTREME = [(f, T, E, k, H, I) for f in synth.FORMATS
           for (T, E, k, H, I) in ((16, 1024, 16, 256, 256), (5, 2, 2, 16384, 256),
                                   (5, 2, 2, 512, 16384), (5, 2, 2, 16384, 128))]


@pytest.mark.parametrize("fmt,T,E,k,H,I", EXTREME)
def test_layer_extreme_shapes(fmt, T, E, k, H, I):
    wl = synth.Workload(f"ext_{fmt}_{E}_{H}_{I}", T=T, H=H, E=E, I=I, k=k, fmt=fmt,
                        seed=160 + E + H // 128 + I // 64)
    flush(f"[layer-extreme] fmt={fmt} T={T} E={E} k={k} H={H} I={I}")
    case = Case(wl, gen_device="cuda")
    ref = OL.forward(case.logits_np, case.x_np, k, case.oracle_experts())
    A = T * k
    for variant in ("prefill", "decode"):
        layer, y = _run_layer(case, variant)
        assert np.array_equal(layer.counts[:E].cpu().numpy(), ref["counts"])
        assert np.array_equal(layer.sorted_idx[:A].cpu().numpy(), ref["sorted_idx"])
        e_perm = rel_err(bf16_to_np(layer.y_perm[:A]), ref["y_perm"])
        err = rel_err(bf16_to_np(y), ref["y"])
        flush(f"   {variant}: rel err y_perm {e_perm:.2e}, y {err:.2e}")
        assert e_perm <= TOL and err <= TOL


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_variants_agree_and_deterministic(fmt):
    wl = SMALL[fmt]
    flush(f"[variants] fmt={fmt}")
    case = Case(wl)
    _, y1 = _run_layer(case, "decode")
    y1 = y1.clone()
    _, y2 = _run_layer(case, "prefill")
    _, y3 = _run_layer(case, "prefill")
    assert torch.equal(y2, y3)                                  # repeatable bits
    assert rel_err(bf16_to_np(y1), bf16_to_np(y2)) <= 1e-2


@pytest.mark.parametrize("name", ["tiny_bf16", "decode_mxfp4"])
def test_layer_full_size_small_workloads(name):
    wl = synth.WORKLOADS[name]
    flush(f"[layer-full] {name}")
    case = Case(wl, gen_device="cuda")
    layer, y = _run_layer(case)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    for key, buf in (("counts", layer.counts[:wl.E]), ("offsets", layer.offsets[:wl.E + 1]),
                     ("sorted_idx", layer.sorted_idx[:wl.T * wl.k]),
                     ("inv_idx", layer.inv_idx[:wl.T * wl.k])):
        assert np.array_equal(buf.cpu().numpy(), ref[key]), key
    err = rel_err(bf16_to_np(y), ref["y"])
    flush(f"   rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("name,tokens", [
    ("prefill_nvfp4", [0, 1, 2047, 4095]),
    ("large_prefill_mxfp4", [0, 9999, 16383]),
])
def test_layer_full_size_sampled_tokens(name, tokens):
    """Full-size launch configuration; outputs checked token by token."""
    wl = synth.WORKLOADS[name]
    flush(f"[layer-full-sampled] {name} tokens={tokens}")
    case = Case(wl, gen_device="cuda")
    layer, y = _run_layer(case)
    ref_ids, _ = OR.route(case.logits_np, wl.k)
    ref_perm = OP.permute(ref_ids, wl.E)
    assert np.array_equal(layer.ids[:wl.T * wl.k].cpu().numpy().reshape(wl.T, wl.k), ref_ids)
    assert np.array_equal(layer.sorted_idx[:wl.T * wl.k].cpu().numpy(), ref_perm[2])
    ex = case.oracle_experts()
    out = OL.forward_tokens(case.logits_np, case.x_np, wl.k, ex, tokens,
                            shared=case.oracle_shared())
    got = bf16_to_np(y[tokens])
    err = rel_err(got, out["y"])
    flush(f"   rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_prefill_layer_graph_replays_match_eager(fmt):
    """The prefill layer (route+permute, expert FFN, shared expert, combine)
    captured in one graph over three batches: every replay, with eager calls of
    the same layer between replays, gives the eager results bit for bit."""
    wl = synth.Workload(f"graph_{fmt}", T=300, H=512, E=16, I=768, k=2, fmt=fmt, seed=170,
                        zipf=0.8, shared_I=256)
    flush(f"[prefill-graph] fmt={fmt}")
    case = Case(wl)
    layer = moe.MoELayer(fmt, wl.E, wl.H, wl.I, wl.k, wl.T, case.stride, shared_I=wl.shared_I,
                         shared_stride=case.shared.shape[1])
    W = layer.weights(case.records)
    Ws = moe.experts("bf16", 1, wl.H, wl.shared_I, case.shared, case.shared.shape[1])
    batches = []
    for b in range(3):
        lg = torch.from_numpy(synth.make_logits(wl, 300 + b)).to(DEV)
        x = torch.from_numpy(synth.make_x(wl, 300 + b).view(np.int16)).to(DEV).view(torch.bfloat16)
        batches.append((lg, x))
    eager = [layer.forward(lg, x, W, Ws, variant="prefill").clone() for lg, x in batches]
    torch.cuda.synchronize()
    ref = OL.forward(synth.make_logits(wl, 300), synth.make_x(wl, 300), wl.k, case.oracle_experts(),
                     case.oracle_shared())
    assert rel_err(bf16_to_np(eager[0]), ref["y"]) <= TOL
    outs = [torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=DEV) for _ in batches]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (lg, x), o in zip(batches, outs):
            layer.forward(lg, x, W, Ws, variant="prefill")
            o.copy_(layer.y[:wl.T])
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"
        layer.forward(batches[2][0], batches[2][1], W, Ws, variant="prefill")  # eager work between
        torch.cuda.synchronize()


def test_layer_empty_batch():
    wl = SMALL["mxfp4"]
    case = Case(wl)
    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, 4, case.stride)
    W = layer.weights(case.records)
    y = layer.forward(case.logits[:0], case.x[:0], W)
    torch.cuda.synchronize()
    assert y.shape == (0, wl.H)


def test_hbm_read_probe_reads_every_word():
    """The read calibration (measurement library) reads each 16-byte piece exactly once:
    the XOR of all threads' folds is the XOR of every 32-bit word of the region."""
    from moe_expert_ffn_router_amd import measure
    rng = np.random.default_rng(7)
    n = (3 << 20) + 16 * 37  # not a multiple of the grid's stride
    host = rng.integers(0, 2**32, size=n // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda")
    for grid in (1, 300, 2048):
        sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
        measure.moe_measure_hbm_read(src, n, grid, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), grid


@pytest.mark.parametrize("T,H,I", [(1, 512, 256), (37, 512, 256), (300, 1024, 512),
                                   (257, 384, 128), (600, 768, 384), (1030, 1280, 640),
                                   (513, 2048, 1024)])
def test_shared_ffn_dense(T, H, I):
    """moe_shared_ffn (dense bf16 GEMMs, 256-row tiles: ragged row tails, column tails
    of the down product when H is not a multiple of 256, one or several gate/up
    column tiles) against the oracle's SwiGLU and against the routed-expert kernels
    run as one expert with k = 1 over every token."""
    from oracle import ffn as OFF
    flush(f"[shared-ffn] T={T} H={H} I={I}")
    rec = synth.make_shared_record(81, H, I, device="cuda")
    W = moe.experts("bf16", 1, H, I, rec, rec.shape[1])
    xb = synth.make_x(synth.Workload("sh", T=T, H=H, E=1, I=I, k=1, fmt="bf16", seed=82), 0)
    x = torch.from_numpy(xb.view(np.int16)).to("cuda").view(torch.bfloat16)
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_shared_ffn_workspace(W, T), dtype=torch.uint8, device="cuda")
    moe.moe_shared_ffn(W, x, T, y, ws)
    # the same FFN through moe_expert_ffn: one expert, k = 1, identity permutation
    counts = torch.tensor([T], dtype=torch.int32, device="cuda")
    offsets = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    sidx = torch.arange(T, dtype=torch.int32, device="cuda")
    y2 = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    ws2 = torch.empty(moe.moe_expert_ffn_workspace(W, T, 1), dtype=torch.uint8, device="cuda")
    moe.moe_expert_ffn(W, None, x, T, 1, counts, offsets, sidx, y2, ws2)
    torch.cuda.synchronize()
    ex = OL.ExpertSet("bf16", H, I, lambda e: rec[0].cpu().numpy())
    ref = OFF.swiglu(OF.bf16_value(xb), *ex.weights(0))
    assert rel_err(bf16_to_np(y), ref) <= TOL
    assert rel_err(bf16_to_np(y), bf16_to_np(y2)) <= TOL
