"""Pins of the oracle's SwiGLU FFN, combine and whole-layer composition (CPU only)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import combine as C
from oracle import ffn as FF
from oracle import formats as F
from oracle import layer as L
from oracle import permute as P
from oracle import route as R


def _torch_dense_swiglu(X, Wg, Wu, Wd):
    X, Wg, Wu, Wd = (torch.tensor(a, dtype=torch.float64) for a in (X, Wg, Wu, Wd))
    return (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T) @ Wd.T).numpy()


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(FF.silu(z), torch.nn.functional.silu(torch.tensor(z)).numpy(),
                       rtol=1e-15, atol=1e-300)


def test_single_expert_equals_dense_mlp():
    """E = 1, k = 1: the MoE layer is a dense SwiGLU MLP on every token."""
    wl = synth.WORKLOADS["tiny_bf16"].scaled(E=1, k=1, T=16)
    rec = synth.make_expert_records("bf16", 1, wl.H, wl.I, wl.seed)
    ex = L.ExpertSet("bf16", wl.H, wl.I, lambda e: rec[e].numpy())
    lg = synth.make_logits(wl)
    xb = synth.make_x(wl)
    out = L.forward(lg, xb, 1, ex)
    x = F.bf16_value(xb)
    ref = _torch_dense_swiglu(x, *ex.weights(0))
    assert np.allclose(out["w"], 1.0)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


def test_scalar_loop_brute_force():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((3, 8))
    Wg, Wu = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    Wd = rng.standard_normal((8, 4))
    got = FF.swiglu(X, Wg, Wu, Wd)
    for t in range(3):
        hid = []
        for i in range(4):
            g = sum(X[t, h] * Wg[i, h] for h in range(8))
            u = sum(X[t, h] * Wu[i, h] for h in range(8))
            hid.append(g / (1.0 + math.exp(-g)) * u)
        for n in range(8):
            ref = sum(hid[i] * Wd[n, i] for i in range(4))
            assert abs(got[t, n] - ref) <= 1e-12 * (1 + abs(ref))


def test_gate_up_not_interchangeable():
    """Swapping the gate and up halves must change the result (catches a swap)."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((4, 16))
    Wg, Wu, Wd = rng.standard_normal((8, 16)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8))
    assert not np.allclose(FF.swiglu(X, Wg, Wu, Wd), FF.swiglu(X, Wu, Wg, Wd))


def test_zero_expert_and_linearity_in_down():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((5, 16))
    Wg, Wu, Wd = rng.standard_normal((8, 16)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8))
    assert np.all(FF.swiglu(X, Wg, Wu, np.zeros_like(Wd)) == 0)
    assert np.all(FF.swiglu(X, np.zeros_like(Wg), Wu, Wd) == 0)
    assert np.array_equal(FF.swiglu(X, Wg, Wu, 2 * Wd), 2 * FF.swiglu(X, Wg, Wu, Wd))


def test_combine_k1_and_one_hot():
    rng = np.random.default_rng(5)
    T, H, E = 6, 4, 3
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    _, _, s, inv = P.permute(ids, E)
    yp = rng.standard_normal((T, H))
    y = C.combine(yp, inv, np.ones((T, 1)), T, 1)
    assert np.array_equal(y, yp[inv])
    # one-hot weights pick a single expert output per token
    k = 2
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, s, inv = P.permute(ids, E)
    yp = rng.standard_normal((T * k, H))
    w = np.zeros((T, k)); w[:, 1] = 1.0
    y = C.combine(yp, inv, w, T, k)
    assert np.array_equal(y, yp[inv.reshape(T, k)[:, 1]])


def test_shared_expert_alone_is_dense_mlp():
    wl = synth.WORKLOADS["tiny_bf16"].scaled(T=8)
    H, I = wl.H, wl.I
    shared = synth.make_shared_record(9, H, I)
    sh = L.ExpertSet("bf16", H, I, lambda e: shared[0].numpy())
    zero = np.zeros(synth.record_layout("bf16", H, I)["stride"], np.uint8)
    ex = L.ExpertSet("bf16", H, I, lambda e: zero)        # routed experts all zero
    lg, xb = synth.make_logits(wl), synth.make_x(wl)
    out = L.forward(lg, xb, wl.k, ex, shared=sh)
    ref = _torch_dense_swiglu(F.bf16_value(xb), *sh.weights(0))
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_forward_tokens_matches_forward(fmt):
    H, I = (256, 128)
    wl = synth.Workload("t", T=24, H=H, E=6, I=I, k=2, fmt=fmt, seed=12, zipf=1.1)
    rec = synth.make_expert_records(fmt, wl.E, H, I, wl.seed)
    ex = L.ExpertSet(fmt, H, I, lambda e: rec[e].numpy())
    lg, xb = synth.make_logits(wl), synth.make_x(wl)
    full = L.forward(lg, xb, wl.k, ex)
    toks = [0, 5, 23]
    part = L.forward_tokens(lg, xb, wl.k, ex, toks)
    assert np.allclose(part["y"], full["y"][toks], rtol=1e-12, atol=1e-14)
    assert np.array_equal(part["ids"], full["ids"][toks])


def test_layer_equals_direct_sum_over_experts():
    """y[t] = sum_j w_tj * FFN_{e_tj}(x_t), computed without any permutation."""
    wl = synth.WORKLOADS["tiny_bf16"]
    rec = synth.make_expert_records("bf16", wl.E, wl.H, wl.I, wl.seed)
    ex = L.ExpertSet("bf16", wl.H, wl.I, lambda e: rec[e].numpy())
    lg, xb = synth.make_logits(wl), synth.make_x(wl)
    out = L.forward(lg, xb, wl.k, ex)
    x = F.bf16_value(xb)
    ids, w = R.route(lg, wl.k)
    ref = np.zeros_like(out["y"])
    for t in range(wl.T):
        for j in range(wl.k):
            ref[t] += w[t, j] * _torch_dense_swiglu(x[t:t + 1], *ex.weights(int(ids[t, j])))[0]
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-14)
