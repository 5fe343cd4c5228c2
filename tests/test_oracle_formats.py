"""Pins of the oracle's weight-format decoders (CPU only).

Each decoder is checked against something other than itself: the published
value tables (tests/golden), torch's own float8 casts, mathematical invariants,
and round trips through the generator's independently written encoders.
"""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from conftest import GOLDEN


def _read_pairs(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            out.append((int(a, 0), float(b)))
    return out


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_published_table():
    rows = _read_pairs("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        assert _same(float(F.e2m1_value(code)), val), (code, val)


def test_e2m1_invariants():
    v = F.e2m1_value(np.arange(16))
    assert np.all(np.diff(v[:8]) > 0)              # magnitudes strictly increase
    assert np.array_equal(v[8:], -v[:8])            # sign bit mirrors
    assert v.max() == 6.0 and np.all(np.isfinite(v))


def test_e4m3_landmarks_and_torch_cast():
    for code, val in _read_pairs("e4m3_landmarks.txt"):
        assert _same(float(F.e4m3_value(code)), val), hex(code)
    ours = F.e4m3_value(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_invariants():
    v = F.e4m3_value(np.arange(0x7F))               # all positive finite codes
    assert np.all(np.diff(v) > 0)
    assert len(np.unique(F.e4m3_value(np.arange(256))[~np.isnan(F.e4m3_value(np.arange(256)))])) == 253


def test_e8m0_landmarks_and_torch_cast():
    for code, val in _read_pairs("e8m0_landmarks.txt"):
        got = float(F.e8m0_value(code))
        assert (math.isnan(val) and math.isnan(got)) or got == val, code
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    ours = F.e8m0_value(np.arange(256))
    assert np.array_equal(ours[:255], ref[:255]) and np.isnan(ours[255])


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(4096, generator=g).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_value(bits), x.double().numpy())


def test_nibble_order_low_first():
    # element 2i lives in the low nibble: byte 0x21 holds codes (1, 2) = (0.5, 1.0)
    codes = F.unpack_e2m1(np.array([[0x21, 0xF0]], dtype=np.uint8), 4)
    assert codes.tolist() == [[1, 2, 0, 15]]


def test_encoder_decoder_round_trip_all_codes():
    # generator encoders are written separately from the oracle decoders
    vals = torch.tensor(F.e2m1_value(np.arange(16)), dtype=torch.float32)
    assert synth._e2m1_encode(vals).tolist() == list(range(16))
    b = np.arange(256)
    fin = ~np.isnan(F.e4m3_value(b))
    enc = synth._e4m3_bytes(torch.tensor(F.e4m3_value(b[fin]), dtype=torch.float32)).numpy()
    assert np.array_equal(enc, b[fin])


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_record_layout_agrees_with_generator(fmt):
    H, I = 256, 128
    ours = F.record_sections(fmt, H, I)
    gen = synth.record_layout(fmt, H, I)["sections"]
    assert ours == {k: tuple(v) for k, v in gen.items()}


def _grid_weights(fmt, N, K, seed):
    """Weights exactly representable in `fmt` so that encode -> decode is exact."""
    rng = np.random.default_rng(seed)
    if fmt == "mxfp4":
        grid = F.e2m1_value(np.arange(16))
        v = rng.choice(grid, size=(N, K))
        v[:, ::32] = 6.0                             # pin each block's amax at 6 * 2^e
        e = rng.integers(-8, -2, size=(N, K // 32))
        return v * np.exp2(np.repeat(e, 32, axis=1))
    if fmt == "fp8_b128":
        vals = F.e4m3_value(np.arange(0x7F))
        v = rng.choice(np.concatenate([vals, -vals]), size=(N, K))
        v[::128, ::128] = 448.0
        s = np.exp2(rng.integers(-12, -6, size=(N // 128, K // 128)).astype(np.float64))
        return v * np.repeat(np.repeat(s, 128, 0), 128, 1)
    if fmt == "bf16":
        return (torch.randn(N, K, dtype=torch.float32) * 0.02).to(torch.bfloat16).double().numpy()
    raise ValueError(fmt)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8_b128", "bf16"])
def test_exact_round_trip_on_grid(fmt):
    H, I = 256, 128
    w13 = _grid_weights(fmt, 2 * I, H, 1)
    w2 = _grid_weights(fmt, H, I, 2)
    rec = synth.encode_record(fmt, torch.tensor(w13, dtype=torch.float32),
                              torch.tensor(w2, dtype=torch.float32)).numpy()
    wg, wu, wd = F.decode_record(rec, fmt, H, I)
    assert np.array_equal(np.concatenate([wg, wu]), w13.astype(np.float32).astype(np.float64))
    assert np.array_equal(wd, w2.astype(np.float32).astype(np.float64))


def test_nvfp4_round_trip_error_bound():
    # w ~ N(0, 0.02): every decoded element lies within half a grid step of the
    # encoder's target at its block scale (the grid step near 6 is 2).
    H, I = 256, 128
    w13, w2 = synth.expert_float_weights(7, 0, 0, H, I)
    rec = synth.encode_record("nvfp4", w13, w2).numpy()
    wg, wu, wd = F.decode_record(rec, "nvfp4", H, I)
    for got, ref in ((wg, w13[:I]), (wu, w13[I:]), (wd, w2)):
        ref = ref.double().numpy()
        blk_amax = np.abs(ref.reshape(ref.shape[0], -1, 16)).max(-1)
        tol = np.repeat(blk_amax, 16, axis=1) / 6.0 * 1.0 * 1.07 + 1e-12
        assert np.all(np.abs(got - ref) <= tol)
        assert np.corrcoef(got.ravel(), ref.ravel())[0, 1] > 0.99


def test_mxfp4_random_round_trip_error_bound():
    H, I = 256, 128
    w13, w2 = synth.expert_float_weights(8, 0, 0, H, I)
    rec = synth.encode_record("mxfp4", w13, w2).numpy()
    wg, wu, wd = F.decode_record(rec, "mxfp4", H, I)
    ref = w13.double().numpy()
    got = np.concatenate([wg, wu])
    blk = np.abs(ref.reshape(2 * I, -1, 32)).max(-1)
    scale = np.exp2(np.floor(np.log2(blk)) - 2)
    # magnitudes below 4*scale round to a grid of step <= 1*scale (half-step 0.5);
    # the top interval [4,6] has step 2, and (6,8) saturates: error < 2*scale
    assert np.all(np.abs(got - ref) <= 2.0 * np.repeat(scale, 32, axis=1))
    assert np.corrcoef(got.ravel(), ref.ravel())[0, 1] > 0.98
