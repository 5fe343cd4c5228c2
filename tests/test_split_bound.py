"""The block-scaled MFMA paths feed each bf16 activation as two E4M3 values,
hi = RNE_e4m3(x / 2^e) and lo = RNE_e4m3(x / 2^e - hi), with one E8M0 scale 2^e
per 32 values placing the block maximum in [128, 256).  This checks, on a CPU
model of that split (torch's float32 -> float8_e4m3fn cast rounds to nearest
even), the error bound the kernels' comments state:

  * |x - (hi + lo) 2^e| <= 2^-10 * 2^e <= 2^-17 * max|block|, for every element;
  * the split is exact for elements within 2^9 of the block maximum;
  * the bound is reached by small elements (so "exact for bf16" would be false).
"""
import numpy as np
import torch


def split(x: np.ndarray):
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    amax = np.max(np.abs(xb))
    e = int(np.floor(np.log2(amax))) - 7            # block maximum in [128, 256)
    v = xb / 2.0 ** e
    hi = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).float().numpy()
    lo = torch.from_numpy((v - hi).astype(np.float32)).to(torch.float8_e4m3fn).float().numpy()
    return xb, e, hi.astype(np.float64), lo.astype(np.float64)


def test_split_error_bound_wide_dynamic_range():
    rng = np.random.default_rng(11)
    worst = 0.0
    reached = False
    for trial in range(400):
        mag = 2.0 ** rng.uniform(-24, 0, 32)          # 24 binades inside one block
        x = mag * rng.choice([-1.0, 1.0], 32) * rng.uniform(1, 2, 32)
        xb, e, hi, lo = split(x)
        err = np.abs(xb - (hi + lo) * 2.0 ** e)
        amax = np.max(np.abs(xb))
        assert np.all(err <= 2.0 ** -10 * 2.0 ** e)
        assert np.all(err <= 2.0 ** -17 * amax)
        near = np.abs(xb / 2.0 ** e) >= 0.25
        assert np.all(err[near] == 0.0)
        worst = max(worst, float(np.max(err / amax)))
        reached |= bool(np.any(err > 0))
    assert reached and worst > 2.0 ** -19


def test_split_exact_on_narrow_blocks():
    rng = np.random.default_rng(12)
    for _ in range(200):
        x = rng.standard_normal(32) * 0.02 + 0.05     # all within 2^9 of the maximum
        x[np.abs(x) < 1e-4] = 1e-3
        xb, e, hi, lo = split(x)
        if np.min(np.abs(xb)) * 512 >= np.max(np.abs(xb)):
            assert np.array_equal((hi + lo) * 2.0 ** e, xb)
