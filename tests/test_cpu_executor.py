"""The CPU expert executor (moe_cpu_expert_ffn: host threads, host memory) against the
oracle, on the CPU: every format, several experts with ragged row counts including
empty ones, outputs rows of listed experts only, results independent of the thread
count.  Bar: y_perm rows within 2e-2 * max|oracle| (bf16 rounding of h and y)."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn as OFF
from oracle import formats as OF
from oracle import permute as OP
from oracle import route as OR

moe = pytest.importorskip("moe_expert_ffn_router_amd")

TOL = 2e-2


def _case(fmt, T=40, H=256, E=6, I=128, k=2, seed=5):
    wl = synth.Workload(f"cpu_{fmt}", T=T, H=H, E=E, I=I, k=k, fmt=fmt, seed=seed, zipf=1.0)
    recs = synth.make_expert_records(fmt, E, H, I, seed)            # host
    stride = recs.shape[1]
    lg, xb = synth.make_logits(wl), synth.make_x(wl)
    ids, _ = OR.route(lg, k)
    counts, offsets, sidx, inv = OP.permute(ids, E)
    return wl, recs, stride, xb, counts, offsets, sidx


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_cpu_executor_matches_oracle(fmt):
    wl, recs, stride, xb, counts, offsets, sidx = _case(fmt)
    W = moe.experts(fmt, wl.E, wl.H, wl.I, recs.data_ptr(), stride)
    pool = moe.CpuPool(4)
    A = wl.T * wl.k
    listed = [e for e in range(wl.E) if e % 2 == 0] + [e for e in range(wl.E) if counts[e] == 0]
    listed = sorted(set(listed))
    y = torch.full((A, wl.H), 7, dtype=torch.int16)                 # sentinel rows
    moe.moe_cpu_expert_ffn(pool, W, torch.tensor(listed, dtype=torch.int32),
                           torch.from_numpy(xb.view(np.int16)), wl.T, wl.k,
                           torch.from_numpy(offsets.astype(np.int32)),
                           torch.from_numpy(sidx.astype(np.int32)), y)
    x = OF.bf16_value(xb)
    got_rows, ref_rows = [], []
    for e in range(wl.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = y[lo:hi].numpy()
        if e not in listed:
            assert np.all(rows == 7), e                             # untouched
            continue
        if hi == lo:
            continue
        g, u, d = OF.decode_record(recs[e].numpy(), fmt, wl.H, wl.I)
        ref_rows.append(OFF.swiglu(x[sidx[lo:hi] // wl.k], g, u, d))
        got_rows.append(OF.bf16_value(rows.view(np.uint16)))
    got, ref = np.concatenate(got_rows), np.concatenate(ref_rows)
    err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    assert err <= TOL, err
    pool.close()


def test_cpu_executor_thread_count_invariant():
    wl, recs, stride, xb, counts, offsets, sidx = _case("mxfp4", T=33, H=512, E=5, I=256, k=3)
    W = moe.experts("mxfp4", wl.E, wl.H, wl.I, recs.data_ptr(), stride)
    outs = []
    for threads in (1, 3, 8):
        pool = moe.CpuPool(threads)
        y = torch.zeros((wl.T * wl.k, wl.H), dtype=torch.int16)
        moe.moe_cpu_expert_ffn(pool, W, torch.arange(wl.E, dtype=torch.int32),
                               torch.from_numpy(xb.view(np.int16)), wl.T, wl.k,
                               torch.from_numpy(offsets.astype(np.int32)),
                               torch.from_numpy(sidx.astype(np.int32)), y)
        outs.append(y)
        pool.close()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_cpu_executor_argument_checks():
    pool = moe.CpuPool(1)
    W = moe.experts("mxfp4", 4, 256, 128, 0, 4096)
    with pytest.raises(moe.MoeError):
        moe.moe_cpu_expert_ffn(pool, W, torch.tensor([0], dtype=torch.int32),
                               torch.zeros((1, 256), dtype=torch.int16), 1, 1,
                               torch.zeros(5, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                               torch.zeros((1, 256), dtype=torch.int16))
    pool.close()
