"""moe_forward_decode_noalloc (the decode layer with the library's fixed per-device
scratch) against moe_forward_decode with a caller workspace: every output identical,
on two calls in a row through the C ABI, the second with a smaller batch (the scratch
keeps the first call's contents; nothing may depend on them).  Passes alone in a fresh
process and after the other tests (its name puts it last in the collection)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_cases import flush

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")
OUTS = ("ids", "w", "counts", "offsets", "sorted_idx", "inv_idx", "y")


def _bufs(T, k, E, H):
    A = T * k
    return {"ids": torch.full((A,), -7, dtype=torch.int32, device=DEV),
            "w": torch.full((A,), -7.0, dtype=torch.float32, device=DEV),
            "counts": torch.full((E,), -7, dtype=torch.int32, device=DEV),
            "offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
            "sorted_idx": torch.full((A,), -7, dtype=torch.int32, device=DEV),
            "inv_idx": torch.full((A,), -7, dtype=torch.int32, device=DEV),
            "y": torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)}


def _call(fn_name, W, logits, x, k, b, ws=None):
    lib = moe._lib
    T = logits.shape[0]
    s = torch.cuda.current_stream().cuda_stream
    args = [ctypes.byref(W), None, logits.data_ptr(), x.data_ptr(), T, k, 1,
            b["ids"].data_ptr(), b["w"].data_ptr(), b["counts"].data_ptr(),
            b["offsets"].data_ptr(), b["sorted_idx"].data_ptr(), b["inv_idx"].data_ptr(),
            None, b["y"].data_ptr()]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    rc = getattr(lib, fn_name)(*args, s)
    assert rc == moe.MOE_OK, (fn_name, rc, lib.moe_last_error().decode())


@pytest.mark.parametrize("fmt,T1,T2", [("mxfp4", 8, 3), ("bf16", 12, 5), ("nvfp4", 24, 9)])
def test_noalloc_matches_workspace_call(fmt, T1, T2):
    wl = synth.Workload(f"noalloc_{fmt}", T=T1, H=2048 if fmt == "mxfp4" else 1024, E=64,
                        I=512, k=8, fmt=fmt, seed=95)
    flush(f"[noalloc] {fmt} T={T1} then T={T2}")
    stride = synth.record_layout(wl.fmt, wl.H, wl.I)["stride"]
    recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, device=DEV)
    W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, recs, stride)
    need = moe.moe_forward_decode_workspace(W, T1, wl.k)
    assert 0 < need <= moe.moe_forward_decode_noalloc_max_scratch()
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for T in (T1, T2):                       # second call smaller than the first
        lg = torch.from_numpy(synth.make_logits(wl, T, T=T)).to(DEV)
        x = torch.from_numpy(synth.make_x(wl, T, T=T).view(np.int16)).to(DEV).view(torch.bfloat16)
        ref, got = _bufs(T, wl.k, wl.E, wl.H), _bufs(T, wl.k, wl.E, wl.H)
        _call("moe_forward_decode", W, lg, x, wl.k, ref, ws)
        _call("moe_forward_decode_noalloc", W, lg, x, wl.k, got)
        torch.cuda.synchronize()
        for n in OUTS:
            a, b = ref[n], got[n]
            if a.dtype in (torch.float32, torch.bfloat16):
                a, b = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16), \
                    b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)
            assert torch.equal(a, b), (fmt, T, n)


def test_noalloc_rejects_oversized_request():
    # the one-stream MXFP4 path at T=16, I=2048 needs 16 MiB of fp32 partials
    wl = synth.Workload("noalloc_big", T=16, H=2048, E=256, I=2048, k=8, fmt="mxfp4", seed=96)
    stride = synth.record_layout(wl.fmt, wl.H, wl.I)["stride"]
    W = moe.experts(wl.fmt, wl.E, wl.H, wl.I, 256, stride)
    assert moe.moe_forward_decode_workspace(W, 16, 8) > moe.moe_forward_decode_noalloc_max_scratch()
    dummy = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    p = dummy.data_ptr()
    rc = moe._lib.moe_forward_decode_noalloc(ctypes.byref(W), None, p, p, 16, 8, 1, p, p, p, p,
                                             p, p, None, p, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    assert "scratch" in moe._lib.moe_last_error().decode()
