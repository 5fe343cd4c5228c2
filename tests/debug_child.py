"""Child process of test_gpu_debug_build: runs with MOE_LIB_PATH naming the
bounds-checked library (built with -DMOE_DEBUG).

1. Clean inputs: the layer in every weight format, both FFN variants and the
   two-launch decode layer, against the oracle, with no range flag raised.
2. Planted inputs, one out-of-range index each (a slot-table entry, a
   sorted_idx value, an expert's row segment, an inv_idx value): the checked
   kernels replace it by an in-range one, so they stay inside their buffers,
   and raise the flag that names it.  The planted cases run only after
   moe_debug_take has succeeded, i.e. only on the checked build.
Prints one line per step and "DEBUG CHILD OK" at the end.
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
from gpu_cases import TOL, Case, bf16_to_np, flush, rel_err  # noqa: E402
from oracle import layer as OL  # noqa: E402

import moe_expert_ffn_router_amd as moe  # noqa: E402

DEV = torch.device("cuda")


def _take() -> int:
    torch.cuda.synchronize()
    return moe.moe_debug_take()


def _expect(flag: int, what: str) -> None:
    got = _take()
    flush(f"   {what}: flags {got:#x}")
    assert got == flag, (what, got, flag)


def _layer_case(fmt: str, seed: int):
    wl = synth.Workload(f"dbg_{fmt}", T=150, H=384, E=6, I=256, k=2, fmt=fmt, seed=seed, zipf=0.7)
    case = Case(wl)
    layer = moe.MoELayer(fmt, wl.E, wl.H, wl.I, wl.k, wl.T, case.stride)
    return wl, case, layer, layer.weights(case.records)


def clean_and_planted_ffn(fmt: str, seed: int) -> None:
    wl, case, layer, W = _layer_case(fmt, seed)
    ref = OL.forward(case.logits_np, case.x_np, wl.k, case.oracle_experts())
    A = wl.T * wl.k
    for variant in ("decode", "prefill"):
        flush(f"[clean] fmt={fmt} variant={variant}")
        y = layer.forward(case.logits, case.x, W, variant=variant)
        torch.cuda.synchronize()
        err = rel_err(bf16_to_np(y), ref["y"])
        flush(f"   rel err y {err:.2e}")
        assert err <= TOL
        _expect(0, "clean run")

    counts = layer.counts[:wl.E].cpu().numpy()
    used = [int(e) for e in np.nonzero(counts)[0]]
    assert len(used) >= 2
    for variant in ("decode", "prefill"):
        flush(f"[planted] fmt={fmt} variant={variant}")
        layer.route_permute(case.logits)
        slot = torch.arange(wl.E, dtype=torch.int32, device=DEV)
        slot[used[0]] = wl.E + 5
        slot[used[1]] = -1
        layer.expert_ffn(W, case.x, wl.T, slot, variant)
        _expect(moe.DBG_SLOT, "slot table entries E+5 and -1")

        keep = layer.sorted_idx.clone()
        layer.sorted_idx[5] = A + 100
        layer.sorted_idx[6] = -3
        layer.expert_ffn(W, case.x, wl.T, None, variant)
        _expect(moe.DBG_SORTED, "sorted_idx values T*k+100 and -3")
        layer.sorted_idx.copy_(keep)

        keep = layer.offsets.clone()
        layer.offsets[used[0]] = A
        layer.expert_ffn(W, case.x, wl.T, None, variant)
        _expect(moe.DBG_SEGMENT, "row segment starting at T*k")
        layer.offsets.copy_(keep)

        # the restored inputs raise nothing and give the oracle's result again
        layer.expert_ffn(W, case.x, wl.T, None, variant)
        layer.combine(wl.T, False)
        torch.cuda.synchronize()
        assert rel_err(bf16_to_np(layer.y[:wl.T]), ref["y"]) <= TOL
        _expect(0, "restored inputs")

    flush(f"[planted] fmt={fmt} combine")
    keep = layer.inv_idx.clone()
    layer.inv_idx[3] = A + 7
    layer.inv_idx[4] = -1
    layer.combine(wl.T, False)
    _expect(moe.DBG_INV, "inv_idx values T*k+7 and -1")
    layer.inv_idx.copy_(keep)


def clean_and_planted_decode(fmt: str, T: int, H: int, E: int, I: int, k: int, seed: int) -> None:
    wl = synth.Workload(f"dbgdec_{fmt}", T=T, H=H, E=E, I=I, k=k, fmt=fmt, seed=seed)
    assert moe.moe_forward_decode_supported(H, I, T, k)
    case = Case(wl)
    layer = moe.MoELayer(fmt, E, H, I, k, T, case.stride)
    W = layer.weights(case.records)
    flush(f"[clean] decode layer fmt={fmt} T={T} H={H} E={E} I={I} k={k}")
    y = layer.forward_decode(case.logits, case.x, W)
    torch.cuda.synchronize()
    ref = OL.forward(case.logits_np, case.x_np, k, case.oracle_experts())
    err = rel_err(bf16_to_np(y), ref["y"])
    flush(f"   rel err y {err:.2e}")
    assert err <= TOL
    _expect(0, "clean run")
    ids = layer.ids[:T * k].cpu().numpy()
    flush(f"[planted] decode layer fmt={fmt}")
    slot = torch.arange(E, dtype=torch.int32, device=DEV)
    slot[int(ids[0])] = E + 3
    layer.forward_decode(case.logits, case.x, W, slot)
    _expect(moe.DBG_SLOT, "slot table entry E+3 of a routed expert")


def main() -> int:
    flush(f"[debug child] library {moe.LIB_PATH}")
    assert os.path.basename(moe.LIB_PATH) == "libmoe_mi355x_debug.so"
    moe.moe_debug_take()  # raises MoeError on a release build: nothing planted runs there
    for i, fmt in enumerate(synth.FORMATS):
        clean_and_planted_ffn(fmt, 40 + i)
    # the fused MXFP4 one-stream shape, a token-major and a tile-major shape
    clean_and_planted_decode("mxfp4", 8, 512, 64, 512, 8, 71)
    clean_and_planted_decode("nvfp4", 4, 1024, 64, 1024, 4, 72)
    clean_and_planted_decode("fp8_b128", 32, 512, 64, 512, 4, 73)   # tile-major + combine
    flush("DEBUG CHILD OK")
    return 0


if __name__ == "__main__":
    sys.exit(main())
