"""The bounds-checked build (-DMOE_DEBUG): a second library with the same C ABI
whose kernels range-check every index taken from a caller's array.

CPU: the release library reports MOE_ERR_UNSUPPORTED from moe_debug_take; the
checked library loads through MOE_LIB_PATH, binds every declared function and
validates its argument without a GPU.
GPU: a child process on the checked library (tests/debug_child.py) runs the
layer in every format against the oracle with no flag raised, then one planted
out-of-range index per kind, each clamped in the kernel and named by its flag.
"""
import os
import subprocess
import sys

import pytest
import torch

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "moe_expert_ffn_router_amd"))
import build as B  # noqa: E402

m = pytest.importorskip("moe_expert_ffn_router_amd")


def _checked_lib() -> str:
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)
            if f.endswith((".hip", ".cpp", ".h"))]
    srcs.append(os.path.join(ROOT, "include", "moe_layer.h"))
    if not os.path.exists(B.DEBUG_OUT) or \
            os.path.getmtime(B.DEBUG_OUT) < max(os.path.getmtime(s) for s in srcs):
        B.build_debug()
    return B.DEBUG_OUT


def _env() -> dict:
    env = dict(os.environ)
    env.update(MOE_LIB_PATH=_checked_lib(), PYTHONPATH=ROOT)
    return env


def test_release_build_has_no_checks():
    with pytest.raises(m.MoeError) as ei:
        m.moe_debug_take()
    assert ei.value.status == m.MOE_ERR_UNSUPPORTED
    assert m._lib.moe_debug_take(None) == m.MOE_ERR_INVALID_ARG


PROBE = r"""
import ctypes, moe_expert_ffn_router_amd as moe
assert moe.LIB_PATH.endswith("libmoe_mi355x_debug.so"), moe.LIB_PATH
print("symbols", len(moe.exported_symbols()))
print("null", moe._lib.moe_debug_take(None))
"""


def test_checked_build_binds_the_same_abi():
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, env=_env(), capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert f"symbols {len(m.exported_symbols())}" in r.stdout
    assert f"null {m.MOE_ERR_INVALID_ARG}" in r.stdout


@pytest.mark.gpu
@pytest.mark.timeout(400)
@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_checked_build_on_gpu():
    print("[debug build] child process on the checked library", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "debug_child.py")],
                       cwd=ROOT, env=_env(), capture_output=True, text=True, timeout=360)
    print(r.stdout[-6000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    assert "DEBUG CHILD OK" in r.stdout
