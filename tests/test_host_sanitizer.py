"""Host-side sanitizer run (no GPU): the library built with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code (device code unchanged) runs the host
tests — the LRU policy, wave and hybrid planners, resize, argument validation and the
CPU expert executor — in a child process with the ASan runtime preloaded; any report
fails it.  A planted out-of-bounds write (an output buffer smaller than the caller
promised) must be reported, which shows the instrumentation is live."""
import glob
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "moe_expert_ffn_router_amd"))
import build as B  # noqa: E402

HOST_TESTS = ["tests/test_host_streaming.py", "tests/test_cpu_executor.py",
              "tests/test_abi_host.py"]


def _asan_lib():
    srcs = glob.glob(os.path.join(B.CSRC, "*.hip")) + glob.glob(os.path.join(B.CSRC, "*.cpp")) + \
        glob.glob(os.path.join(B.CSRC, "*.h"))
    if not os.path.exists(B.ASAN_OUT) or \
            os.path.getmtime(B.ASAN_OUT) < max(os.path.getmtime(s) for s in srcs):
        B.build_host_sanitized()
    return B.ASAN_OUT


def _env():
    env = dict(os.environ)
    env.update(MOE_LIB_PATH=_asan_lib(), LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    return env


def test_host_code_clean_under_asan_ubsan():
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + HOST_TESTS,
                       cwd=ROOT, env=_env(), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


PLANTED = r"""
import numpy as np, torch, synth
import moe_expert_ffn_router_amd as moe
from oracle import route as OR, permute as OP
wl = synth.Workload("x", T=8, H=256, E=4, I=128, k=2, fmt="bf16", seed=1)
recs = synth.make_expert_records("bf16", 4, 256, 128, 1)
W = moe.experts("bf16", 4, 256, 128, recs.data_ptr(), recs.shape[1])
ids, _ = OR.route(synth.make_logits(wl), 2)
c, o, s, i = OP.permute(ids, 4)
pool = moe.CpuPool(1)
y = torch.zeros((3, 256), dtype=torch.int16)      # 16 rows promised, 3 given
moe.moe_cpu_expert_ffn(pool, W, torch.arange(4, dtype=torch.int32),
                       torch.from_numpy(synth.make_x(wl).view(np.int16)), 8, 2,
                       torch.from_numpy(o.astype(np.int32)), torch.from_numpy(s.astype(np.int32)), y)
print("NO REPORT")
"""


def test_planted_overflow_is_reported():
    r = subprocess.run([sys.executable, "-c", PLANTED], cwd=ROOT, env=_env(),
                       capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert "heap-buffer-overflow" in out and "NO REPORT" not in out, out[-3000:]
