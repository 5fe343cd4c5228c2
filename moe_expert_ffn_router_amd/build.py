"""Build libmoe_mi355x.so (gfx950) in-tree with hipcc.

Each source is compiled to an object under _build/ in parallel, then linked
into moe_expert_ffn_router_amd/libmoe_mi355x.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe_mi355x.so")
OBJ = os.path.join(ROOT, "_build", "obj")
ARCH = "gfx950"

SOURCES = ["status.cpp", "cache.cpp", "cpu_expert.cpp", "route.hip", "permute.hip", "ffn.hip", "combine.hip",
           "decode.hip", "shared.hip"]
# measurement helpers: a library of their own (include/moe_measure.h)
MEASURE_SOURCES = ["measure/hbm_read.hip"]
MEASURE_OUT = os.path.join(PKG, "libmoe_measure.so")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay disabled in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj_dir: str = OBJ, extra: tuple = ()) -> str:
    obj = os.path.join(obj_dir, src.replace("/", "_") + ".o")
    cmd = [hipcc()] + COMMON + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def _link(objs: list[str], out: str, libs: list[str]) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + libs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, debug: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + MEASURE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[len(SOURCES):], MEASURE_OUT, [])
    _link(objs[:len(SOURCES)], OUT, [])
    if verbose:
        print(f"[build] wrote {OUT}")
    if debug:
        build_debug(verbose)
    return OUT


# Host-sanitizer build: the same sources with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host side only (device code unchanged), as
# a separate library; the CPU tests load it through MOE_LIB_PATH with the ASan
# runtime preloaded.
ASAN_OUT = os.path.join(ROOT, "_build", "asan", "libmoe_mi355x_asan.so")
ASAN_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
              "-fno-omit-frame-pointer", "-g")


def asan_runtime() -> str:
    import glob
    c = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not c:
        raise RuntimeError("ASan runtime not found")
    return c[-1]


def build_host_sanitized(verbose: bool = False) -> str:
    obj_dir = os.path.join(ROOT, "_build", "asan")
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, ASAN_FLAGS), SOURCES))
    _link(objs, ASAN_OUT, ["-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"])
    if verbose:
        print(f"[build] wrote {ASAN_OUT}")
    return ASAN_OUT


# Bounds-checked build: the same sources with -DMOE_DEBUG (every index taken
# from a caller's array range-checked and clamped in the kernels, flags read
# back by moe_debug_take), as a separate library next to the release one,
# loaded through MOE_LIB_PATH; build() makes both.
DEBUG_OUT = os.path.join(PKG, "libmoe_mi355x_debug.so")


def build_debug(verbose: bool = False) -> str:
    obj_dir = os.path.join(ROOT, "_build", "debug")
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, ("-DMOE_DEBUG",)), SOURCES))
    _link(objs, DEBUG_OUT, [])
    if verbose:
        print(f"[build] wrote {DEBUG_OUT}")
    return DEBUG_OUT


if __name__ == "__main__":
    if "asan" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    elif "debug" in sys.argv[1:]:
        build_debug(verbose=True)
    else:
        build(verbose=True)
