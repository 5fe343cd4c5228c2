"""Binding of libmoe_measure.so: measurement helpers kept apart from the layer's library
(include/moe_measure.h).  Used by the benchmark's read calibration only."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_measure.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (moe_expert_ffn_router_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)
_lib.moe_measure_hbm_read.restype = ctypes.c_int
_lib.moe_measure_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]


def exported_symbols() -> list[str]:
    return ["moe_measure_hbm_read"]


def moe_measure_hbm_read(src: torch.Tensor, nbytes: int, grid: int, sink: torch.Tensor,
                         stream=None) -> None:
    if nbytes > src.numel() * src.element_size() or sink.numel() * sink.element_size() < grid * 1024:
        raise ValueError("moe_measure_hbm_read: region or sink too small")
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = _lib.moe_measure_hbm_read(src.data_ptr(), nbytes, grid, sink.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"moe_measure_hbm_read failed with status {rc}")
