"""MI355X (gfx950) MoE-layer forward: Python binding of libmoe_mi355x.so.

Thin ctypes marshalling over the C ABI declared in include/moe_layer.h: every
function here has the name of the C entry point it calls, turns torch tensors
into device pointers and the current torch stream into a hipStream_t, and
raises MoeError on a non-zero status.  Every step of the layer runs in the
library's HIP kernels; there is no Python or CPU fallback — importing this
package fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (the host-sanitizer build,
# the bounds-checked build)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_CAPACITY, \
    MOE_ERR_WORKSPACE = range(6)
FMT = {"bf16": 0, "mxfp4": 1, "nvfp4": 2, "fp8_b128": 3}
VARIANT = {"auto": 0, "decode": 1, "prefill": 2}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python moe_expert_ffn_router_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_p, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class ExpertLayout(ctypes.Structure):
    _fields_ = [("w13", _i64), ("w13_scale", _i64), ("w2", _i64), ("w2_scale", _i64),
                ("tensor_scale", _i64), ("payload_bytes", _i64), ("stride", _i64)]


class BwProfile(ctypes.Structure):
    _fields_ = [("h2d_bytes_per_s", ctypes.c_double), ("cpu_bytes_per_s", ctypes.c_double),
                ("threshold", ctypes.c_double), ("fetch_fraction", ctypes.c_double),
                ("hybrid_recommended", ctypes.c_int32)]


class Experts(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("E", _i32), ("H", _i32), ("I", _i32), ("base", _p),
                ("stride", _i64)]


_SIGS = {
    "moe_expert_layout_query": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(ExpertLayout)]),
    "moe_route": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _p, _p, _p]),
    "moe_permute_workspace": (_sz, [_i32, _i32, _i32]),
    "moe_permute": (ctypes.c_int, [_p, _i32, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_route_permute": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p,
                                         _sz, _p]),
    "moe_expert_ffn_workspace": (_sz, [ctypes.POINTER(Experts), _i32, _i32]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(Experts), _p, _p, _i32, _i32, _p, _p, _p, _p,
                                      _i32, _p, _sz, _p]),
    "moe_combine": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p]),
    "moe_forward_decode_supported": (ctypes.c_int, [_i32, _i32, _i32, _i32]),
    "moe_forward_decode_workspace": (_sz, [ctypes.POINTER(Experts), _i32, _i32]),
    "moe_forward_decode": (ctypes.c_int, [ctypes.POINTER(Experts), _p, _p, _p, _i32, _i32, _i32, _p,
                                          _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_forward_decode_noalloc_max_scratch": (_sz, []),
    "moe_forward_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(Experts), _p, _p, _p, _i32, _i32,
                                                  _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_dequant_expert": (ctypes.c_int, [ctypes.POINTER(Experts), _i32, _p, _p, _p]),
    "moe_cache_create": (ctypes.c_int, [ctypes.POINTER(_p), _i32, _i32, _i32, _i64, _p, _p, _p]),
    "moe_cache_destroy": (None, [_p]),
    "expert_cache_lookup": (ctypes.c_int, [_p, _i32, _p, _p, _p, _p, _p, _p]),
    "expert_cache_row": (ctypes.c_int, [_p, _i32, _p]),
    "expert_cache_fill": (ctypes.c_int, [_p, _i32, _p, _p, _i32, _p, _p]),
    "expert_cache_fill_groups": (ctypes.c_int, [_p, _i32, _p, _p, _i32, _i32, _p, _p]),
    "expert_cache_wait_group": (ctypes.c_int, [_p, _i32, _p]),
    "expert_cache_plan": (ctypes.c_int, [_p, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_expert_ffn_streamed_workspace": (_sz, [ctypes.POINTER(Experts), _i32, _i32]),
    "moe_expert_ffn_streamed": (ctypes.c_int, [_p, _i32, ctypes.POINTER(Experts), _p, _i32, _i32,
                                               _p, _p, _p, _p, _i32, _p, _sz, _p, _p, _p, _p, _p,
                                               _p, _p]),
    "moe_cache_resize": (ctypes.c_int, [_p, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_cache_stats": (ctypes.c_int, [_p, _p, _p, _p, _p]),
    "moe_cpu_pool_create": (ctypes.c_int, [ctypes.POINTER(_p), _i32]),
    "moe_cpu_pool_destroy": (None, [_p]),
    "moe_cpu_expert_ffn": (ctypes.c_int, [_p, ctypes.POINTER(Experts), _p, _i32, _p, _i32, _i32,
                                          _p, _p, _p]),
    "expert_cache_plan_hybrid": (ctypes.c_int, [_p, _i32, _p, ctypes.c_double, _i32, _p, _p, _p,
                                                _p, _p, _p, _p]),
    "moe_expert_ffn_hybrid_host_bytes": (_sz, [ctypes.POINTER(Experts), _i32, _i32]),
    "moe_expert_ffn_hybrid": (ctypes.c_int, [_p, _i32, ctypes.POINTER(Experts), _p, _p, _i32, _i32,
                                             _p, _p, _p, _p, ctypes.c_double, _i32, _i32, _p, _sz,
                                             _p, _sz, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_bench_bw": (ctypes.c_int, [_p, ctypes.POINTER(Experts), _p, _i32, _p, ctypes.c_double,
                                    ctypes.POINTER(BwProfile)]),
    "moe_shared_ffn_workspace": (_sz, [ctypes.POINTER(Experts), _i32]),
    "moe_shared_ffn": (ctypes.c_int, [ctypes.POINTER(Experts), _p, _i32, _p, _p, _sz, _p]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_int, []),
    "moe_debug_take": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32)]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def exported_symbols() -> list[str]:
    return sorted(_SIGS)


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        msg = _lib.moe_last_error().decode(errors="replace")
        name = _lib.moe_status_str(status).decode()
        raise MoeError(status, f"{what}: {name}: {msg}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, got {type(t)}")
    if t.numel() and not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_check(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor) and t.numel() and not t.is_cuda:
            raise ValueError("device tensor expected")


# ---------------------------------------------------------------------------
def moe_expert_layout_query(fmt: str | int, H: int, I: int) -> dict:
    out = ExpertLayout()
    _check(_lib.moe_expert_layout_query(FMT.get(fmt, fmt), H, I, ctypes.byref(out)),
           "moe_expert_layout_query")
    return {f: getattr(out, f) for f, _ in ExpertLayout._fields_}


def experts(fmt: str | int, E: int, H: int, I: int, base: torch.Tensor | int, stride: int) -> Experts:
    """moe_experts descriptor over `base` (a device tensor or a raw pointer)."""
    return Experts(FMT.get(fmt, fmt), E, H, I, _ptr(base), stride)


def moe_route(logits, k: int, topk_ids, topk_w, renorm: bool = True, stream=None) -> None:
    _dev_check(logits, topk_ids, topk_w)
    T, E = logits.shape
    _check(_lib.moe_route(_ptr(logits), T, E, k, int(renorm), _ptr(topk_ids), _ptr(topk_w),
                          _stream(stream)), "moe_route")


def moe_permute_workspace(T: int, k: int, E: int) -> int:
    return int(_lib.moe_permute_workspace(T, k, E))


def moe_permute(topk_ids, T: int, k: int, E: int, counts, offsets, sorted_idx, inv_idx, ws,
                stream=None) -> None:
    _dev_check(topk_ids, counts, offsets, sorted_idx, inv_idx, ws)
    _check(_lib.moe_permute(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets),
                            _ptr(sorted_idx), _ptr(inv_idx), _ptr(ws),
                            ws.numel() * ws.element_size() if ws is not None else 0,
                            _stream(stream)), "moe_permute")


def moe_route_permute(logits, k: int, topk_ids, topk_w, counts, offsets, sorted_idx, inv_idx, ws,
                      renorm: bool = True, stream=None) -> None:
    _dev_check(logits, topk_ids, topk_w, counts, offsets, sorted_idx, inv_idx, ws)
    T, E = logits.shape
    _check(_lib.moe_route_permute(_ptr(logits), T, E, k, int(renorm), _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(counts), _ptr(offsets), _ptr(sorted_idx), _ptr(inv_idx),
                                  _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                  _stream(stream)), "moe_route_permute")


def moe_expert_ffn_workspace(W: Experts, T: int, k: int) -> int:
    return int(_lib.moe_expert_ffn_workspace(ctypes.byref(W), T, k))


def moe_expert_ffn(W: Experts, slot_of_expert, x, T: int, k: int, counts, offsets, sorted_idx,
                   y_perm, ws, variant: str | int = "auto", stream=None) -> None:
    _dev_check(slot_of_expert, x, counts, offsets, sorted_idx, y_perm, ws)
    _check(_lib.moe_expert_ffn(ctypes.byref(W), _ptr(slot_of_expert), _ptr(x), T, k, _ptr(counts),
                               _ptr(offsets), _ptr(sorted_idx), _ptr(y_perm),
                               VARIANT.get(variant, variant), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)),
           "moe_expert_ffn")


def moe_combine(y_perm, inv_idx, topk_w, T: int, k: int, H: int, y_shared, y, stream=None) -> None:
    _dev_check(y_perm, inv_idx, topk_w, y_shared, y)
    _check(_lib.moe_combine(_ptr(y_perm), _ptr(inv_idx), _ptr(topk_w), T, k, H, _ptr(y_shared),
                            _ptr(y), _stream(stream)), "moe_combine")


def moe_forward_decode_supported(H: int, I: int, T: int, k: int) -> bool:
    return bool(_lib.moe_forward_decode_supported(H, I, T, k))


def moe_forward_decode_workspace(W: Experts, T: int, k: int) -> int:
    return int(_lib.moe_forward_decode_workspace(ctypes.byref(W), T, k))


def moe_forward_decode(W: Experts, slot_of_expert, logits, x, k: int, topk_ids, topk_w, counts,
                       offsets, sorted_idx, inv_idx, y_shared, y, ws, renorm: bool = True,
                       stream=None) -> None:
    """Whole layer for decode-sized batches in two launches."""
    _dev_check(slot_of_expert, logits, x, topk_ids, topk_w, counts, offsets, sorted_idx, inv_idx,
               y_shared, y, ws)
    T = logits.shape[0]
    _check(_lib.moe_forward_decode(ctypes.byref(W), _ptr(slot_of_expert), _ptr(logits), _ptr(x), T,
                                   k, int(renorm), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                                   _ptr(offsets), _ptr(sorted_idx), _ptr(inv_idx), _ptr(y_shared),
                                   _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "moe_forward_decode")


def moe_forward_decode_noalloc_max_scratch() -> int:
    return int(_lib.moe_forward_decode_noalloc_max_scratch())


def moe_forward_decode_noalloc(W: Experts, slot_of_expert, logits, x, k: int, topk_ids, topk_w,
                               counts, offsets, sorted_idx, inv_idx, y_shared, y,
                               renorm: bool = True, stream=None) -> None:
    """moe_forward_decode with the library's fixed per-device scratch (no workspace)."""
    _dev_check(slot_of_expert, logits, x, topk_ids, topk_w, counts, offsets, sorted_idx, inv_idx,
               y_shared, y)
    T = logits.shape[0]
    _check(_lib.moe_forward_decode_noalloc(ctypes.byref(W), _ptr(slot_of_expert), _ptr(logits),
                                           _ptr(x), T, k, int(renorm), _ptr(topk_ids),
                                           _ptr(topk_w), _ptr(counts), _ptr(offsets),
                                           _ptr(sorted_idx), _ptr(inv_idx), _ptr(y_shared),
                                           _ptr(y), _stream(stream)), "moe_forward_decode_noalloc")


def moe_dequant_expert(W: Experts, expert: int, w13, w2, stream=None) -> None:
    _dev_check(w13, w2)
    _check(_lib.moe_dequant_expert(ctypes.byref(W), expert, _ptr(w13), _ptr(w2), _stream(stream)),
           "moe_dequant_expert")


class ExpertCache:
    """Owner of a moe_cache_t handle (host metadata only)."""

    def __init__(self, n_layers: int, E: int, S: int, slot_bytes: int, pool=None, bank=None,
                 slot_table=None):
        h = ctypes.c_void_p()
        _check(_lib.moe_cache_create(ctypes.byref(h), n_layers, E, S, slot_bytes, _ptr(pool),
                                     _ptr(bank), _ptr(slot_table)), "moe_cache_create")
        self._h = h
        self.E, self.S = E, S
        self._keep = (pool, bank, slot_table)
        self.miss_e = torch.zeros(E, dtype=torch.int32)
        self.miss_s = torch.zeros(E, dtype=torch.int32)
        self.row = torch.zeros(E, dtype=torch.int32)

    def close(self):
        if self._h:
            _lib.moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def expert_cache_lookup(self, layer: int, counts_host: torch.Tensor):
        c = counts_host.to(torch.int32).contiguous()
        nm, nh = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.expert_cache_lookup(self._h, layer, _ptr(c), _ptr(self.miss_e),
                                        _ptr(self.miss_s), ctypes.byref(nm), ctypes.byref(nh),
                                        _ptr(self.row)), "expert_cache_lookup")
        n = nm.value
        return (self.miss_e[:n].clone(), self.miss_s[:n].clone(), n, nh.value, self.row.clone())

    def expert_cache_row(self, layer: int) -> torch.Tensor:
        row = torch.zeros(self.E, dtype=torch.int32)
        _check(_lib.expert_cache_row(self._h, layer, _ptr(row)), "expert_cache_row")
        return row

    def expert_cache_fill(self, layer: int, miss_expert, miss_slot, side=None, compute=None):
        me = miss_expert.to(torch.int32).contiguous()
        ms = miss_slot.to(torch.int32).contiguous()
        _check(_lib.expert_cache_fill(self._h, layer, _ptr(me), _ptr(ms), int(me.numel()),
                                      _stream(side), _stream(compute)), "expert_cache_fill")

    def expert_cache_fill_groups(self, layer: int, miss_expert, miss_slot, n_groups: int,
                                 side=None, compute=None):
        me = miss_expert.to(torch.int32).contiguous()
        ms = miss_slot.to(torch.int32).contiguous()
        _check(_lib.expert_cache_fill_groups(self._h, layer, _ptr(me), _ptr(ms), int(me.numel()),
                                             n_groups, _stream(side), _stream(compute)),
               "expert_cache_fill_groups")

    def expert_cache_wait_group(self, group: int, compute=None):
        _check(_lib.expert_cache_wait_group(self._h, group, _stream(compute)),
               "expert_cache_wait_group")

    def expert_cache_plan(self, layer: int, counts_host: torch.Tensor):
        """The step's waves and fills (host-only policy; advances the cache state)."""
        c = counts_host.to(torch.int32).contiguous()
        E = self.E
        wave_of = torch.zeros(E, dtype=torch.int32)
        fe, fs, we = (torch.zeros(E, dtype=torch.int32) for _ in range(3))
        nw, nh = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.expert_cache_plan(self._h, layer, _ptr(c), _ptr(wave_of), _ptr(fe), _ptr(fs),
                                      _ptr(we), ctypes.byref(nw), ctypes.byref(nh)),
               "expert_cache_plan")
        return _plan_result(wave_of, fe, fs, we, nw.value, nh.value)

    def moe_expert_ffn_streamed(self, layer: int, pool_W: Experts, x, T: int, k: int,
                                counts_host: torch.Tensor, offsets, sorted_idx, y_perm,
                                n_groups: int, ws, side=None, compute=None, out=None):
        """One step's expert FFN through the pool with streamed fills.  `out` (optional):
        three host int32 [E] tensors that receive the fills' experts, their slots and each
        wave's fill end (reused across calls).  Returns (n_waves, n_hit)."""
        E = self.E
        if out is None:
            out = tuple(torch.zeros(E, dtype=torch.int32) for _ in range(3))
        fe, fs, we = out
        nw, nh = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.moe_expert_ffn_streamed(self._h, layer, ctypes.byref(pool_W), _ptr(x), T, k,
                                            _ptr(counts_host), _ptr(offsets), _ptr(sorted_idx),
                                            _ptr(y_perm), n_groups, _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(side),
                                            _stream(compute), _ptr(fe), _ptr(fs), _ptr(we),
                                            ctypes.byref(nw), ctypes.byref(nh)),
               "moe_expert_ffn_streamed")
        return nw.value, nh.value

    def expert_cache_plan_hybrid(self, layer: int, counts_host: torch.Tensor,
                                 fetch_fraction: float, max_fetch: int = -1) -> dict:
        """One hybrid step's policy (host only; advances the cache state)."""
        c = counts_host.to(torch.int32).contiguous()
        E = self.E
        cpu, fe, fs, we = (torch.zeros(E, dtype=torch.int32) for _ in range(4))
        nc, nw, nh = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.expert_cache_plan_hybrid(self._h, layer, _ptr(c), fetch_fraction, max_fetch,
                                             _ptr(cpu), ctypes.byref(nc), _ptr(fe), _ptr(fs),
                                             _ptr(we), ctypes.byref(nw), ctypes.byref(nh)),
               "expert_cache_plan_hybrid")
        r = _plan_result(torch.full((E,), -1, dtype=torch.int32), fe, fs, we, nw.value, nh.value)
        r["cpu"] = cpu[:nc.value].tolist()
        return r

    def moe_expert_ffn_hybrid(self, layer: int, pool_W: Experts, cpu_pool, x, T: int, k: int,
                              counts_host: torch.Tensor, offsets, sorted_idx, y_perm,
                              fetch_fraction: float, max_fetch: int, n_groups: int, ws,
                              host_stage, side=None, compute=None, out=None):
        """One hybrid step (see the header).  `out`: four host int32 [E] tensors reused
        across calls (CPU experts, fills' experts, their slots, wave ends).  Returns
        (n_cpu, n_waves, n_hit)."""
        E = self.E
        if out is None:
            out = tuple(torch.zeros(E, dtype=torch.int32) for _ in range(4))
        ce, fe, fs, we = out
        nc, nw, nh = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.moe_expert_ffn_hybrid(self._h, layer, ctypes.byref(pool_W), cpu_pool._h,
                                          _ptr(x), T, k, _ptr(counts_host), _ptr(offsets),
                                          _ptr(sorted_idx), _ptr(y_perm), fetch_fraction,
                                          max_fetch, n_groups, _ptr(ws),
                                          ws.numel() * ws.element_size(), _ptr(host_stage),
                                          host_stage.numel() * host_stage.element_size(),
                                          _stream(side), _stream(compute), _ptr(ce),
                                          ctypes.byref(nc), _ptr(fe), _ptr(fs), _ptr(we),
                                          ctypes.byref(nw), ctypes.byref(nh)),
               "moe_expert_ffn_hybrid")
        return nc.value, nw.value, nh.value

    def moe_cache_resize(self, new_S: int, pool=None, side=None, compute=None):
        """Resize to new_S slots (into `pool` if given, else in place); returns the
        (old slot, new slot) pairs of the kept residents as two int32 tensors."""
        m = min(self.S, new_S)
        frm = torch.zeros(m, dtype=torch.int32)
        to = torch.zeros(m, dtype=torch.int32)
        n = ctypes.c_int32()
        _check(_lib.moe_cache_resize(self._h, new_S, _ptr(pool), _ptr(frm), _ptr(to),
                                     ctypes.byref(n), _stream(side), _stream(compute)),
               "moe_cache_resize")
        self.S = new_S
        if pool is not None:
            self._keep = (pool,) + self._keep[1:]
        return frm[:n.value].clone(), to[:n.value].clone()

    def stats(self) -> dict:
        v = [ctypes.c_int64() for _ in range(4)]
        _check(_lib.moe_cache_stats(self._h, *[ctypes.byref(x) for x in v]), "moe_cache_stats")
        return dict(zip(("steps", "hits", "misses", "bytes_filled"), (x.value for x in v)))


class CpuPool:
    """Owner of a moe_cpu_pool_t (host threads of the CPU expert executor)."""

    def __init__(self, threads: int):
        h = ctypes.c_void_p()
        _check(_lib.moe_cpu_pool_create(ctypes.byref(h), threads), "moe_cpu_pool_create")
        self._h = h
        self.threads = threads

    def close(self):
        if self._h:
            _lib.moe_cpu_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _host_check(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor) and t.numel() and t.is_cuda:
            raise ValueError("host tensor expected")


def moe_cpu_expert_ffn(pool: CpuPool, W: Experts, experts, x, T: int, k: int, offsets, sorted_idx,
                       y_perm) -> None:
    """The listed experts' FFN on the CPU (host tensors throughout; W.base is host memory)."""
    _host_check(experts, x, offsets, sorted_idx, y_perm)
    ex = experts.to(torch.int32).contiguous()
    _check(_lib.moe_cpu_expert_ffn(pool._h, ctypes.byref(W), _ptr(ex), int(ex.numel()), _ptr(x), T,
                                   k, _ptr(offsets), _ptr(sorted_idx), _ptr(y_perm)),
           "moe_cpu_expert_ffn")


def moe_bench_bw(pool: CpuPool, bank_W: Experts, pool_dev, n_records: int, threshold: float = 2.0,
                 stream=None) -> dict:
    out = BwProfile()
    _check(_lib.moe_bench_bw(pool._h, ctypes.byref(bank_W), _ptr(pool_dev), n_records,
                             _stream(stream), threshold, ctypes.byref(out)), "moe_bench_bw")
    return {f: getattr(out, f) for f, _ in BwProfile._fields_}


def _plan_result(wave_of, fe, fs, we, n_waves: int, n_hit: int) -> dict:
    ends = we[:n_waves].tolist()
    starts = [0] + ends[:-1]
    fills = list(zip(fe[:ends[-1] if ends else 0].tolist(), fs[:ends[-1] if ends else 0].tolist()))
    waves = [[] for _ in range(n_waves)]
    for e, w in enumerate(wave_of.tolist()):
        if w >= 0:
            waves[w].append(e)
    return {"waves": waves, "fills": [fills[a:b] for a, b in zip(starts, ends)],
            "n_waves": n_waves, "hits": n_hit, "misses": len(fills)}


def moe_expert_ffn_hybrid_host_bytes(W: Experts, T: int, k: int) -> int:
    return int(_lib.moe_expert_ffn_hybrid_host_bytes(ctypes.byref(W), T, k))


def moe_expert_ffn_streamed_workspace(W: Experts, T: int, k: int) -> int:
    return int(_lib.moe_expert_ffn_streamed_workspace(ctypes.byref(W), T, k))


def moe_shared_ffn_workspace(W: Experts, T: int) -> int:
    return int(_lib.moe_shared_ffn_workspace(ctypes.byref(W), T))


def moe_shared_ffn(W: Experts, x: torch.Tensor, T: int, y: torch.Tensor, ws: torch.Tensor,
                   stream=None) -> None:
    _check(_lib.moe_shared_ffn(ctypes.byref(W), _ptr(x), T, _ptr(y), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "moe_shared_ffn")


def moe_version() -> int:
    return int(_lib.moe_version())


DBG_SLOT, DBG_SORTED, DBG_SEGMENT, DBG_INV = 1, 2, 4, 8


def moe_debug_take() -> int:
    """Flags raised by a bounds-checked build's range checks since the last call
    (cleared); raises MoeError (MOE_ERR_UNSUPPORTED) on a release build."""
    f = ctypes.c_uint32(0)
    _check(_lib.moe_debug_take(ctypes.byref(f)), "moe_debug_take")
    return int(f.value)


from .layer import MoELayer  # noqa: E402,F401


def moe_status_str_py(status: int) -> str:
    return _lib.moe_status_str(status).decode()
