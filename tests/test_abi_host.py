"""Host-side checks of the C-ABI library (no GPU needed).

* the shared library loads and exports every function include/*.h declares;
* the library's record layout agrees with the generator's and the oracle's;
* argument validation returns the documented status codes;
* the C++ LRU (expert_cache_lookup) reproduces the oracle policy step by step.
"""
import ctypes
import glob
import os
import re

import numpy as np
import pytest
import torch

import synth
from conftest import GOLDEN, ROOT
from oracle import formats as OF
from oracle import lru as OL

m = pytest.importorskip("moe_expert_ffn_router_amd")


def _declared_functions(header: str):
    names = set()
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    for mm in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                          src, flags=re.M):
        name = mm.group(1)
        if name not in ("if", "sizeof", "defined"):
            names.add(name)
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h"))) \
        == ["moe_layer.h", "moe_measure.h"]


def test_every_declared_symbol_is_exported():
    declared = _declared_functions("moe_layer.h")
    assert len(declared) >= 14, declared
    lib = ctypes.CDLL(m.LIB_PATH)
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared) == set(m.exported_symbols())


def test_measure_library_exports_its_header():
    from moe_expert_ffn_router_amd import measure
    declared = _declared_functions("moe_measure.h")
    lib = ctypes.CDLL(measure.LIB_PATH)
    assert declared and all(hasattr(lib, n) for n in declared)
    assert set(declared) == set(measure.exported_symbols())
    # the layer's library carries no measurement helper
    assert not hasattr(ctypes.CDLL(m.LIB_PATH), "moe_measure_hbm_read")
    assert measure._lib.moe_measure_hbm_read(None, 16, 1, None, None) == 1


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("H,I", [(256, 128), (2048, 512), (4096, 1024), (7168, 2048)])
def test_layout_agrees(fmt, H, I):
    lib = m.moe_expert_layout_query(fmt, H, I)
    gen = synth.record_layout(fmt, H, I)
    orc = OF.record_sections(fmt, H, I)
    assert lib["stride"] == gen["stride"] and lib["payload_bytes"] == gen["payload"]
    names = {"w13": "w13", "w13_scale": "w13s", "w2": "w2", "w2_scale": "w2s", "tensor_scale": "ts"}
    for k, g in names.items():
        if lib[k] < 0:
            assert g not in gen["sections"]
        else:
            assert lib[k] == gen["sections"][g][0] == orc[g][0]


def test_layout_rejects_unsupported():
    with pytest.raises(m.MoeError) as e:
        m.moe_expert_layout_query("mxfp4", 200, 128)
    assert e.value.status == m.MOE_ERR_UNSUPPORTED
    with pytest.raises(m.MoeError):
        m.moe_expert_layout_query(7, 256, 128)


def test_validation_before_enqueue():
    # invalid arguments are refused before any device work (no GPU touched)
    lib = m._lib
    assert lib.moe_route(None, 4, 0, 1, 1, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, 4, 8, 9, 1, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, 4, 2000, 2, 1, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, 0, 8, 2, 1, None, None, None) == m.MOE_OK     # empty input
    assert lib.moe_route(None, 4, 8, 2, 1, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert "null" in lib.moe_last_error().decode()
    assert lib.moe_combine(None, None, None, 4, 2, 100, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(None, None, None, 0, 2, 64, None, None, None) == m.MOE_OK
    W = m.experts("mxfp4", 8, 256, 128, 4096, 70000)   # stride not a multiple of 256
    assert lib.moe_expert_ffn(ctypes.byref(W), None, None, 4, 2, None, None, None, None, 0, None,
                              0, None) == m.MOE_ERR_INVALID_ARG
    W = m.experts("mxfp4", 8, 256, 128, 4096, 1 << 20)
    assert lib.moe_expert_ffn(ctypes.byref(W), None, None, 0, 2, None, None, None, None, 0, None,
                              0, None) == m.MOE_OK
    assert lib.moe_expert_ffn(ctypes.byref(W), None, 16, 4, 2, 16, 16, 16, 16, 0, 16, 0,
                              None) == m.MOE_ERR_WORKSPACE
    assert m.moe_status_str_py(m.MOE_ERR_CAPACITY) == "MOE_ERR_CAPACITY"


def test_workspace_queries_monotone():
    assert m.moe_permute_workspace(4096, 8, 256) >= 32 * 256 * 4
    W = m.experts("nvfp4", 256, 2048, 512, 4096, synth.record_layout("nvfp4", 2048, 512)["stride"])
    a = m.moe_expert_ffn_workspace(W, 8, 8)
    b = m.moe_expert_ffn_workspace(W, 4096, 8)
    assert b > a >= 8 * 8 * 512 * 2


def _golden_trace():
    import test_oracle_lru as T
    return T._trace()


def test_cpp_lru_hand_worked_trace():
    c = m.ExpertCache(2, 8, 3, 256)
    for layer, needed, exp in _golden_trace():
        counts = torch.zeros(8, dtype=torch.int32)
        counts[needed] = 1
        if exp is None:
            with pytest.raises(m.MoeError) as e:
                c.expert_cache_lookup(layer, counts)
            assert e.value.status == m.MOE_ERR_CAPACITY
            continue
        me, ms, nm, nh, _ = c.expert_cache_lookup(layer, counts)
        assert (list(zip(me.tolist(), ms.tolist())), nh, nm) == exp


@pytest.mark.parametrize("seed", range(6))
def test_cpp_lru_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    L, E, S = 3, 40, 14
    cpp = m.ExpertCache(L, E, S, 256)
    ora = OL.LruSlots(S)
    for step in range(300):
        layer = int(rng.integers(0, L))
        n = int(rng.integers(0, S + 2))
        counts = np.zeros(E, np.int32)
        counts[rng.permutation(E)[:n]] = rng.integers(1, 9, size=n)
        try:
            r = ora.step(layer, counts)
        except OL.CapacityError:
            with pytest.raises(m.MoeError) as e:
                cpp.expert_cache_lookup(layer, torch.from_numpy(counts))
            assert e.value.status == m.MOE_ERR_CAPACITY
            continue
        me, ms, nm, nh, row = cpp.expert_cache_lookup(layer, torch.from_numpy(counts))
        assert list(zip(me.tolist(), ms.tolist())) == r["fills"]
        assert (nm, nh) == (r["misses"], r["hits"])
        assert np.array_equal(row.numpy(), ora.slot_table(layer, E))
        other = int(rng.integers(0, L))   # another layer's current row, as it stands now
        assert np.array_equal(cpp.expert_cache_row(other).numpy(), ora.slot_table(other, E))
    st = cpp.stats()
    assert st["bytes_filled"] == 0 and st["steps"] > 0


@pytest.mark.parametrize("seed", range(4))
def test_cpp_resize_matches_oracle(seed):
    """Pool resizes between steps (host-only handle): the same kept residents and
    placements as the oracle, then the same fills."""
    rng = np.random.default_rng(40 + seed)
    L, E, S = 3, 32, 12
    cpp = m.ExpertCache(L, E, S, 256)
    ora = OL.LruSlots(S)
    for step in range(250):
        if rng.random() < 0.08:
            new_S = int(rng.integers(1, 20))
            frm, to = cpp.moe_cache_resize(new_S, side=0, compute=0)
            assert list(zip(frm.tolist(), to.tolist())) == ora.resize(new_S)
            for layer in range(L):
                assert np.array_equal(cpp.expert_cache_row(layer).numpy(),
                                      ora.slot_table(layer, E))
            continue
        layer = int(rng.integers(0, L))
        n = int(rng.integers(0, ora.S + 1))
        counts = np.zeros(E, np.int32)
        counts[rng.permutation(E)[:n]] = rng.integers(1, 9, size=n)
        r = ora.step(layer, counts)
        me, ms, nm, nh, row = cpp.expert_cache_lookup(layer, torch.from_numpy(counts))
        assert list(zip(me.tolist(), ms.tolist())) == r["fills"]
        assert np.array_equal(row.numpy(), ora.slot_table(layer, E))


def test_cache_resize_argument_checks():
    c = m.ExpertCache(1, 8, 3, 256)
    with pytest.raises(m.MoeError) as e:
        c.moe_cache_resize(0, side=0, compute=0)
    assert e.value.status == m.MOE_ERR_INVALID_ARG
    with pytest.raises(m.MoeError) as e:   # host-only handle: no pool to move into
        c.moe_cache_resize(4, pool=torch.zeros(4 * 256, dtype=torch.uint8), side=0, compute=0)
    assert e.value.status == m.MOE_ERR_INVALID_ARG
    assert c.S == 3


def test_cache_fill_requires_device_pieces():
    c = m.ExpertCache(1, 8, 3, 256)
    with pytest.raises(m.MoeError):
        c.expert_cache_fill(0, torch.zeros(0, dtype=torch.int32), torch.zeros(0, dtype=torch.int32),
                            side=0, compute=0)
    with pytest.raises(m.MoeError) as e:
        m.ExpertCache(1, 8, 0, 256)
    assert e.value.status == m.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("H,I,E", [(2048, 512, 256), (512, 1024, 128), (2048, 2048, 64)])
def test_decode_workspace_serves_smaller_batches(fmt, H, I, E):
    """The decode-layer workspace sized for T also fits every batch of T' <= T tokens
    (the MXFP4 one-stream path's partials exist only for some batch sizes)."""
    W = m.experts(fmt, E, H, I, None, synth.record_layout(fmt, H, I)["stride"])
    k = 8
    sizes = [m.moe_forward_decode_workspace(W, T, k) for T in range(0, 65)]
    for T in range(65):
        assert sizes[T] >= max(sizes[:T + 1]), (T, sizes[T], max(sizes[:T + 1]))
    # the h and y_perm sections alone
    for T in (1, 8, 16, 64):
        assert sizes[T] >= T * k * (I + H) * 2
