"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each case replaces one oracle function with a subtly wrong version and runs
the pin that is meant to catch it; the pin must raise AssertionError.  This
shows the pins are not just re-typings of the oracle's formulas.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import combine as C
from oracle import ffn as FF
from oracle import formats as F
from oracle import lru as LR
from oracle import permute as P
from oracle import route as R

import test_oracle_ffn_layer as T_ffn
import test_oracle_formats as T_fmt
import test_oracle_lru as T_lru
import test_oracle_route_permute as T_rp


def test_bf16_record_gate_rows_first():
    """Decoded gate / up / down equal the generator's float weights rounded to bf16."""
    H, I = 256, 128
    w13, w2 = synth.expert_float_weights(3, 0, 5, H, I)
    rec = synth.encode_record("bf16", w13, w2).numpy()
    wg, wu, wd = F.decode_record(rec, "bf16", H, I)
    b = lambda t: t.to(torch.bfloat16).double().numpy()
    assert np.array_equal(wg, b(w13[:I])) and np.array_equal(wu, b(w13[I:]))
    assert np.array_equal(wd, b(w2))


# ---- the planted mistakes --------------------------------------------------
def _e2m1_wrong_bias(code):
    c = np.asarray(code, dtype=np.int64)
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e))
    return np.where(s == 1, -mag, mag)


def _unpack_swapped(packed, K):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], K), dtype=np.uint8)
    out[:, 0::2] = p >> 4
    out[:, 1::2] = p & 0x0F
    return out


def _e4m3_bias8(b):
    b = np.asarray(b, dtype=np.int64)
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _route_high_index_ties(logits, k, renorm=True):
    lg = np.asarray(logits, np.float32).astype(np.float64)
    E = lg.shape[1]
    rev = lg[:, ::-1]
    order = (E - 1) - np.argsort(-rev, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(lg, ids.astype(np.int64), 1)
    z = np.exp(sel - sel[:, :1])
    return ids, z / z.sum(1, keepdims=True)


def _route_no_renorm_as_default(logits, k, renorm=True):
    lg = np.asarray(logits, np.float32).astype(np.float64)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)
    m = lg.max(1, keepdims=True)
    w = np.exp(np.take_along_axis(lg, ids.astype(np.int64), 1) - m) / np.exp(lg - m).sum(1, keepdims=True)
    return ids, w


def _permute_unstable(ids, E):
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    A = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    # descending assignment index inside each expert segment
    sorted_idx = np.lexsort((-np.arange(A), flat)).astype(np.int32)
    inv = np.empty(A, np.int32)
    inv[sorted_idx] = np.arange(A)
    return counts, offsets, sorted_idx, inv


def _silu_sign(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(z))


def _combine_reversed(y_perm, inv_idx, w, T, k, y_shared=None):
    w = np.asarray(w, np.float64).reshape(T, k)[:, ::-1]
    return C.__wrapped_combine(y_perm, inv_idx, w, T, k, y_shared)


def _decode_gate_up_swapped(record, fmt, H, I):
    wg, wu, wd = F.__wrapped_decode(record, fmt, H, I)
    return wu, wg, wd


class _LruMru(LR.LruSlots):
    def step(self, layer, counts):
        # evicts the MOST recently used unneeded slot
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        if len(needed) > self.S:
            raise LR.CapacityError("cap")
        keys = {(layer, e) for e in needed}
        misses = [e for e in needed if (layer, e) not in self.where]
        fills = []
        for e in misses:
            empty = [s for s in range(self.S) if self.owner[s] is None]
            if empty:
                s = empty[0]
            else:
                cands = [s for s in range(self.S) if self.owner[s] not in keys]
                s = max(cands, key=lambda q: (self.recency[q], -q))
                del self.where[self.owner[s]]
            self.owner[s] = (layer, e)
            self.where[(layer, e)] = s
            fills.append((e, s))
        for e in needed:
            self.recency[self.where[(layer, e)]] = self.clock
        self.clock += 1
        return {"needed": needed, "slot_of": {e: self.where[(layer, e)] for e in needed},
                "fills": fills, "hits": len(needed) - len(misses), "misses": len(misses)}


class _LruResizeKeepsOldest(LR.LruSlots):
    def resize(self, new_S):
        # keeps the LEAST recently used residents
        resident = [s for s in range(self.S) if self.owner[s] is not None]
        kept = sorted(sorted(resident, key=lambda q: (self.recency[q], q))[:new_S])
        owner = [self.owner[q] for q in kept] + [None] * (new_S - len(kept))
        recency = [self.recency[q] for q in kept] + [-1] * (new_S - len(kept))
        self.S, self.owner, self.recency = new_S, owner, recency
        self.where = {key: p for p, key in enumerate(owner) if key is not None}
        return [(q, p) for p, q in enumerate(kept)]


class _LruResizeNoPacking(LR.LruSlots):
    def resize(self, new_S):
        # keeps the right residents but leaves them in their old slots when they fit
        resident = [s for s in range(self.S) if self.owner[s] is not None]
        kept = sorted(sorted(resident, key=lambda q: (-self.recency[q], q))[:new_S])
        owner, recency = [None] * new_S, [-1] * new_S
        free = [p for p in range(new_S) if p not in kept]
        moves = []
        for q in kept:
            p = q if q < new_S else free.pop(0)
            owner[p], recency[p] = self.owner[q], self.recency[q]
            moves.append((q, p))
        self.S, self.owner, self.recency = new_S, owner, recency
        self.where = {key: p for p, key in enumerate(owner) if key is not None}
        return moves


class _LruWavesOfS(LR.LruSlots):
    def waves(self, layer, counts):
        # one staging set: waves as large as the pool
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        order = ([e for e in needed if (layer, e) in self.where]
                 + [e for e in needed if (layer, e) not in self.where])
        return [order[i:i + self.S] for i in range(0, len(order), self.S)]


class _LruWavesNotResidentFirst(LR.LruSlots):
    def waves(self, layer, counts):
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        if len(needed) <= self.S:
            return [needed] if needed else []
        size = max(1, self.S // 2)
        return [needed[i:i + size] for i in range(0, len(needed), size)]


class _LruHybridFetchesOldest(LR.LruSlots):
    def split_hybrid(self, layer, counts, fetch_fraction, max_fetch=-1):
        # fetch cap filled with the LEAST recently active misses
        counts = np.asarray(counts)
        needed = [int(e) for e in np.nonzero(counts > 0)[0]]
        misses = [e for e in needed if (layer, e) not in self.where]
        order = sorted(misses, key=lambda e: (self.last_active.get((layer, e), -1), e))
        n = int(np.ceil(fetch_fraction * len(misses)))
        if max_fetch >= 0:
            n = min(n, max_fetch)
        return order[:n], order[n:]


CASES = [
    ("e2m1 exponent bias", F, "e2m1_value", _e2m1_wrong_bias, lambda: T_fmt.test_e2m1_published_table()),
    ("nibble order", F, "unpack_e2m1", _unpack_swapped, lambda: T_fmt.test_nibble_order_low_first()),
    ("e4m3 bias 8 (FNUZ-style)", F, "e4m3_value", _e4m3_bias8, lambda: T_fmt.test_e4m3_landmarks_and_torch_cast()),
    ("tie-break to high index", R, "route", _route_high_index_ties, lambda: [T_rp.test_route_brute_force_tiny(s) for s in range(25)]),
    ("weights not renormalised", R, "route", _route_no_renorm_as_default, lambda: T_rp.test_route_two_expert_closed_form()),
    ("unstable permutation", P, "permute", _permute_unstable, lambda: [T_rp.test_permute_brute_force(s) for s in range(10)]),
    ("SiLU sign", FF, "silu", _silu_sign, lambda: T_ffn.test_silu_matches_torch()),
    ("combine weight order", C, "combine", _combine_reversed, lambda: T_ffn.test_combine_k1_and_one_hot()),
    ("gate/up swapped in decode", F, "decode_record", _decode_gate_up_swapped, lambda: test_bf16_record_gate_rows_first()),
    ("LRU evicts most recent", LR, "LruSlots", _LruMru, lambda: T_lru.test_hand_worked_trace()),
    ("resize keeps least recent", LR, "LruSlots", _LruResizeKeepsOldest,
     lambda: [T_lru.test_resize_single_expert_steps_match_textbook_lru(s) for s in range(8)]),
    ("resize does not pack", LR, "LruSlots", _LruResizeNoPacking,
     lambda: T_lru.test_resize_hand_worked()),
    ("waves as large as the pool", LR, "LruSlots", _LruWavesOfS,
     lambda: T_lru.test_waves_hand_worked_trace()),
    ("waves not resident-first", LR, "LruSlots", _LruWavesNotResidentFirst,
     lambda: T_lru.test_waves_hand_worked_trace()),
    ("hybrid fetches least active", LR, "LruSlots", _LruHybridFetchesOldest,
     lambda: T_lru.test_hybrid_hand_worked_trace()),
]


@pytest.mark.parametrize("name,mod,attr,bad,pin", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, mod, attr, bad, pin):
    # the pins import the oracle modules by name, so patching the module attribute
    # is what they see
    monkeypatch.setattr(C, "__wrapped_combine", C.combine, raising=False)
    monkeypatch.setattr(F, "__wrapped_decode", F.decode_record, raising=False)
    monkeypatch.setattr(mod, attr, bad)
    with pytest.raises(AssertionError):
        pin()
