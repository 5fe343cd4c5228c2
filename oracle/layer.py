"""Whole-layer forward (oracle): route -> permute -> expert FFN -> combine.

Composes the step definitions of this package exactly in the order the layer
runs them; see each module for the reading it follows.  `forward_tokens`
evaluates the same definition for a chosen subset of tokens only (each token's
output depends on its own logits and activations and on the weights alone),
which is how outputs of full-size workloads are checked one by one.
"""
from __future__ import annotations

import numpy as np

from . import combine as _combine
from . import ffn as _ffn
from . import formats as _formats
from . import permute as _permute
from . import route as _route


class ExpertSet:
    """Expert records as bytes: rec(e) -> uint8 record of expert e."""

    def __init__(self, fmt: str, H: int, I: int, rec):
        self.fmt, self.H, self.I, self._rec = fmt, H, I, rec
        self._cache = {}

    def weights(self, e: int):
        if e not in self._cache:
            self._cache[e] = _formats.decode_record(self._rec(e), self.fmt, self.H, self.I)
        return self._cache[e]

    def drop(self):
        self._cache.clear()


def forward(logits, x_bits, k: int, experts: ExpertSet, shared: ExpertSet | None = None,
            renorm: bool = True) -> dict:
    """Full layer; returns every intermediate (float64 where floating point)."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    x = _formats.bf16_value(x_bits)
    ids, w = _route.route(lg, k, renorm)
    counts, offsets, sorted_idx, inv_idx = _permute.permute(ids, E)
    y_perm = _ffn.expert_ffn(x, k, offsets, sorted_idx, experts.weights)
    y_shared = None
    if shared is not None:
        y_shared = _ffn.swiglu(x, *shared.weights(0))
    y = _combine.combine(y_perm, inv_idx, w, T, k, y_shared)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_idx=sorted_idx,
                inv_idx=inv_idx, y_perm=y_perm, y_shared=y_shared, y=y)


def forward_tokens(logits, x_bits, k: int, experts: ExpertSet, tokens,
                   shared: ExpertSet | None = None, renorm: bool = True) -> dict:
    """Layer output for the listed tokens only: y[t] = sum_j w_tj FFN_{e_tj}(x_t) (+ shared)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    lg = np.asarray(logits, dtype=np.float32)[tokens]
    x = _formats.bf16_value(np.asarray(x_bits)[tokens])
    ids, w = _route.route(lg, k, renorm)
    H = x.shape[1]
    y = np.zeros((len(tokens), H))
    for i in range(len(tokens)):
        for j in range(k):
            y[i] += w[i, j] * _ffn.swiglu(x[i:i + 1], *experts.weights(int(ids[i, j])))[0]
    if shared is not None:
        y += _ffn.swiglu(x, *shared.weights(0))
    return dict(tokens=tokens, ids=ids, w=w, y=y)
