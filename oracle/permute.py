"""Token -> expert permutation (oracle).

Each expert runs one product over the rows routed to it, so the (token, slot)
assignments are grouped by expert.  The pages imply per-expert row blocks (the
fork README's key customizations speak of a prefill MoE kernel for M >= 2048
rows) but define no order; the plainest deterministic reading is a stable
counting sort of the flat assignment index a = t*k + j by its expert:

  counts[e]      = #{a : ids.flat[a] == e}
  offsets        = exclusive prefix sum of counts, offsets[E] = T*k
  sorted_idx[p]  = the assignments in expert order, ascending a within each
                   expert (equivalently ascending token, since a token's k
                   experts are distinct)
  inv_idx[a]     = p such that sorted_idx[p] == a

Parity: pinned by an O(A*E) brute-force construction and invariants
(permutation, inverse, segment contents, unpermute(permute(X)) == X).
"""
from __future__ import annotations

import numpy as np


def permute(ids: np.ndarray, E: int):
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    A = flat.size
    if A and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_idx = np.argsort(flat, kind="stable").astype(np.int32)
    inv_idx = np.empty(A, dtype=np.int32)
    inv_idx[sorted_idx] = np.arange(A, dtype=np.int32)
    return counts, offsets, sorted_idx, inv_idx


def gather_rows(X: np.ndarray, sorted_idx: np.ndarray, k: int) -> np.ndarray:
    """Rows of X (one per token) in permuted order: row p is token sorted_idx[p] // k."""
    return np.asarray(X)[np.asarray(sorted_idx) // k]


def unpermute(Xp: np.ndarray, inv_idx: np.ndarray) -> np.ndarray:
    """Permuted rows back to flat-assignment order: out[a] = Xp[inv_idx[a]]."""
    return np.asarray(Xp)[np.asarray(inv_idx)]
