"""Weighted combine of the k expert outputs of each token (oracle).

Plainest reading of the layer output (the pages give no formula):

  y[t] = sum_{j=0..k-1} w[t,j] * Y_perm[inv_idx[t*k + j]]  (+ y_shared[t])

summed in j order, float64, result kept unrounded.  The shared expert, when
present, is always on with weight 1.0 and no gate.

Parity: pinned by k=1 -> y = FFN_e(x), one-hot weights, and shared-only ->
dense MLP (tests).
"""
from __future__ import annotations

import numpy as np


def combine(y_perm: np.ndarray, inv_idx: np.ndarray, w: np.ndarray, T: int, k: int,
            y_shared: np.ndarray | None = None) -> np.ndarray:
    yp = np.asarray(y_perm, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(T, k)
    inv = np.asarray(inv_idx).reshape(T, k)
    y = np.zeros((T, yp.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * yp[inv[:, j]]
    if y_shared is not None:
        y += np.asarray(y_shared, dtype=np.float64)
    return y
