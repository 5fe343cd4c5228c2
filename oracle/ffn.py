"""Per-expert SwiGLU FFN (oracle).

The pages name the expert MLP but not its activation; the model families the
supported-models guide lists are SwiGLU-MoE LLMs, so the plainest reading is
the gated SiLU MLP with no bias, clamp or output scaling:

  G = X W_g^T,  U = X W_u^T,  Hh = SiLU(G) * U,  SiLU(z) = z / (1 + e^-z),
  Y = Hh W_d^T

evaluated in float64 on exactly decoded weights, with no intermediate
rounding.  Rows of X for expert e are the token rows of its permuted segment.

Parity: pinned by (i) E=1,k=1 equal to a dense SwiGLU MLP written with
torch.nn.functional.silu, (ii) zero expert -> zero output, (iii) scaling W_d by
2 doubles Y exactly, (iv) a pure-Python scalar loop on tiny shapes.
"""
from __future__ import annotations

import numpy as np


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    G = X @ np.asarray(Wg, dtype=np.float64).T
    U = X @ np.asarray(Wu, dtype=np.float64).T
    return (silu(G) * U) @ np.asarray(Wd, dtype=np.float64).T


def expert_ffn(x_tokens: np.ndarray, k: int, offsets: np.ndarray, sorted_idx: np.ndarray,
               expert_weights, experts=None) -> np.ndarray:
    """Y_perm [A, H]: row p = FFN_e(x[token(p)]) for the expert e owning row p.

    expert_weights(e) -> (Wg, Wu, Wd) float64.  `experts` limits the work to a
    subset (rows of other experts are left as NaN)."""
    x = np.asarray(x_tokens, dtype=np.float64)
    A = int(offsets[-1])
    E = len(offsets) - 1
    H = x.shape[1]
    out = np.full((A, H), np.nan)
    todo = range(E) if experts is None else experts
    for e in todo:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        rows = x[np.asarray(sorted_idx[lo:hi]) // k]
        Wg, Wu, Wd = expert_weights(e)
        out[lo:hi] = swiglu(rows, Wg, Wu, Wd)
    return out
