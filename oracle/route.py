"""Router: top-k experts per token with renormalised softmax weights (oracle).

The pages state that each token of an MoE layer activates only a few experts
(FreeToken supported-models guide, section "MoE strategies"; the aitujian
feature article speaks of "activated experts") but give no router formula.
Plainest reading, taken here:

  * experts are ordered by (logit descending, expert index ascending), with
    -0.0 equal to +0.0; the first k are the token's experts, in that order;
  * weights are the softmax restricted to the k selected logits, i.e. the full
    softmax renormalised over the selection:
        w[t,j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0);
  * without renormalisation (kept for completeness), the full softmax values
    of the selected experts.

Selecting on logits equals selecting on softmax probabilities (softmax is
strictly increasing), and avoids ties that rounding of exp() could create.

Parity: pinned by brute-force enumeration of k-subsets on tiny inputs, the
two-expert closed form w0 = sigmoid(l0 - l1), scipy's softmax, and invariants.
"""
from __future__ import annotations

import numpy as np


def route(logits: np.ndarray, k: int, renorm: bool = True):
    """logits fp32 [T,E] -> (ids int32 [T,k], weights float64 [T,k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    l64 = lg.astype(np.float64)
    order = np.argsort(-l64, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l64, ids.astype(np.int64), axis=1)
    if renorm:
        z = np.exp(sel - sel[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    else:
        m = l64.max(axis=1, keepdims=True)
        w = np.exp(sel - m) / np.exp(l64 - m).sum(axis=1, keepdims=True)
    return ids, w
