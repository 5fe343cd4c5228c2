"""Pins of the oracle's router and permutation (CPU only)."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import permute as P
from oracle import route as R


def _better(l, a, b):
    """Explicit tie rule: higher logit wins, equal logits -> lower index wins."""
    return l[a] > l[b] or (l[a] == l[b] and a < b)


def _brute_topk(l, k):
    E = len(l)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(_better(l, a, b) for a in S for b in rest):
            winners.append(S)
    assert len(winners) == 1              # exactly one dominating subset
    S = list(winners[0])
    # order inside the subset: insertion sort with the explicit rule
    out = []
    for e in S:
        i = 0
        while i < len(out) and _better(l, out[i], e):
            i += 1
        out.insert(i, e)
    return out


@pytest.mark.parametrize("seed", range(25))
def test_route_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    T, E = 4, int(rng.integers(1, 7))
    k = int(rng.integers(1, E + 1))
    # coarse values make ties common
    lg = (rng.integers(-2, 3, size=(T, E)) * 0.5).astype(np.float32)
    ids, w = R.route(lg, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(lg[t].astype(np.float64), k)


def test_route_two_expert_closed_form():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 9)).astype(np.float32)
    ids, w = R.route(lg, 2)
    l0 = lg[np.arange(50), ids[:, 0]].astype(np.float64)
    l1 = lg[np.arange(50), ids[:, 1]].astype(np.float64)
    assert np.allclose(w[:, 0], scipy.special.expit(l0 - l1), rtol=0, atol=1e-15)
    assert np.allclose(w[:, 1], scipy.special.expit(l1 - l0), rtol=0, atol=1e-15)


def test_route_weights_match_scipy_softmax():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((40, 32)).astype(np.float32)
    ids, w = R.route(lg, 5, renorm=True)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), 1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), atol=1e-15)
    ids2, w2 = R.route(lg, 5, renorm=False)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w2, np.take_along_axis(full, ids.astype(np.int64), 1), atol=1e-15)


def test_route_invariants():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((64, 256)).astype(np.float32)
    ids, w = R.route(lg, 8)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    sel = np.take_along_axis(lg, ids.astype(np.int64), 1)
    assert np.all(np.diff(sel, axis=1) <= 0)


def test_route_special_cases():
    ids, w = R.route(np.array([[0.3]], np.float32), 1)
    assert ids.tolist() == [[0]] and w.tolist() == [[1.0]]
    ids, w = R.route(np.zeros((3, 7), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3 and np.allclose(w, 0.25)
    lg = np.array([[0.0, -0.0, -1.0, -0.0]], np.float32)   # -0.0 ties +0.0
    assert R.route(lg, 3)[0].tolist() == [[0, 1, 3]]
    lg = np.array([[-0.0, 0.0]], np.float32)
    assert R.route(lg, 1)[0].tolist() == [[0]]
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((5, 6)).astype(np.float32)
    ids, _ = R.route(lg, 6)                                # k = E: full ordering
    assert all(sorted(r) == list(range(6)) for r in ids.tolist())


def _brute_permute(ids, E):
    flat = ids.reshape(-1).tolist()
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    sorted_idx = [a for e in range(E) for a in range(len(flat)) if flat[a] == e]
    return counts, sorted_idx


@pytest.mark.parametrize("seed", range(10))
def test_permute_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E = int(rng.integers(1, 40)), int(rng.integers(1, 12))
    k = int(rng.integers(1, E + 1))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_idx, inv_idx = P.permute(ids, E)
    bc, bs = _brute_permute(ids, E)
    assert counts.tolist() == bc
    assert sorted_idx.tolist() == bs
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(sorted_idx[inv_idx], np.arange(T * k))
    assert np.array_equal(inv_idx[sorted_idx], np.arange(T * k))


def test_unpermute_permute_identity():
    rng = np.random.default_rng(11)
    T, E, k, H = 33, 9, 3, 5
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, sorted_idx, inv_idx = P.permute(ids, E)
    X = rng.standard_normal((T * k, H))
    Xp = X[sorted_idx]
    assert np.array_equal(P.unpermute(Xp, inv_idx), X)
    # gathered token rows in expert order
    x_tok = rng.standard_normal((T, H))
    g = P.gather_rows(x_tok, sorted_idx, k)
    assert np.array_equal(P.unpermute(g, inv_idx), np.repeat(x_tok, k, axis=0))


def test_permute_empty_and_degenerate():
    c, o, s, i = P.permute(np.zeros((0, 2), np.int32), 4)
    assert c.tolist() == [0, 0, 0, 0] and o.tolist() == [0] * 5 and s.size == 0 and i.size == 0
    c, o, s, i = P.permute(np.full((5, 1), 2, np.int32), 3)   # every token to one expert
    assert c.tolist() == [0, 0, 5] and s.tolist() == [0, 1, 2, 3, 4]
