"""Pins of the oracle's router and permutation against brute force with Python sorted()."""
import math

import numpy as np
import pytest

from oracle import routing as orr


def _brute_route(lg, k):
    T, E = lg.shape
    idx = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        row = [float(v) for v in lg[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        m = max(row)
        z = sum(math.exp(v - m) for v in row)
        idx[t] = order
        w[t] = [math.exp(row[e] - m) / z for e in order]
    return idx, w


@pytest.mark.parametrize("T,E,k", [(17, 8, 2), (40, 16, 8), (5, 4, 4), (1, 1, 1)])
def test_route_matches_brute_force_with_ties(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    lg = rng.integers(-3, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)  # many exact ties
    idx, w = orr.route(lg, k)
    bi, bw = _brute_route(lg, k)
    assert (idx == bi).all()
    assert np.allclose(w, bw, rtol=1e-13, atol=0)


def test_route_renorm_and_neg_inf():
    lg = np.array([[0.0, -np.inf, 1.0, 0.5]], dtype=np.float32)
    idx, w = orr.route(lg, 2)
    assert idx.tolist() == [[2, 3]]
    p = np.exp([0.0, 1.0, 0.5]) / np.exp([0.0, 1.0, 0.5]).sum()
    assert np.allclose(w[0], [p[1], p[2]])
    _, wr = orr.route(lg, 2, renorm=True)
    assert np.isclose(wr.sum(), 1.0)


@pytest.mark.parametrize("T,E,k", [(33, 8, 2), (64, 16, 4), (3, 64, 3), (0, 4, 2)])
def test_permute_matches_sorted(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) if T else np.zeros((0, k), int)
    perm, inv, off = orr.permute(idx, E)
    R = T * k
    pairs = sorted(range(R), key=lambda f: (int(idx.reshape(-1)[f]), f // k, f % k))
    assert perm.tolist() == pairs
    assert (inv[perm] == np.arange(R)).all()
    counts = [sum(1 for f in range(R) if idx.reshape(-1)[f] == e) for e in range(E)]
    assert off.tolist() == [0] + list(np.cumsum(counts))
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert (idx.reshape(-1)[seg] == e).all()
