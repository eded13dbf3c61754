"""Pins for the oracle's top-k routing and token-by-expert permutation (no GPU)."""

import numpy as np
import pytest

from oracle import route, permute


def _select_loop(row, k):
    """k rounds of 'largest remaining logit, lowest id on ties' (plain loop)."""
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (5, 5), (128, 8)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    logits = rng.integers(-3, 4, size=(40, E)).astype(np.float32)  # many exact ties
    logits[0] = 0.0  # every logit tied
    logits[1, :] = -0.0
    idx, w = route(logits, k)
    for t in range(logits.shape[0]):
        assert list(idx[t]) == _select_loop(logits[t], k)


def test_weights_are_softmax_topk_renormalized():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((64, 16)).astype(np.float32) * 3
    idx, w = route(logits, 4)
    full = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    ref = sel / sel.sum(1, keepdims=True)
    assert np.max(np.abs(w - ref)) <= 1e-12
    assert np.max(np.abs(w.sum(1) - 1.0)) <= 1e-12
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_edge_cases():
    idx, w = route(np.zeros((0, 8), np.float32), 2)
    assert idx.shape == (0, 2) and w.shape == (0, 2)
    idx, w = route(np.array([[1.0, 2.0]], np.float32), 2)
    assert list(idx[0]) == [1, 0]
    with pytest.raises(ValueError):
        route(np.zeros((2, 4), np.float32), 5)
    with pytest.raises(ValueError):
        route(np.zeros((2, 4), np.float32), 0)


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (1, 128, 8), (300, 64, 8), (0, 4, 2)])
def test_permute_invariants(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) if T else np.zeros((0, k), int)
    counts, offsets, sp, pos = permute(idx, E)
    flat = idx.reshape(-1)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    for e in range(E):
        seg = sp[offsets[e] : offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)  # stable: ascending pair id
        assert len(seg) == np.sum(flat == e)
    assert np.array_equal(np.sort(sp), np.arange(T * k))
    assert np.array_equal(sp[pos], np.arange(T * k))
