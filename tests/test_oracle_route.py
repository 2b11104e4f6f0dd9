"""Pins for the oracle's router: top-k selection and renormalised weights.

Selection is checked against brute-force enumeration of every ordered k-tuple
of experts; weights against closed forms (k=1, k=2, equal logits) and against
scipy's softmax followed by renormalisation.
"""

import itertools
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import expit, softmax

from oracle import route, router_logits


def _brute_topk(l, k):
    """Largest ordered k-tuple under the slot key (logit desc, index asc)."""
    E = len(l)
    best = None
    for tup in itertools.permutations(range(E), k):
        key = tuple((l[i], -i) for i in tup)
        if best is None or key > best[0]:
            best = (key, tup)
    return list(best[1])


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (5, 3), (6, 2), (6, 6), (3, 3)])
def test_topk_matches_brute_force_with_ties(E, k, rng):
    for _ in range(40):
        # integer logits in {0..3} force ties; some -inf entries
        l = rng.integers(0, 4, size=E).astype(np.float32)
        l[rng.random(E) < 0.2] = -np.inf
        idx, _ = route(l[None, :], k)
        assert list(idx[0]) == _brute_topk(list(l), k)


def test_topk_exchange_property_random(rng):
    T, E, k = 64, 40, 7
    l = rng.normal(size=(T, E)).astype(np.float32)
    l[:, 5] = l[:, 9]  # exact ties at fp32
    idx, _ = route(l, k)
    for t in range(T):
        S = set(idx[t].tolist())
        for i in S:
            for j in range(E):
                if j in S:
                    continue
                assert l[t, i] > l[t, j] or (l[t, i] == l[t, j] and i < j)
        for a, b in zip(idx[t][:-1], idx[t][1:]):
            assert l[t, a] > l[t, b] or (l[t, a] == l[t, b] and a < b)


def test_signed_zero_is_a_tie():
    l = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    idx, w = route(l, 1)
    assert idx[0, 0] == 0
    l = np.array([[0.0, -0.0, -1.0]], dtype=np.float32)
    idx, w = route(l, 2)
    assert list(idx[0]) == [0, 1]
    assert w[0, 0] == w[0, 1] == 0.5


def test_weights_k1_is_one(rng):
    l = rng.normal(size=(10, 16)).astype(np.float32)
    _, w = route(l, 1)
    assert np.all(w == 1.0)


def test_weights_k2_sigmoid(rng):
    l = rng.normal(size=(20, 9)).astype(np.float32)
    idx, w = route(l, 2)
    a = l[np.arange(20), idx[:, 0]].astype(np.float64)
    b = l[np.arange(20), idx[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], expit(a - b), rtol=1e-14)
    np.testing.assert_allclose(w[:, 1], expit(b - a), rtol=1e-14)


def test_weights_equal_logits_uniform():
    l = np.full((3, 12), 0.75, dtype=np.float32)
    idx, w = route(l, 5)
    assert (idx == np.arange(5)).all()
    np.testing.assert_allclose(w, 0.2, rtol=0, atol=1e-16)


def test_weights_match_scipy_softmax_renormalised(rng):
    l = (rng.normal(size=(30, 64)) * 3).astype(np.float32)
    idx, w = route(l, 8)
    p = softmax(l.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_weights_shift_invariant(rng):
    l = rng.normal(size=(8, 32)).astype(np.float32)
    _, w1 = route(l, 4)
    _, w2 = route(l + np.float32(100.0), 4)  # shift keeps order for these values
    np.testing.assert_allclose(w1, w2, rtol=1e-5)


def test_neg_inf_selected_gets_zero_weight():
    l = np.array([[1.0, -np.inf, -np.inf, 0.0]], dtype=np.float32)
    idx, w = route(l, 3)
    assert list(idx[0]) == [0, 3, 1]
    assert w[0, 2] == 0.0
    np.testing.assert_allclose(w[0, :2], [expit(1.0), expit(-1.0)], rtol=1e-15)


def test_all_neg_inf_row_is_uniform():
    l = np.full((1, 6), -np.inf, dtype=np.float32)
    idx, w = route(l, 3)
    assert list(idx[0]) == [0, 1, 2]
    assert np.all(w == 1.0 / 3)


def test_nan_rejected():
    with pytest.raises(AssertionError):
        route(np.array([[0.0, np.nan]], dtype=np.float32), 1)


@settings(max_examples=60, deadline=None)
@given(st.integers(2, 7), st.data())
def test_topk_property(E, data):
    k = data.draw(st.integers(1, E))
    vals = data.draw(st.lists(st.sampled_from([-np.inf, -1.5, 0.0, 0.5, 2.0]), min_size=E, max_size=E))
    l = np.array(vals, dtype=np.float32)
    idx, w = route(l[None], k)
    assert list(idx[0]) == _brute_topk(vals, k)
    assert math.isclose(w.sum(), 1.0, rel_tol=1e-15)


def test_router_logits_one_hot_and_brute_force(rng):
    E, d = 5, 7
    w_r = rng.normal(size=(E, d))
    for i in range(d):
        x = np.zeros((1, d))
        x[0, i] = 1.0
        np.testing.assert_array_equal(router_logits(x, w_r)[0], w_r[:, i])
    xi = rng.integers(-3, 4, size=(3, d)).astype(np.float64)
    wi = rng.integers(-3, 4, size=(E, d)).astype(np.float64)
    brute = [[sum(xi[t, q] * wi[e, q] for q in range(d)) for e in range(E)] for t in range(3)]
    np.testing.assert_array_equal(router_logits(xi, wi), np.array(brute))
