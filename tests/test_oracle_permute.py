"""Pins for the oracle's permutation: brute-force grouping and invariants."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import permute


def _brute(idx, E):
    flat = [int(v) for v in np.asarray(idx).ravel()]
    counts = [0] * E
    for v in flat:
        counts[v] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    sorted_src = []
    for e in range(E):
        for q, v in enumerate(flat):
            if v == e:
                sorted_src.append(q)
    return counts, offsets, sorted_src


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (5, 3, 3), (33, 17, 4), (7, 256, 8)])
def test_permute_brute_force(T, E, k, rng):
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_src, dest_row = permute(idx, E)
    bc, bo, bs = _brute(idx, E)
    assert counts.tolist() == bc
    assert offsets.tolist() == bo
    assert sorted_src.tolist() == bs
    assert offsets[-1] == T * k
    # bijection and inverse
    assert sorted(sorted_src.tolist()) == list(range(T * k))
    for q in range(T * k):
        assert sorted_src[dest_row[q]] == q


def test_permute_empty_experts_and_skew():
    idx = np.array([[3, 0], [3, 1], [3, 0]], dtype=np.int32)
    counts, offsets, sorted_src, dest_row = permute(idx, 6)
    assert counts.tolist() == [2, 1, 0, 3, 0, 0]
    assert offsets.tolist() == [0, 2, 3, 3, 6, 6, 6]
    assert sorted_src.tolist() == [1, 5, 3, 0, 2, 4]
    assert dest_row.tolist() == [3, 0, 4, 2, 5, 1]


@settings(max_examples=80, deadline=None)
@given(st.integers(1, 12), st.integers(1, 9), st.data())
def test_permute_invariants(T, E, data):
    k = data.draw(st.integers(1, E))
    rows = [data.draw(st.permutations(range(E)))[:k] for _ in range(T)]
    idx = np.array(rows, dtype=np.int32)
    counts, offsets, sorted_src, dest_row = permute(idx, E)
    key = idx.ravel()
    assert counts.sum() == T * k
    assert np.all(np.diff(key[sorted_src]) >= 0)            # grouped by expert
    for e in range(E):
        seg = sorted_src[offsets[e]:offsets[e + 1]]
        assert np.all(key[seg] == e)
        assert np.all(np.diff(seg) > 0)                     # stable
    assert np.array_equal(np.sort(sorted_src), np.arange(T * k))
    assert np.array_equal(sorted_src[dest_row], np.arange(T * k))
