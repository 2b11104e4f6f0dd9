"""Pins for the oracle's expert FFN, combine and whole layer.

Closed-form worked example, reduction to a textbook SwiGLU MLP built from
torch's own ``silu``, the dense (every-expert) mixture, and invariants
(identical experts, zero input, linearity, token-permutation equivariance).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import combine, dense_layer, expert_ffn, layer, permute, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _experts(rng, E, d, f, sg=0.3, su=0.3, sd=0.3):
    wg = rng.normal(size=(E, f, d)) * sg
    wu = rng.normal(size=(E, f, d)) * su
    wd = rng.normal(size=(E, d, f)) * sd
    return wg, wu, wd


def _getter(wg, wu, wd):
    return lambda e: (wg[e], wu[e], wd[e])


def test_golden_two_expert_closed_form():
    with open(os.path.join(GOLDEN, "two_expert_closed_form.json")) as fh:
        g = json.load(fh)
    wg, wu, wd = (np.array(g[n]) for n in ("w_gate", "w_up", "w_down"))
    res = layer(np.array(g["x"]), np.array(g["logits"]), g["k"], _getter(wg, wu, wd))
    np.testing.assert_allclose(res["w"], g["expected_w"], rtol=1e-15)
    np.testing.assert_allclose(res["out"] / math.log(3.0), g["expected_out_over_ln3"], rtol=1e-14)


def test_k1_reduces_to_textbook_swiglu(rng):
    """With k=1 each token's output is its expert's SwiGLU MLP (weight 1)."""
    T, E, d, f = 9, 4, 12, 20
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f, 1.0, 1.0, 1.0)   # SiLU in its nonlinear range
    logits = rng.normal(size=(T, E)).astype(np.float32)
    res = layer(x, logits, 1, _getter(wg, wu, wd))
    for t in range(T):
        e = int(np.argmax(logits[t]))
        xt = torch.tensor(x[t], dtype=torch.float64)
        gate = torch.tensor(wg[e]) @ xt
        up = torch.tensor(wu[e]) @ xt
        ref = torch.tensor(wd[e]) @ (torch.nn.functional.silu(gate) * up)
        np.testing.assert_allclose(res["out"][t], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_experts_give_single_ffn_for_any_routing(rng):
    T, E, d, f, k = 10, 6, 8, 16, 3
    x = rng.normal(size=(T, d))
    g1, u1, d1 = _experts(rng, 1, d, f, 1.0, 1.0, 1.0)
    get = lambda e: (g1[0], u1[0], d1[0])
    logits = rng.normal(size=(T, E)).astype(np.float32)
    res = layer(x, logits, k, get)
    gate = x @ g1[0].T
    ref = (gate * torch.sigmoid(torch.tensor(gate)).numpy() * (x @ u1[0].T)) @ d1[0].T
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-13)


def test_zero_input_gives_zero(rng):
    T, E, d, f = 4, 5, 8, 8
    wg, wu, wd = _experts(rng, E, d, f)
    res = layer(np.zeros((T, d)), rng.normal(size=(T, E)).astype(np.float32), 2, _getter(wg, wu, wd))
    assert np.all(res["out"] == 0.0)


def test_linear_in_w_down_and_w_up(rng):
    T, E, d, f, k = 6, 5, 8, 12, 2
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f)
    wd2 = rng.normal(size=wd.shape)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    o1 = layer(x, logits, k, _getter(wg, wu, wd))["out"]
    o2 = layer(x, logits, k, _getter(wg, wu, wd2))["out"]
    o12 = layer(x, logits, k, _getter(wg, wu, wd + 2.5 * wd2))["out"]
    np.testing.assert_allclose(o12, o1 + 2.5 * o2, rtol=1e-11, atol=1e-12)
    o3 = layer(x, logits, k, _getter(wg, -3.0 * wu, wd))["out"]
    np.testing.assert_allclose(o3, -3.0 * o1, rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariance(rng):
    T, E, d, f, k = 11, 7, 8, 10, 3
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    perm = rng.permutation(T)
    o = layer(x, logits, k, _getter(wg, wu, wd))["out"]
    op = layer(x[perm], logits[perm], k, _getter(wg, wu, wd))["out"]
    np.testing.assert_allclose(op, o[perm], rtol=1e-13, atol=1e-14)


def test_k_equals_E_uniform_is_dense_mixture(rng):
    T, E, d, f = 5, 6, 8, 10
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f, 1.0, 1.0, 1.0)
    res = layer(x, np.zeros((T, E), dtype=np.float32), E, _getter(wg, wu, wd))
    ref = np.zeros((T, d))
    for e in range(E):
        gate = torch.tensor(x @ wg[e].T)
        ref += (torch.nn.functional.silu(gate).numpy() * (x @ wu[e].T)) @ wd[e].T / E
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (7, 5, 5), (3, 9, 1), (20, 16, 4)])
def test_sparse_equals_dense_formulation(T, E, k, rng):
    d, f = 8, 12
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    sparse = layer(x, logits, k, _getter(wg, wu, wd))["out"]
    dense = dense_layer(x, logits, k, _getter(wg, wu, wd))
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-13)


def test_expert_ffn_rows_follow_sorted_src(rng):
    T, E, d, f, k = 6, 4, 8, 8, 2
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f)
    idx, w = route(rng.normal(size=(T, E)).astype(np.float32), k)
    counts, offsets, sorted_src, dest_row = permute(idx, E)
    y = expert_ffn(x, offsets, sorted_src, k, _getter(wg, wu, wd))
    for r in range(T * k):
        q = sorted_src[r]
        t, j = divmod(int(q), k)
        e = int(idx[t, j])
        gate = x[t] @ wg[e].T
        h = gate / (1 + np.exp(-gate)) * (x[t] @ wu[e].T)
        np.testing.assert_allclose(y[r], wd[e] @ h, rtol=1e-12, atol=1e-14)
    out = combine(y, dest_row, w)
    for t in range(T):
        ref = sum(w[t, j] * y[dest_row[t * k + j]] for j in range(k))
        np.testing.assert_allclose(out[t], ref, rtol=1e-15)


def test_expert_getter_only_called_for_routed_experts(rng):
    T, E, d, f, k = 2, 64, 8, 8, 2
    x = rng.normal(size=(T, d))
    wg, wu, wd = _experts(rng, E, d, f)
    seen = []

    def get(e):
        seen.append(e)
        return wg[e], wu[e], wd[e]
    res = layer(x, rng.normal(size=(T, E)).astype(np.float32), k, get)
    assert sorted(seen) == sorted(set(res["idx"].ravel().tolist()))


# ------------------------------------------------- per-expert normalisation
def test_expert_norm_scale_invariance_and_unit_rms(rng):
    """With per-expert RMS normalisation the output does not change when an
    expert's output row is scaled by c > 0 (eps aside), and each normalised
    row has unit RMS; without it the combine is linear in the rows."""
    from oracle import EXPERT_NORM_EPS, combine
    T, k, d = 3, 4, 64
    y = rng.normal(size=(T * k, d)) * 10.0
    dest = rng.permutation(T * k)
    w = rng.dirichlet(np.ones(k), size=T)
    base = combine(y, dest, w, expert_norm=True)
    y2 = y.copy()
    y2[dest[5]] *= 7.0
    np.testing.assert_allclose(combine(y2, dest, w, expert_norm=True), base, rtol=0, atol=1e-7)
    assert not np.allclose(combine(y2, dest, w), combine(y, dest, w))
    # one slot with weight 1: the output is that row over its RMS
    one = combine(y[:1], np.array([0]), np.ones((1, 1)), expert_norm=True)
    rms = np.sqrt(np.mean(one ** 2))
    assert abs(rms - 1.0) < EXPERT_NORM_EPS
    np.testing.assert_allclose(one[0] * np.linalg.norm(y[0]) / np.sqrt(d), y[0], rtol=1e-8)


def test_expert_norm_eps_inside_the_root_and_zero_rows():
    """A constant row of value c with c^2 equal to eps maps to 1/sqrt(2)
    (eps inside the square root: c / sqrt(c^2 + eps)); a zero row stays zero."""
    from oracle import EXPERT_NORM_EPS, combine
    d = 96
    c = np.sqrt(EXPERT_NORM_EPS)
    y = np.stack([np.full(d, c), np.zeros(d), np.full(d, -3.0)])
    out = combine(y, np.array([0, 1, 2]), np.array([[1.0], [1.0], [0.5]]), expert_norm=True)
    np.testing.assert_allclose(out[0], np.full(d, 2 ** -0.5), rtol=1e-12)
    assert np.all(out[1] == 0.0)
    np.testing.assert_allclose(out[2], np.full(d, -0.5 * 3.0 / np.sqrt(9.0 + EXPERT_NORM_EPS)), rtol=1e-12)
