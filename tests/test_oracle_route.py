"""Pins for the oracle's router logits, top-k selection and gate weights."""
import math

import numpy as np
import pytest


def bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest even (numpy only)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_logits_match_numpy_matmul(orc, dt):
    rng = np.random.default_rng(1)
    T, d, E = 37, 96, 11
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    if dt == "bf16":
        x, w = bf16_bits(x), bf16_bits(w)
        xf, wf = bits_to_f64(x), bits_to_f64(w)
    else:
        xf, wf = x.astype(np.float64), w.astype(np.float64)
    lg, ad = orc.router_logits(x, w, bias)
    ref = xf @ wf.T + bias.astype(np.float64)
    np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ad, np.abs(xf) @ np.abs(wf).T, rtol=1e-12)
    lg0, _ = orc.router_logits(x, w, None)
    np.testing.assert_allclose(lg0, xf @ wf.T, rtol=1e-12, atol=1e-12)


def brute_topk(l, k):
    E = len(l)
    return sorted(range(E), key=lambda e: (-float(l[e]), e))[:k]


@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (5, 2), (8, 2), (8, 8), (33, 4), (256, 8)])
def test_selection_brute_force_with_ties(orc, E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 64
    # values from a small set: many exact ties, including -0.0 vs +0.0
    pool = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 3.0], dtype=np.float32)
    lg = rng.choice(pool, size=(T, E)).astype(np.float32)
    idx, _ = orc.topk(lg, k)
    for t in range(T):
        assert list(idx[t]) == brute_topk(lg[t], k), t


def test_selection_matches_lexsort_on_random(orc):
    rng = np.random.default_rng(3)
    T, E, k = 200, 64, 64
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, 5] = lg[:, 9]  # forced ties
    idx, _ = orc.topk(lg, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))
        np.testing.assert_array_equal(idx[t], order)


def test_all_equal_logits(orc):
    T, E, k = 5, 16, 4
    lg = np.full((T, E), 0.7, dtype=np.float32)
    idx, w = orc.topk(lg, k)
    assert (idx == np.arange(k)).all()
    np.testing.assert_allclose(w, 1.0 / E, rtol=1e-15)


def test_two_experts_is_logistic(orc):
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((50, 2)).astype(np.float32) * 3
    idx, w = orc.topk(lg, 1)
    for t in range(50):
        sel, other = idx[t, 0], 1 - idx[t, 0]
        delta = float(lg[t, sel]) - float(lg[t, other])
        assert delta >= 0
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(-delta))) < 1e-15


def test_weights_are_selected_softmax_probabilities(orc):
    rng = np.random.default_rng(9)
    T, E, k = 40, 12, 3
    lg = rng.standard_normal((T, E)).astype(np.float32) * 2
    idx, w = orc.topk(lg, k)
    _, wall = orc.topk(lg, E)  # k = E: every probability, in selection order
    assert np.allclose(wall.sum(axis=1), 1.0, atol=1e-14)
    for t in range(T):
        p = dict(zip(orc.topk(lg[t:t + 1], E)[0][0], wall[t]))
        for j in range(k):
            assert w[t, j] == p[idx[t, j]]
        assert all(w[t, j] >= w[t, j + 1] for j in range(k - 1))
    # raw probabilities do not sum to one at k < E
    assert (w.sum(axis=1) < 1.0).all()


def test_renorm_equals_softmax_over_selected_logits(orc):
    rng = np.random.default_rng(10)
    T, E, k = 30, 9, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, wr = orc.topk(lg, k, renorm=True)
    for t in range(T):
        sel = lg[t, idx[t]].astype(np.float64)
        ex = [math.exp(v - sel.max()) for v in sel]
        ref = [e / sum(ex) for e in ex]
        np.testing.assert_allclose(wr[t], ref, rtol=1e-13)
    # top-1 renormalised is exactly one
    _, w1 = orc.topk(lg, 1, renorm=True)
    assert (w1 == 1.0).all()
