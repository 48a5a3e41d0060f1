"""Pins for softmax and top-k selection.

"Expert Parallelism" (narrativegoldmine.com), "Formal Algorithm":
p_t = softmax(g_t / tau), e(t) = argmax p_t, w_t = p_{t,e(t)};
"Expert Parallelism" glossary (inferensys.com): top-k of the distribution.
"""
import itertools
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def test_softmax_closed_forms():
    l = np.array([[0.0, 0.0, 0.0, 0.0], [1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    p = oracle.softmax(l)
    np.testing.assert_allclose(p[0], 0.25, rtol=0, atol=1e-16)
    ez = [math.exp(v) for v in (1, 2, 3, 4)]
    np.testing.assert_allclose(p[1], [v / sum(ez) for v in ez], rtol=1e-15)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-15)
    # shift invariance and temperature
    np.testing.assert_allclose(oracle.softmax(l + 7.0), p, rtol=1e-14)
    pt = oracle.softmax(l, tau=2.0)
    ez2 = [math.exp(v / 2) for v in (1, 2, 3, 4)]
    np.testing.assert_allclose(pt[1], [v / sum(ez2) for v in ez2], rtol=1e-15)


def test_k1_is_argmax():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((50, 9)).astype(np.float32)
    l[3, 2] = l[3, 5] = l[3].max() + 1  # tie: lower index wins, like argmax
    idx, w = oracle.route(l, 1)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(l, axis=1))
    p = oracle.softmax(l)
    np.testing.assert_allclose(w[:, 0], p.max(axis=1), rtol=0, atol=0)


def test_k_equals_E_selects_all_in_order():
    l = np.array([[0.5, -1.0, 2.0, 0.5]], dtype=np.float32)
    idx, w = oracle.route(l, 4)
    assert idx.tolist() == [[2, 0, 3, 1]]
    np.testing.assert_allclose(w.sum(), 1.0, atol=1e-15)


def test_equal_logits_pick_lowest_indices():
    l = np.zeros((3, 10), dtype=np.float32)
    idx, w = oracle.route(l, 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 3
    np.testing.assert_allclose(w, 0.1, atol=1e-16)


def test_weights_not_renormalised():
    l = np.array([[3.0, 2.0, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    _, w = oracle.route(l, 2)
    assert w.sum() < 1.0
    S = math.exp(3) + math.exp(2) + 6
    np.testing.assert_allclose(w[0], [math.exp(3) / S, math.exp(2) / S], rtol=1e-15)


def test_signed_zero_is_a_tie():
    l = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    idx, _ = oracle.route(l, 1)
    assert idx[0, 0] == 0


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 6), st.integers(1, 7), st.data())
def test_brute_force_topk(B, E, data):
    """Against an exhaustive search: the chosen ordered tuple is the
    lexicographically best permutation of k distinct experts under the key
    (higher logit first, then lower index)."""
    k = data.draw(st.integers(1, E))
    vals = data.draw(st.lists(st.lists(st.sampled_from([-1.0, 0.0, 0.5, 1.0, 2.5]),
                                       min_size=E, max_size=E), min_size=B, max_size=B))
    l = np.array(vals, dtype=np.float32)
    idx, w = oracle.route(l, k)
    for t in range(B):
        best = None
        for perm in itertools.permutations(range(E), k):
            key = [(-float(l[t, e]), e) for e in perm]
            if best is None or key < best[0]:
                best = (key, perm)
        assert tuple(idx[t]) == best[1]
        # chosen set dominates the rest
        rest = [e for e in range(E) if e not in idx[t]]
        for e in rest:
            assert all((l[t, s] > l[t, e]) or (l[t, s] == l[t, e] and s < e) for s in idx[t])
        ex = [math.exp(float(v) - float(l[t].max())) for v in l[t]]
        for j in range(k):
            assert abs(w[t, j] - ex[idx[t, j]] / sum(ex)) < 1e-15
