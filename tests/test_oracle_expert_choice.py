"""Pins for expert-choice routing ("Expert Parallelism", narrativegoldmine.com,
"Major Variants and Families", expert choice routing: every expert picks its
top-C tokens of the batch, so every expert processes exactly C tokens while
a token may be picked by any number of experts).

* the choice against a rank-counting brute force: t is picked by e iff fewer
  than C tokens beat it (higher score, or equal score and lower index);
* exact balance and token-ordered rows;
* all-equal scores pick the first C tokens;
* C >= B: every expert takes every token and the layer is the dense soft
  mixture sum_e p_te E_e(x_t) of the textbook mixture of experts;
* a token no expert picks gets 0 (or its residual)."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


@st.composite
def scored(draw):
    B = draw(st.integers(1, 9))
    E = draw(st.integers(1, 5))
    # few distinct values, so that ties are common
    vals = draw(st.lists(st.sampled_from([0.0, 0.125, 0.25, 0.5, 0.75, 1.0]),
                         min_size=B * E, max_size=B * E))
    p = np.array(vals, np.float32).reshape(B, E)
    C = draw(st.integers(0, B + 2))
    return p, C


@settings(max_examples=300, deadline=None)
@given(scored())
def test_choice_matches_rank_counting(case):
    p, C = case
    B, E = p.shape
    Ce = min(C, B)
    sel, eo, src, pw = oracle.expert_choice(p, C)
    np.testing.assert_array_equal(eo, np.arange(E + 1) * Ce)
    for e in range(E):
        picked = []
        for t in range(B):
            beat = sum(1 for u in range(B)
                       if p[u, e] > p[t, e] or (p[u, e] == p[t, e] and u < t))
            if beat < Ce:
                picked.append(t)
        assert len(picked) == Ce                      # balanced by construction
        for i, t in enumerate(picked):                # rows in token order
            assert sel[t, e] == e * Ce + i
            assert src[e * Ce + i] == t and pw[e * Ce + i] == p[t, e]
        others = sorted(set(range(B)) - set(picked))
        assert (sel[others, e] == -1).all()


def test_equal_scores_pick_the_first_tokens():
    p = np.full((7, 3), 0.5, np.float32)
    sel, eo, src, pw = oracle.expert_choice(p, 4)
    for e in range(3):
        np.testing.assert_array_equal(src[e * 4:(e + 1) * 4], [0, 1, 2, 3])
    assert (sel[4:] == -1).all()


def _layer(rng, B, d, f, E, act):
    x = rng.normal(size=(B, d)).astype(np.float32)
    Wg = rng.normal(scale=0.7, size=(d, E)).astype(np.float32)
    W1 = rng.normal(scale=d ** -0.5, size=(E, d, f)).astype(np.float32)
    W3 = rng.normal(scale=d ** -0.5, size=(E, d, f)).astype(np.float32) if act == "swiglu" else None
    W2 = rng.normal(scale=f ** -0.5, size=(E, f, d)).astype(np.float32)
    return x, Wg, W1, W3, W2


def test_capacity_of_the_whole_batch_is_the_dense_soft_mixture():
    rng = np.random.default_rng(1)
    B, d, f, E = 12, 8, 16, 4
    x, Wg, W1, W3, W2 = _layer(rng, B, d, f, E, "swiglu")
    r = oracle.forward_expert_choice(x, Wg, None, W1, W3, W2, k=1, c=1.0, act="swiglu", C=B)
    assert (r["sel"] >= 0).all()
    p = oracle.softmax(oracle.gate_logits(x, Wg)).astype(np.float32).astype(np.float64)
    dense = sum(p[:, e:e + 1] * oracle.expert_mlp(x.astype(np.float64), W1[e], W2[e], W3[e],
                                                  "swiglu") for e in range(E))
    np.testing.assert_allclose(r["y"], dense, rtol=1e-12, atol=1e-13)


def test_unpicked_tokens_get_zero_or_the_residual():
    rng = np.random.default_rng(2)
    B, d, f, E = 20, 8, 16, 3
    x, Wg, W1, W3, W2 = _layer(rng, B, d, f, E, "gelu")
    r = oracle.forward_expert_choice(x, Wg, None, W1, None, W2, k=1, c=0.5, act="gelu")
    assert r["C"] == oracle.capacity(B, 1, E, 0.5)
    none = (r["sel"] < 0).all(axis=1)
    assert none.any()
    assert (r["y"][none] == 0).all()
    rr = oracle.forward_expert_choice(x, Wg, None, W1, None, W2, k=1, c=0.5, act="gelu",
                                      add_residual=True)
    np.testing.assert_array_equal(rr["y"][none], x[none].astype(np.float64))
