"""Pins for the routing-health signals and the unavailable-expert mask.

"Expert Parallelism" (inferensys.com glossary), "Practitioner Guidance":
expert utilisation and routing entropy are health signals; "Risk and Threat
Considerations": an expert can become unavailable.  "Expert Parallelism"
(narrativegoldmine.com), "Components and Architecture": the Switch-form
auxiliary loss, here sum_e f_e P_e (token share times mean router
probability per expert); a full expert drops what it cannot take.  "Expert Parallelism" (theinfinity.ai), figure text: a bar is
the share of an expert's capacity in use.

The statistics are pinned by closed forms (equal logits, one-hot logits, a
perfectly balanced top-1 batch, a single hot expert, a two-expert softmax
with known probabilities); the mask by a claim queue that counts kept rows
per expert (a different formulation from the oracle's rank < capacity)."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _queue_kept(idx, E, C, unavailable):
    """Brute force: walk the assignments in claim order (all first choices in
    token order, then all second choices, ...); one is kept when its expert
    is available and has kept fewer than C so far."""
    B, k = idx.shape
    kept_so_far = [0] * E
    keep = [[False] * k for _ in range(B)]
    for j in range(k):
        for t in range(B):
            e = int(idx[t][j])
            if not unavailable[e] and kept_so_far[e] < C:
                keep[t][j] = True
                kept_so_far[e] += 1
    return np.array(keep, dtype=bool).reshape(B, k), np.array(kept_so_far)


@st.composite
def routed_masked(draw):
    B = draw(st.integers(0, 9))
    E = draw(st.integers(1, 7))
    k = draw(st.integers(1, E))
    rows = [draw(st.permutations(list(range(E))))[:k] for _ in range(B)]
    idx = np.array(rows, dtype=np.int32).reshape(B, k)
    C = draw(st.integers(0, B * k + 1))
    mask = np.array(draw(st.lists(st.booleans(), min_size=E, max_size=E)), dtype=bool)
    return idx, E, k, C, mask


@settings(max_examples=300, deadline=None)
@given(routed_masked())
def test_mask_matches_claim_queue(case):
    idx, E, k, C, mask = case
    B = idx.shape[0]
    pos, keep, load, count = oracle.assign_slots(idx, E, C, mask)
    qkeep, qkept = _queue_kept(idx, E, C, mask)
    np.testing.assert_array_equal(keep, qkeep)
    np.testing.assert_array_equal(count, qkept)
    assert (count[mask] == 0).all()
    # the layout gives masked experts empty segments and no rows
    eo, ro, dest, src = oracle.layout(idx, pos, keep, E, 1, C, mask)
    seg = np.diff(eo)
    np.testing.assert_array_equal(seg, count)
    assert (dest[np.isin(idx, np.flatnonzero(mask))] == -1).all()
    assert len(src) == int(keep.sum())
    # experts that are available keep exactly the slots they had unmasked
    pos0, keep0, _, _ = oracle.assign_slots(idx, E, C)
    np.testing.assert_array_equal(pos, pos0)
    avail = ~mask[idx] if B else np.zeros((0, k), bool)
    np.testing.assert_array_equal(keep[avail], keep0[avail])


def test_all_false_mask_changes_nothing():
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(40, 6)).astype(np.float32)
    x = rng.normal(size=(40, 8)).astype(np.float32)
    a = oracle.forward(x, None, None, None, None, None, k=2, c=1.0, act="gelu", logits=logits)
    b = oracle.forward(x, None, None, None, None, None, k=2, c=1.0, act="gelu", logits=logits,
                       unavailable=np.zeros(6, bool))
    for key in ("pos", "keep", "expert_count", "expert_offset", "dest", "pack_src"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_masked_expert_drops_everything_routed_to_it():
    # worked-example shape: 6 tokens, 8 experts, top-2, capacity 2
    rng = np.random.default_rng(0)
    logits = rng.normal(size=(6, 8)).astype(np.float32)
    idx, _ = oracle.route(logits, 2)
    hot = int(np.bincount(idx.reshape(-1), minlength=8).argmax())
    mask = np.zeros(8, bool)
    mask[hot] = True
    pos, keep, load, count = oracle.assign_slots(idx, 8, 2, mask)
    assert count[hot] == 0 and load[hot] > 0
    assert not keep[idx == hot].any()


def _stats(logits, idx, E, C, k, tau=1.0):
    _, _, load, count = oracle.assign_slots(idx, E, C)
    return oracle.routing_stats(logits, load, count, C, k, tau), load, count


@pytest.mark.parametrize("tau", [1.0, 0.5, 3.0])
def test_equal_logits_give_uniform_probability_and_log_E_entropy(tau):
    B, E, k = 12, 5, 2
    logits = np.full((B, E), 0.25, np.float32)
    idx, _ = oracle.route(logits, k, tau)
    s, _, _ = _stats(logits, idx, E, 3, k, tau)
    np.testing.assert_allclose(s["prob_mean"], np.full(E, 1 / E), rtol=1e-15)
    assert abs(s["entropy"] - math.log(E)) < 1e-14


def test_two_expert_softmax_entropy_closed_form():
    # logits (0, ln 3): p = (1/4, 3/4) for every token
    B = 7
    logits = np.tile(np.array([0.0, math.log(3.0)], np.float32), (B, 1))
    # the logit is the float32 nearest ln 3, so p is (1/4, 3/4) to ~1e-8
    l1 = float(np.float32(math.log(3.0)))
    p1 = math.exp(l1) / (1.0 + math.exp(l1))
    p0 = 1.0 - p1
    idx, _ = oracle.route(logits, 1)
    s, _, _ = _stats(logits, idx, 2, B, 1)
    expect = -(p0 * math.log(p0) + p1 * math.log(p1))
    assert abs(s["entropy"] - expect) < 1e-14
    assert abs(expect - (2 * math.log(2) - 0.75 * math.log(3))) < 1e-7  # (1/4, 3/4)
    np.testing.assert_allclose(s["prob_mean"], [p0, p1], rtol=1e-14)
    # every token picks expert 1: f = (0, 1), aux = P_1
    np.testing.assert_array_equal(s["token_frac"], [0.0, 1.0])
    assert abs(s["aux_loss"] - p1) < 1e-15
    assert s["load_entropy"] == 0.0


def test_balanced_top1_batch_gives_aux_one_over_E():
    # token t hot on expert t % E: f_e = 1/E, P_e -> 1/E, aux -> 1/E,
    # load entropy ln E, routing entropy -> 0
    E, m = 8, 5
    B = E * m
    logits = np.zeros((B, E), np.float32)
    logits[np.arange(B), np.arange(B) % E] = 200.0
    idx, _ = oracle.route(logits, 1)
    s, load, count = _stats(logits, idx, E, m, 1)
    np.testing.assert_array_equal(s["token_frac"], np.full(E, 1 / E))
    np.testing.assert_allclose(s["prob_mean"], np.full(E, 1 / E), rtol=1e-12)
    assert abs(s["aux_loss"] - 1 / E) < 1e-12
    assert abs(s["load_entropy"] - math.log(E)) < 1e-14
    assert s["entropy"] < 1e-60
    np.testing.assert_array_equal(s["utilization"], np.ones(E))  # C = m: every expert full
    np.testing.assert_array_equal(s["dropped"], np.zeros(E))


def test_single_hot_expert_overflow_and_utilization():
    # all B tokens choose expert 2 first (k = 2): the page's overflow
    # max(0, n_e - C) is what is dropped, the bar of expert 2 is full
    B, E, k, C = 10, 4, 2, 3
    logits = np.zeros((B, E), np.float32)
    logits[:, 2] = 50.0
    logits[:, 0] = 10.0
    idx, _ = oracle.route(logits, k)
    s, load, count = _stats(logits, idx, E, C, k)
    np.testing.assert_array_equal(load, [B, 0, B, 0])
    np.testing.assert_array_equal(s["dropped"], np.maximum(0, load - C))
    np.testing.assert_array_equal(s["utilization"], [1.0, 0.0, 1.0, 0.0])
    np.testing.assert_array_equal(s["token_frac"], [1.0, 0.0, 1.0, 0.0])
    assert abs(s["load_entropy"] - math.log(2)) < 1e-15
    assert abs(s["aux_loss"] - (s["prob_mean"][0] + s["prob_mean"][2])) < 1e-15
    assert abs(s["prob_mean"].sum() - 1.0) < 1e-15


def test_empty_batch_statistics_are_zero():
    s = oracle.routing_stats(np.zeros((0, 6), np.float32), np.zeros(6, np.int32),
                             np.zeros(6, np.int32), 0, 2)
    assert s["aux_loss"] == 0.0 and s["entropy"] == 0.0 and s["load_entropy"] == 0.0
    assert not s["prob_mean"].any() and not s["utilization"].any()
