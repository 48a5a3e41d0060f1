"""The worked example of "Expert Parallelism" (theinfinity.ai, figure under the
capacity paragraph): 6 tokens, 8 experts on 4 devices, top-2, capacity 2,
two assignments dropped, experts 1 and 8 (1-based) idle.

The page prints only those aggregates; tests/golden/worked_example.json
realises them with hand-made choices and hand-derived expected values."""
import json
import math
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixture():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        g = json.load(f)
    pb = g["printed_by_page"]
    B, E = pb["B"], pb["E"]
    logits = np.full((B, E), g["logit_other"], dtype=np.float32)
    for t, (a, b) in enumerate(g["choices_0based"]):
        logits[t, a] = g["logit_first"]
        logits[t, b] = g["logit_second"]
    return g, logits


def _run(g, logits):
    pb = g["printed_by_page"]
    B, E, k, D = pb["B"], pb["E"], pb["k"], pb["D"]
    C = oracle.capacity(B, k, E, g["capacity_factor"])
    idx, w = oracle.route(logits, k)
    pos, keep, load, count = oracle.assign_slots(idx, E, C)
    eo, ro, dest, ps = oracle.layout(idx, pos, keep, E, D, C)
    return C, idx, w, pos, keep, load, count, eo, ro, dest, ps


def test_page_aggregates():
    g, logits = _fixture()
    pb = g["printed_by_page"]
    C, idx, w, pos, keep, load, count, eo, ro, dest, ps = _run(g, logits)
    assert C == pb["capacity"]
    assert int((~keep).sum()) == pb["dropped"]
    idle = sorted(int(e) + 1 for e in np.nonzero(load == 0)[0])
    assert idle == pb["idle_experts_1based"]
    # every token wakes exactly its top-2
    assert idx.shape == (pb["B"], pb["k"])
    # no expert exceeds its capacity
    assert count.max() <= pb["capacity"]
    assert len(ro) == pb["D"] + 1


def test_hand_derived_values():
    g, logits = _fixture()
    ex = g["expected"]
    C, idx, w, pos, keep, load, count, eo, ro, dest, ps = _run(g, logits)
    np.testing.assert_array_equal(idx, np.array(g["choices_0based"]))
    np.testing.assert_array_equal(load, ex["expert_load"])
    np.testing.assert_array_equal(count, ex["expert_count"])
    np.testing.assert_array_equal(pos, ex["pos"])
    np.testing.assert_array_equal(eo, ex["expert_offset"])
    np.testing.assert_array_equal(ro, ex["rank_offset"])
    np.testing.assert_array_equal(dest, ex["dest"])
    np.testing.assert_array_equal(ps, ex["pack_src"])
    dropped = sorted([int(t), int(j)] for t, j in zip(*np.nonzero(~keep)))
    assert dropped == sorted(ex["dropped_assignments"])
    S = math.exp(3) + math.exp(2) + 6
    np.testing.assert_allclose(w[:, 0], math.exp(3) / S, rtol=0, atol=1e-15)
    np.testing.assert_allclose(w[:, 1], math.exp(2) / S, rtol=0, atol=1e-15)
    np.testing.assert_allclose(w[0], [ex["w_first_value"], ex["w_second_value"]],
                               rtol=0, atol=1e-10)


def test_fixture_discriminates_claim_order():
    """A plausible mistake -- token-major claim order -- must fail the
    fixture: it drops a different pair of assignments."""
    g, logits = _fixture()
    idx, _ = oracle.route(logits, 2)
    cnt = np.zeros(8, dtype=int)
    dropped = []
    for t in range(6):          # token-major: t outer, j inner (the mistake)
        for j in range(2):
            e = idx[t, j]
            if cnt[e] >= 2:
                dropped.append([t, j])
            cnt[e] += 1
    assert sorted(dropped) == sorted(g["expected"]["token_major_would_drop"])
    assert sorted(dropped) != sorted(g["expected"]["dropped_assignments"])
