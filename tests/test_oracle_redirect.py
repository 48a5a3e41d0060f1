"""Pins for overflow redirected to the next-best expert ("Expert
Parallelism", narrativegoldmine.com, "Components and Architecture": tokens
routed to a full expert are dropped or redirected to a secondary expert).

A sequential claim queue -- round 1 walks the top-k assignments in claim
order, then the dropped ones, again in claim order, each try the token's
next unused ranked expert -- against the oracle's rank-and-count
formulation; capacity, distinctness and monotonicity invariants; the drop
policy when nothing overflows; weights are the fallback expert's
probability."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


def _queue(ranked, k, E, C, mask):
    B, K2 = ranked.shape
    cap = [0 if mask[e] else C for e in range(E)]
    kept = [0] * E
    expert = [[int(ranked[t][j]) for j in range(k)] for t in range(B)]
    slot = [[-1] * k for _ in range(B)]
    keep = [[False] * k for _ in range(B)]
    for j in range(k):                      # round 1, claim order q = j*B + t
        for t in range(B):
            e = int(ranked[t][j])
            if kept[e] < cap[e]:
                keep[t][j], slot[t][j] = True, kept[e]
                kept[e] += 1
    nxt = [k] * B                           # each token's next unused rank
    for j in range(k):                      # round 2, same order, dropped only
        for t in range(B):
            if keep[t][j]:
                continue
            r = nxt[t]
            nxt[t] += 1
            if r >= K2:
                continue
            e = int(ranked[t][r])
            if kept[e] < cap[e]:
                keep[t][j], slot[t][j], expert[t][j] = True, kept[e], e
                kept[e] += 1
    return np.array(expert), np.array(slot), np.array(keep, bool), np.array(kept)


@st.composite
def ranked_case(draw):
    B = draw(st.integers(0, 9))
    E = draw(st.integers(1, 7))
    k = draw(st.integers(1, E))
    K2 = min(2 * k, E)
    rows = [draw(st.permutations(list(range(E))))[:K2] for _ in range(B)]
    ranked = np.array(rows, dtype=np.int32).reshape(B, K2)
    C = draw(st.integers(0, B * k + 1))
    mask = np.array(draw(st.lists(st.booleans(), min_size=E, max_size=E)), bool)
    return ranked, k, E, C, mask


@settings(max_examples=300, deadline=None)
@given(ranked_case())
def test_redirect_matches_sequential_queue(case):
    ranked, k, E, C, mask = case
    B = ranked.shape[0]
    expert, rank, slot, keep, load, count = oracle.assign_slots_redirect(ranked, k, E, C, mask)
    qe, qs, qk, qc = _queue(ranked, k, E, C, mask)
    np.testing.assert_array_equal(keep, qk.reshape(B, k))
    np.testing.assert_array_equal(count, qc)
    np.testing.assert_array_equal(slot[keep], qs.reshape(B, k)[keep])
    np.testing.assert_array_equal(expert[keep], qe.reshape(B, k)[keep])
    assert (count <= C).all() and (count[mask] == 0).all()
    for t in range(B):                      # a token's kept experts are distinct
        ex = expert[t][keep[t]]
        assert len(set(ex.tolist())) == ex.size
        assert all(ranked[t][rank[t][j]] == expert[t][j] for j in range(k) if keep[t][j])
    # never fewer kept than dropping the overflow
    _, keep0, _, _ = oracle.assign_slots(ranked[:, :k], E, C, mask)
    assert keep.sum() >= keep0.sum()


def test_no_overflow_means_the_drop_policy():
    rng = np.random.default_rng(4)
    logits = rng.normal(size=(30, 8)).astype(np.float32)
    x = rng.normal(size=(30, 8)).astype(np.float32)
    a = oracle.forward(x, None, None, None, None, None, k=2, c=4.0, act="gelu", logits=logits)
    b = oracle.forward(x, None, None, None, None, None, k=2, c=4.0, act="gelu", logits=logits,
                       overflow="next")
    assert a["keep"].all()
    for key in ("idx", "pos", "keep", "dest", "expert_offset", "pack_src"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_redirected_weights_are_the_fallback_probabilities():
    rng = np.random.default_rng(6)
    logits = rng.normal(size=(40, 6)).astype(np.float32)
    logits[:, :2] += 3.0          # two hot experts overflow, the others have room
    x = rng.normal(size=(40, 8)).astype(np.float32)
    r = oracle.forward(x, None, None, None, None, None, k=2, c=1.0, act="gelu", logits=logits,
                       overflow="next")
    p = oracle.softmax(logits)
    moved = r["keep"] & (r["idx"] != oracle.route(logits, 2)[0])
    assert moved.any()
    t, j = np.nonzero(moved)
    np.testing.assert_array_equal(r["w"][t, j], p[t, r["idx"][t, j]])
    # the layout counts both rounds
    np.testing.assert_array_equal(np.diff(r["expert_offset"]), r["expert_count"])
