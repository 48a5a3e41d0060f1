"""Pins for capacity-limited slot assignment and the packed layout.

Slot-major claim order (all first choices in token order, then second
choices, ...) is checked against a literal sequential claim queue; the
layout against the invariants that define it ("Expert Parallelism",
theinfinity.ai, capacity paragraph; "Expert Parallelism and the All-to-All
Bottleneck", sections "The Mechanism of Expert Parallelism" and "The
All-to-All Communication Pattern")."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


def _queue(idx, E, C):
    """Brute force: walk the assignments one at a time in claim order."""
    B, k = idx.shape
    cnt = [0] * E
    pos = [[0] * k for _ in range(B)]
    for j in range(k):
        for t in range(B):
            e = int(idx[t][j])
            pos[t][j] = cnt[e]
            cnt[e] += 1
    return pos, cnt


@st.composite
def routed(draw):
    B = draw(st.integers(0, 9))
    E = draw(st.integers(1, 7))
    k = draw(st.integers(1, E))
    D = draw(st.sampled_from([d for d in range(1, E + 1) if E % d == 0]))
    rows = []
    for _ in range(B):
        perm = draw(st.permutations(list(range(E))))
        rows.append(perm[:k])
    idx = np.array(rows, dtype=np.int32).reshape(B, k)
    C = draw(st.integers(0, B * k + 1))
    return idx, E, k, D, C


@settings(max_examples=300, deadline=None)
@given(routed())
def test_slots_match_claim_queue_and_invariants(case):
    idx, E, k, D, C = case
    B = idx.shape[0]
    pos, keep, load, count = oracle.assign_slots(idx, E, C)
    qpos, qcnt = _queue(idx, E, C)
    np.testing.assert_array_equal(pos, np.array(qpos, dtype=np.int32).reshape(B, k))
    np.testing.assert_array_equal(load, qcnt)
    np.testing.assert_array_equal(keep, pos < C)
    # I1-I4
    assert load.sum() == B * k
    assert (count <= C).all()
    np.testing.assert_array_equal(count, np.minimum(load, C))
    assert count.sum() + np.maximum(0, load - C).sum() == B * k
    # I5: at most k kept per token, experts distinct per token
    for t in range(B):
        assert len(set(idx[t].tolist())) == k
    # I10: no drops when C >= B*k
    if C >= B * k:
        assert keep.all()
    eo, ro, dest, ps = oracle.layout(idx, pos, keep, E, D, C)
    K = int(eo[-1])
    assert K == int(count.sum()) and len(ps) == K
    # I6: pack_src is a bijection onto kept assignments; dest lies in its segment
    seen = np.zeros(K, dtype=int)
    for t in range(B):
        for j in range(k):
            if keep[t, j]:
                r = dest[t, j]
                e = idx[t, j]
                assert eo[e] <= r < eo[e + 1]
                assert ps[r] == t
                seen[r] += 1
            else:
                assert dest[t, j] == -1
    assert (seen == 1).all()
    # I7: rows inside a segment are in claim order q = j*B + t
    qrow = np.full(K, -1)
    for t in range(B):
        for j in range(k):
            if keep[t, j]:
                qrow[dest[t, j]] = j * B + t
    for e in range(E):
        seg = qrow[eo[e]:eo[e + 1]]
        assert (np.diff(seg) > 0).all()
    # I8: rank offsets sample the expert offsets at rank boundaries
    np.testing.assert_array_equal(ro, [eo[r * (E // D)] for r in range(D + 1)])


def test_zero_capacity_drops_everything():
    idx = np.array([[0, 1], [1, 0], [2, 1]], dtype=np.int32)
    pos, keep, load, count = oracle.assign_slots(idx, 3, 0)
    assert not keep.any() and count.sum() == 0
    eo, ro, dest, ps = oracle.layout(idx, pos, keep, 3, 1, 0)
    assert (dest == -1).all() and len(ps) == 0 and (eo == 0).all()


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(3)
    x = rng.integers(0, 2 ** 16, size=(7, 8), dtype=np.uint16)
    x &= np.uint16(0x7F7F)  # finite bf16 patterns
    idx = np.array([[0, 1], [1, 2], [2, 0], [0, 2], [1, 0], [2, 1], [0, 1]], dtype=np.int32)
    C = 3
    pos, keep, load, count = oracle.assign_slots(idx, 3, C)
    eo, ro, dest, ps = oracle.layout(idx, pos, keep, 3, 1, C)
    packed = oracle.pack(x, ps)
    un = oracle.unpack(packed, dest)
    for t in range(7):
        for j in range(2):
            if keep[t, j]:
                np.testing.assert_array_equal(un[t, j], x[t])
            else:
                assert (un[t, j] == 0).all()
