"""Pins for the capacity formula and the overflow identity.

"Expert Parallelism" (theinfinity.ai), capacity paragraph: C = ceil((B*k/D)*c)
and overflow = max(0, p*B*k - C); read per expert (E for D), which the worked
example's "capacity of 2" fixes.
"""
import math

import numpy as np
import pytest

import oracle
from moe_synth import WORKLOADS


def test_worked_example_capacity_is_two():
    # 6 tokens, 8 experts, top-2, capacity factor 1.25 -> the page's capacity 2
    assert oracle.capacity(6, 2, 8, 1.25) == 2


def test_per_device_reading_would_not_give_two():
    # documents why the per-expert reading is taken: with D = 4 devices the
    # printed per-device formula gives 4, not the page's 2
    assert math.ceil((6 * 2 / 4) * 1.25) == 4


@pytest.mark.parametrize("name,C", [("toy", 2), ("uniform", 160), ("mixtral", 2048),
                                    ("skewed", 256), ("ep_share", 1280)])
def test_workload_capacities(name, C):
    w = WORKLOADS[name]
    # closed form by hand: B*k/E is an exact mean load for all five workloads
    assert (w.B * w.k) % w.E == 0 or name == "toy"
    assert oracle.capacity(w.B, w.k, w.E, w.c) == C


def test_capacity_rounds_up_and_zero_batch():
    assert oracle.capacity(10, 1, 4, 1.0) == 3      # 2.5 -> 3
    assert oracle.capacity(8, 1, 4, 1.0) == 2       # exact
    assert oracle.capacity(0, 2, 8, 1.25) == 0


def test_uniform_mean_load_matches_page():
    # expected arrivals per expert under uniform routing are B*k/E (per device
    # B*k/D in the page; with one expert per device they coincide)
    B, k, E = 4096, 2, 64
    assert oracle.capacity(B, k, E, 1.0) == B * k // E


@pytest.mark.parametrize("seed", range(5))
def test_overflow_identity_per_expert(seed):
    # dropped_e = max(0, n_e - C): holds for any claim order, so it checks the
    # slot assignment independently of the slot-major rule
    rng = np.random.default_rng(seed)
    B, E, k = 200, 12, 3
    logits = rng.standard_normal((B, E)).astype(np.float32)
    logits[:, 0] += 1.5  # one hot expert
    idx, _ = oracle.route(logits, k)
    C = oracle.capacity(B, k, E, 1.0)
    pos, keep, load, count = oracle.assign_slots(idx, E, C)
    dropped = np.array([np.sum((idx == e) & ~keep) for e in range(E)])
    np.testing.assert_array_equal(dropped, np.maximum(0, load - C))
    np.testing.assert_array_equal(count, np.minimum(load, C))
    assert load.sum() == B * k
    assert count.sum() + dropped.sum() == B * k
