"""The seeded input generators: deterministic, shaped like the workloads."""
import numpy as np

import moe_synth
from moe_synth import WORKLOADS, make_inputs, scaled


def test_deterministic_and_shapes():
    w = scaled(WORKLOADS["uniform"], B=64, d=32, f=48, E=8, e_end=8)
    a = make_inputs(w)
    b = make_inputs(w)
    for n in ("x", "Wg", "W1", "W2"):
        np.testing.assert_array_equal(a[n], b[n])
    assert a["x"].shape == (64, 32) and a["x"].dtype == np.uint16
    assert a["W1"].shape == (8, 32, 48) and a["W2"].shape == (8, 48, 32)
    assert a["W3"] is None


def test_expert_weights_independent_of_local_range():
    w = scaled(WORKLOADS["ep_share"], B=16, d=16, f=8, E=8, k=2, n_ranks=2, e_begin=0, e_end=4)
    full = make_inputs(scaled(w, e_end=8))
    part = make_inputs(scaled(w, e_begin=4, e_end=8))
    np.testing.assert_array_equal(full["W1"][4:], part["W1"])


def test_toy_keeps_fp32_and_rounded_copies():
    a = make_inputs(WORKLOADS["toy"])
    assert a["x"].dtype == np.float32 and a["x"].shape == (6, 16)
    assert a["W1"].shape == (8, 16, 32) and a["W1_bits"].dtype == np.uint16


def test_zipf_bias():
    b = moe_synth.zipf_bias(128)
    assert b[0] > b[1] > b[-1]
    p = np.exp(b / 1.5)
    np.testing.assert_allclose(p.sum(), 1.0, rtol=1e-5)
    np.testing.assert_allclose(p[0] / p[1], 2 ** 1.2, rtol=1e-5)
