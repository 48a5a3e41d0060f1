"""Pins for the shared expert ("Expert Parallelism", narrativegoldmine.com,
"Major Variants and Families", shared expert routing: one expert processes
every token in addition to the routed experts).

The shared expert is pinned against the routed path: with a single expert
(E = 1, k = 1, no drops) the router gives every token probability 1, so the
routed layer -- route, slots, layout, expert FFN, combine -- must produce the
shared expert's output for every token.  The combine's extra term and the
whole forward are checked as exact sums."""
import numpy as np
import pytest

import oracle


def _weights(rng, d, f, swiglu):
    W1 = rng.normal(scale=d ** -0.5, size=(1, d, f)).astype(np.float32)
    W3 = rng.normal(scale=d ** -0.5, size=(1, d, f)).astype(np.float32) if swiglu else None
    W2 = rng.normal(scale=f ** -0.5, size=(1, f, d)).astype(np.float32)
    return W1, W3, W2


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_shared_expert_is_the_expert_every_token_chooses(act):
    rng = np.random.default_rng(7)
    B, d, f = 23, 16, 24
    x = rng.normal(size=(B, d)).astype(np.float32)
    W1, W3, W2 = _weights(rng, d, f, act == "swiglu")
    Wg = rng.normal(size=(d, 1)).astype(np.float32)
    routed = oracle.forward(x, Wg, None, W1, W3, W2, k=1, c=1.0, act=act)
    assert routed["keep"].all() and np.all(routed["w"] == 1.0)
    sh = oracle.shared_ffn(x, W1[0], W2[0], None if W3 is None else W3[0], act)
    np.testing.assert_allclose(sh, routed["y"], rtol=1e-12, atol=1e-14)
    # a token subset selects the same rows
    tok = np.array([3, 0, 22])
    np.testing.assert_array_equal(
        oracle.shared_ffn(x, W1[0], W2[0], None if W3 is None else W3[0], act, tokens=tok),
        sh[tok])


def test_forward_adds_the_shared_output_to_every_token():
    rng = np.random.default_rng(3)
    B, d, f, E = 40, 16, 24, 6
    x = rng.normal(size=(B, d)).astype(np.float32)
    Wg = rng.normal(size=(d, E)).astype(np.float32)
    W1 = rng.normal(scale=0.25, size=(E, d, f)).astype(np.float32)
    W2 = rng.normal(scale=0.2, size=(E, f, d)).astype(np.float32)
    S1, _, S2 = _weights(rng, d, f, False)
    base = oracle.forward(x, Wg, None, W1, None, W2, k=2, c=0.75, act="gelu", C=2)
    with_sh = oracle.forward(x, Wg, None, W1, None, W2, k=2, c=0.75, act="gelu", C=2,
                             shared=(S1[0], None, S2[0]))
    np.testing.assert_array_equal(with_sh["shared_out"],
                                  oracle.shared_ffn(x, S1[0], S2[0], None, "gelu"))
    np.testing.assert_allclose(with_sh["y"], base["y"] + with_sh["shared_out"], rtol=0,
                               atol=1e-15)
    # tokens whose routed choices were all dropped get exactly the shared output
    gone = ~base["keep"].any(axis=1)
    assert gone.any()
    np.testing.assert_array_equal(with_sh["y"][gone], with_sh["shared_out"][gone])
