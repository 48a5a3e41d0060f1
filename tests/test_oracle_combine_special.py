"""Pins for the combine step and the remaining special cases.

Combine: "Expert Parallelism" (narrativegoldmine.com), "Components and
Architecture": the k outputs are weighted by the gating probabilities and
summed.  Without drops this is the dense soft-gated mixture restricted to the
top-k, computed here densely over all experts with an independent library
(torch float64) -- no gather, no scatter, no slots."""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import f32_to_bf16_bits


def _dense_mixture(x, Wg, bias, W1, W3, W2, k, act):
    tx = torch.from_numpy(np.asarray(x, np.float32)).double()
    l = torch.from_numpy(oracle.gate_logits(x, Wg, bias)).double()
    p = torch.softmax(l, dim=1)
    E = p.shape[1]
    # top-k mask from a plain per-row sort (ties to lower index)
    G = torch.zeros_like(p)
    for t in range(p.shape[0]):
        order = sorted(range(E), key=lambda e: (-float(l[t, e]), e))[:k]
        G[t, order] = p[t, order]
    y = torch.zeros_like(tx)
    for e in range(E):
        h = tx @ torch.from_numpy(W1[e]).double()
        if act == "gelu":
            h = torch.nn.functional.gelu(h)
        else:
            h = torch.nn.functional.silu(h) * (tx @ torch.from_numpy(W3[e]).double())
        y += G[:, e:e + 1] * (h @ torch.from_numpy(W2[e]).double())
    return y.numpy()


@pytest.mark.parametrize("act,k", [("gelu", 2), ("swiglu", 3), ("gelu", 5)])
def test_no_drop_equals_dense_topk_mixture(act, k):
    rng = np.random.default_rng(13)
    B, d, f, E = 12, 8, 12, 5
    x = rng.standard_normal((B, d)).astype(np.float32)
    Wg = rng.standard_normal((d, E)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    W1 = rng.standard_normal((E, d, f)).astype(np.float32) / 3
    W3 = rng.standard_normal((E, d, f)).astype(np.float32) / 3
    W2 = rng.standard_normal((E, f, d)).astype(np.float32) / 3
    out = oracle.forward(x, Wg, bias, W1, W3 if act == "swiglu" else None, W2,
                         k=k, c=float(E), act=act)  # c = E -> C = B*k, no drops
    assert out["keep"].all()
    ref = _dense_mixture(x, Wg, bias, W1, W3, W2, k, act)
    # the oracle takes w at float32 precision: relative effect <= 2^-24
    np.testing.assert_allclose(out["y"], ref, rtol=1e-6, atol=1e-6)


def test_zero_capacity_gives_zero_output_and_residual_passthrough():
    rng = np.random.default_rng(17)
    B, d, f, E = 4, 8, 8, 3
    x = rng.standard_normal((B, d)).astype(np.float32)
    Wg = rng.standard_normal((d, E)).astype(np.float32)
    W1 = rng.standard_normal((E, d, f)).astype(np.float32)
    W2 = rng.standard_normal((E, f, d)).astype(np.float32)
    out = oracle.forward(x, Wg, None, W1, None, W2, k=2, c=1.0, act="gelu", C=0)
    assert (out["y"] == 0).all()
    out = oracle.forward(x, Wg, None, W1, None, W2, k=2, c=1.0, act="gelu", C=0,
                         add_residual=True)
    np.testing.assert_array_equal(out["y"], x.astype(np.float64))


def test_remote_rows_come_back_unchanged():
    """Experts outside [e_begin, e_end) return their packed rows (identity)."""
    rng = np.random.default_rng(19)
    B, d, f, E = 10, 8, 8, 4
    x = f32_to_bf16_bits(rng.standard_normal((B, d)).astype(np.float32))
    Wg = rng.standard_normal((d, E)).astype(np.float32)
    W1 = f32_to_bf16_bits(rng.standard_normal((2, d, f)).astype(np.float32))
    W2 = f32_to_bf16_bits(rng.standard_normal((2, f, d)).astype(np.float32))
    out = oracle.forward(x, Wg, None, W1, None, W2, k=2, c=4.0, act="gelu",
                         n_ranks=2, e_begin=0, e_end=2)
    eo = out["expert_offset"]
    xs = oracle.bf16_bits_to_f64(x)
    for r in range(eo[2], eo[4]):
        np.testing.assert_array_equal(out["ret"][r], xs[out["pack_src"][r]])


def test_placement_example():
    # 64 experts on 8 GPUs: expert 55 on GPU 6, expert 5 local to GPU 0
    assert oracle.rank_of_expert(55, 64, 8) == 6
    assert oracle.rank_of_expert(5, 64, 8) == 0


def test_active_fraction_example():
    # 128 experts, top-2 -> about 1.6 % of the expert parameters per token
    assert abs(2 / 128 - 0.016) < 0.001


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    cases = {
        1.0: 0x3F80,
        float(one + ulp / 2): 0x3F80,            # tie, kept part even -> down
        float(one + 3 * ulp / 2): 0x3F82,        # tie, kept part odd -> up
        float(one + ulp / 2 + 2.0 ** -20): 0x3F81,  # just above half -> up
        -2.5: 0xC020,
        0.0: 0x0000,
    }
    for v, bits in cases.items():
        assert int(oracle.f32_to_bf16_bits_rne(np.array([v], np.float32))[0]) == bits, v
    # agrees with torch's own conversion on random values
    rng = np.random.default_rng(23)
    a = (rng.standard_normal(10000) * 10).astype(np.float32)
    t = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_bits_rne(a), t)


@pytest.mark.parametrize("case", ["local", "remote_rows", "drops_residual"])
def test_combine_by_segment_equals_j_order_combine(case):
    """The memory-bounded combine (one expert segment at a time) gives the
    j-order combine's y up to float64 rounding."""
    rng = np.random.default_rng({"local": 23, "remote_rows": 29, "drops_residual": 31}[case])
    B, d, f, E, k = 40, 16, 24, 8, 3
    x = f32_to_bf16_bits(rng.standard_normal((B, d)).astype(np.float32))
    Wg = rng.standard_normal((d, E)).astype(np.float32)
    nl = 4 if case == "remote_rows" else E
    W1 = f32_to_bf16_bits((rng.standard_normal((nl, d, f)) / 4).astype(np.float32))
    W3 = f32_to_bf16_bits((rng.standard_normal((nl, d, f)) / 4).astype(np.float32))
    W2 = f32_to_bf16_bits((rng.standard_normal((nl, f, d)) / 5).astype(np.float32))
    kw = dict(k=k, c=0.5 if case == "drops_residual" else 4.0, act="swiglu",
              add_residual=case == "drops_residual")
    if case == "remote_rows":
        kw.update(n_ranks=2, e_begin=0, e_end=4)
    a = oracle.forward(x, Wg, None, W1, W3, W2, keep_ret=True, **kw)
    b = oracle.forward(x, Wg, None, W1, W3, W2, keep_ret=False, **kw)
    if case == "drops_residual":
        assert (~a["keep"]).any()
    assert "ret" not in b
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-13, atol=1e-13)
