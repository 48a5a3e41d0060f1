"""Pins for the router logits and the expert MLP.

Logits: "Expert Parallelism" (narrativegoldmine.com), "Formal Algorithm":
g_t from the routing linear projection -- checked against exact rational dot
products.  Expert: "Components and Architecture", Expert GEMM, a standard
transformer MLP -- checked against textbook values and an independent
float64 library implementation (torch CPU)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from moe_synth import f32_to_bf16_bits


def _exact_logit(xrow, wcol, b):
    s = sum((Fraction(float(a)) * Fraction(float(w)) for a, w in zip(xrow, wcol)), Fraction(0))
    if b is not None:
        s += Fraction(float(b))
    return np.float32(float(s))  # exact -> nearest double -> float32


@pytest.mark.parametrize("bf16", [False, True])
def test_logits_are_rounded_exact_dot_products(bf16):
    rng = np.random.default_rng(5)
    B, d, E = 5, 24, 6
    xf = rng.standard_normal((B, d)).astype(np.float32)
    x = f32_to_bf16_bits(xf) if bf16 else xf
    xv = oracle.bf16_bits_to_f64(x) if bf16 else xf.astype(np.float64)
    Wg = (rng.standard_normal((d, E)) * 0.3).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    l = oracle.gate_logits(x, Wg, bias)
    assert l.dtype == np.float32
    for t in range(B):
        for e in range(E):
            ref = _exact_logit(xv[t], Wg[:, e], bias[e])
            # equal up to a double-rounding step that cannot occur at this size
            assert abs(float(l[t, e]) - float(ref)) <= float(np.spacing(np.abs(ref)))


def test_gelu_silu_textbook_values():
    # GELU(z) = z * Phi(z); Phi(1) = 0.8413447460685429 (normal table)
    z = np.array([0.0, 1.0, -1.0, 2.0])
    g = oracle.gelu(z)
    np.testing.assert_allclose(g, [0.0, 0.8413447460685429, -0.15865525393145707,
                                   2 * 0.9772498680518208], rtol=1e-15, atol=1e-16)
    s = oracle.silu(np.array([0.0, 1.0, -2.0]))
    np.testing.assert_allclose(s, [0.0, 1 / (1 + math.exp(-1)), -2 / (1 + math.exp(2))],
                               rtol=1e-15)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_expert_mlp_against_library(act):
    rng = np.random.default_rng(7)
    n, d, f = 9, 16, 40
    xr = rng.standard_normal((n, d))
    W1 = f32_to_bf16_bits(rng.standard_normal((d, f)).astype(np.float32) / 4)
    W3 = f32_to_bf16_bits(rng.standard_normal((d, f)).astype(np.float32) / 4)
    W2 = f32_to_bf16_bits(rng.standard_normal((f, d)).astype(np.float32) / 6)
    out = oracle.expert_mlp(xr, W1, W2, W3 if act == "swiglu" else None, act)
    # independent: torch float64, weights widened by torch's own bf16 type
    tw = lambda b: torch.from_numpy(b.astype(np.int16)).view(torch.bfloat16).double()
    tx = torch.from_numpy(xr)
    h = torch.matmul(tx, tw(W1))
    if act == "gelu":
        h = torch.nn.functional.gelu(h, approximate="none")
    else:
        h = torch.nn.functional.silu(h) * torch.matmul(tx, tw(W3))
    ref = torch.matmul(h, tw(W2)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_single_expert_reduces_to_plain_mlp():
    """E = 1, k = 1: p = 1, no drops at C >= B, so y is the MLP itself."""
    rng = np.random.default_rng(11)
    B, d, f = 6, 8, 16
    x = rng.standard_normal((B, d)).astype(np.float32)
    Wg = rng.standard_normal((d, 1)).astype(np.float32)
    W1 = rng.standard_normal((1, d, f)).astype(np.float32)
    W2 = rng.standard_normal((1, f, d)).astype(np.float32)
    out = oracle.forward(x, Wg, None, W1, None, W2, k=1, c=1.0, act="gelu")
    assert (out["w"] == 1.0).all()
    tx = torch.from_numpy(x).double()
    ref = torch.matmul(
        torch.nn.functional.gelu(torch.matmul(tx, torch.from_numpy(W1[0]).double())),
        torch.from_numpy(W2[0]).double()).numpy()
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
