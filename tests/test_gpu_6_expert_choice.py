"""Expert-choice routing on the GPU against the oracle ("Expert Parallelism",
narrativegoldmine.com, "Major Variants and Families", expert choice routing:
every expert picks its top-C tokens of the batch).

* router probabilities (fp32, transposed) within 1e-6 of the float64 softmax;
* the choice, fed the oracle's float32 probabilities, bit-exact: rows,
  tokens, weights, offsets -- random scores, heavy ties, C = 0, C >= B, one
  expert, 256 experts x 32768 tokens (the EP-share shape);
* pack and combine fed the oracle's rows, y within 2e-2;
* the whole layer, with the choice compared on the GPU's own probabilities
  (a choice is a decision on float32 values; both sides take it on the
  same ones)."""
import numpy as np
import pytest

import moe_synth
import oracle
from _helpers import assert_bf16_close, packed_weights_for_gpu, problem_for, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _prob(B, E, k=2, c=1.0, C=-1, d=32, f=48, act="gelu", x_dtype="bf16"):
    import expert_token_routing_fp32_amd as moe
    return moe.make_problem(B=B, d=d, E=E, k=k, c=c, C=C, f=f, act=act, x_dtype=x_dtype)


def test_router_probs():
    import expert_token_routing_fp32_amd as moe
    rng = np.random.default_rng(0)
    for B, E in [(300, 8), (777, 300), (64, 1024)]:
        logits = (rng.normal(size=(B, E)) * 3).astype(np.float32)
        p = _prob(B, E)
        pt = to_np(moe.router_probs(p, to_dev(logits)))
        exp = oracle.softmax(logits)
        np.testing.assert_allclose(pt.T, exp, rtol=2e-6, atol=1e-9)


CHOICE_CASES = {
    "random": dict(B=1000, E=16, k=2, c=1.0, ties=False),
    "ties": dict(B=700, E=12, k=3, c=1.25, ties=True),
    "zero_capacity": dict(B=100, E=8, k=2, c=1.0, C=0, ties=False),
    "whole_batch": dict(B=90, E=6, k=6, c=1.0, ties=False),
    "one_expert": dict(B=333, E=1, k=1, c=0.5, ties=True),
    "ep_share_shape": dict(B=32768, E=256, k=8, c=1.25, ties=False),
    # past 36864 tokens the score column no longer fits in LDS and the
    # select reads it from global memory (the other kernel variant)
    "column_in_global": dict(B=40000, E=8, k=2, c=1.0, ties=False),
    "column_in_global_ties": dict(B=40000, E=8, k=2, c=1.0, ties=True),
}


@pytest.mark.parametrize("case", list(CHOICE_CASES))
def test_expert_choice_bit_exact(case):
    import expert_token_routing_fp32_amd as moe
    kw = dict(CHOICE_CASES[case])
    ties = kw.pop("ties")
    rng = np.random.default_rng(len(case))
    B, E = kw["B"], kw["E"]
    if ties:
        probs = rng.choice(np.array([0.0, 0.1, 0.25, 0.5], np.float32), size=(B, E))
    else:
        probs = oracle.router_probs((rng.normal(size=(B, E)) * 2).astype(np.float32))
    p = _prob(**kw)
    C = moe.problem_capacity(p)
    say(f"[choice {case}] B={B} E={E} C={C}")
    o = moe.expert_choice(p, to_dev(np.ascontiguousarray(probs.T)))
    sel, eo, src, pw = oracle.expert_choice(probs, C)
    R = E * min(C, B)
    np.testing.assert_array_equal(to_np(o["sel_t"]).T, sel)
    np.testing.assert_array_equal(to_np(o["expert_offset"]), eo)
    np.testing.assert_array_equal(to_np(o["pack_src"])[:R], src)
    np.testing.assert_array_equal(to_np(o["pack_w"])[:R], pw)


def test_pack_and_combine():
    import expert_token_routing_fp32_amd as moe
    rng = np.random.default_rng(3)
    B, E, d = 500, 10, 72
    x = oracle.f32_to_bf16_bits_rne(rng.normal(size=(B, d)).astype(np.float32))
    probs = oracle.router_probs((rng.normal(size=(B, E)) * 2).astype(np.float32))
    p = _prob(B, E, k=2, c=1.0, d=d)
    C = moe.problem_capacity(p)
    sel, eo, src, pw = oracle.expert_choice(probs, C)
    packed = moe.expert_choice_pack(p, to_dev(x), to_dev(src))
    np.testing.assert_array_equal(to_np(packed), oracle.pack(x, src))
    ret = oracle.f32_to_bf16_bits_rne(rng.normal(size=(src.size, d)).astype(np.float32))
    y = moe.expert_choice_combine(p, to_dev(ret), to_dev(np.ascontiguousarray(sel.T)),
                                  to_dev(pw))
    exp = oracle.expert_choice_combine(oracle.bf16_bits_to_f64(ret), sel, pw)
    assert_bf16_close(oracle.bf16_bits_to_f64(to_np(y)), exp, what="expert-choice combine")
    none = (sel < 0).all(axis=1)
    if none.any():
        assert (oracle.bf16_bits_to_f64(to_np(y))[none] == 0).all()


@pytest.mark.parametrize("act,x_dtype,res", [("gelu", "bf16", False), ("swiglu", "bf16", True),
                                             ("gelu", "f32", False)])
def test_forward_expert_choice(act, x_dtype, res):
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.Workload(name="ec", B=600, d=64, E=8, k=2, c=1.0, f=96, act=act,
                           x_dtype=x_dtype, n_ranks=1, e_begin=0, e_end=8, router_std=None,
                           zipf_bias=False, tau=1.0, seed=6)
    inp = moe_synth.make_inputs(w)
    p = problem_for(w, add_residual=res)
    wp = packed_weights_for_gpu(p, inp)
    y, o = moe.forward_expert_choice(p, to_dev(inp["x"]), to_dev(inp["Wg"]), None, wp,
                                     outputs=True)
    gprobs = to_np(o["probs_t"]).T.copy()
    ref = oracle.forward_expert_choice(inp["x"], inp["Wg"], None, inp["W1"], inp["W3"],
                                       inp["W2"], k=w.k, c=w.c, act=act, add_residual=res,
                                       probs=gprobs)
    np.testing.assert_allclose(gprobs, oracle.router_probs(ref["logits"]), rtol=2e-6, atol=1e-9)
    np.testing.assert_array_equal(to_np(o["sel_t"]).T, ref["sel"])
    np.testing.assert_array_equal(to_np(o["pack_src"]), ref["pack_src"])
    yg = to_np(y)
    got = oracle.bf16_bits_to_f64(yg) if yg.dtype == np.uint16 else yg.astype(np.float64)
    assert_bf16_close(got, ref["y"], what=f"expert-choice forward {act} {x_dtype}")
