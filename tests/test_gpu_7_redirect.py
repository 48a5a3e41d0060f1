"""Overflow redirected to the next-best expert (moe_problem_t.overflow =
MOE_OVERFLOW_NEXT) through moe_forward, against the oracle run on the GPU's
own logits ("Expert Parallelism", narrativegoldmine.com, "Components and
Architecture": overflow tokens dropped or redirected to a secondary
expert).  Every integer output bit-exact -- final expert, slot, keep,
dest, counts, offsets, pack order -- the final weights within 1e-5, y
within 2e-2; both slot paths (fused count scan and separate scan), with
unavailable experts, and the skewed workload at full size (integer outputs
and weights)."""
import numpy as np
import pytest

import moe_synth
import oracle
from _helpers import (assert_bf16_close, assert_f32_close, packed_weights_for_gpu,
                      problem_for, say, to_dev, to_np)

pytestmark = pytest.mark.gpu

KEYS = ("pos", "dest", "expert_load", "expert_count", "expert_offset", "rank_offset")


def _check(w, inp, ref_y=True, mask=None):
    import torch
    import expert_token_routing_fp32_amd as moe
    kw = {}
    if mask is not None:
        kw["unavailable"] = torch.from_numpy(mask.astype(np.uint8)).cuda()
    p = problem_for(w, overflow="next", **kw)
    wp = packed_weights_for_gpu(p, inp)
    y, o = moe.forward(p, to_dev(inp["x"]), to_dev(inp["Wg"]),
                       None if inp["bias"] is None else to_dev(inp["bias"]), wp, outputs=True)
    logits = to_np(o["logits"])
    W = (inp["W1"], inp["W3"], inp["W2"]) if ref_y else (None, None, None)
    ref = oracle.forward(inp["x"], inp["Wg"], inp["bias"], *W, k=w.k, c=w.c, act=w.act,
                         n_ranks=w.n_ranks, e_begin=w.e_begin, e_end=w.e_end, tau=w.tau,
                         logits=logits, unavailable=mask, overflow="next")
    np.testing.assert_array_equal(to_np(o["topk_idx"]), ref["idx"])
    for key in KEYS:
        np.testing.assert_array_equal(to_np(o[key]).reshape(np.shape(ref[key])), ref[key],
                                      err_msg=key)
    np.testing.assert_array_equal(to_np(o["keep"]).astype(bool), ref["keep"])
    K = int(ref["expert_offset"][-1])
    np.testing.assert_array_equal(to_np(o["pack_src"])[:K], ref["pack_src"])
    assert_f32_close(to_np(o["topk_w"]), ref["w"], what="final weights")
    drop = oracle.forward(inp["x"], inp["Wg"], inp["bias"], None, None, None, k=w.k, c=w.c,
                          act=w.act, tau=w.tau, logits=logits, unavailable=mask)
    say(f"  kept {int(ref['keep'].sum())} (dropping the overflow: {int(drop['keep'].sum())})")
    assert ref["keep"].sum() >= drop["keep"].sum()
    if ref_y:
        yg = to_np(y)
        got = oracle.bf16_bits_to_f64(yg) if yg.dtype == np.uint16 else yg.astype(np.float64)
        assert_bf16_close(got, ref["y"], what="forward y with redirects")


def _wl(**kw):
    base = dict(name="redirect", B=512, d=64, E=16, k=2, c=1.0, f=48, act="gelu",
                x_dtype="bf16", n_ranks=1, e_begin=0, e_end=None, router_std=None,
                zipf_bias=True, tau=1.0, seed=8)
    base.update(kw)
    if base["e_end"] is None:
        base["e_end"] = base["E"]
    return moe_synth.Workload(**base)


@pytest.mark.parametrize("kw", [dict(), dict(E=6, e_end=6, k=2, B=300),
                                dict(E=32, e_end=32, k=4, B=700, act="swiglu", f=40),
                                dict(E=8, e_end=8, k=8, B=200, c=0.5),
                                dict(E=1024, e_end=1024, n_ranks=1024, k=2, B=600)],
                         ids=["fused_scan", "separate_scan_E6", "k4_swiglu", "k_equals_E",
                              "E1024_D1024"])
def test_forward_redirect(kw):
    w = _wl(**kw)
    say(f"[redirect] {w}")
    _check(w, moe_synth.make_inputs(w))


def test_forward_redirect_with_unavailable_experts():
    w = _wl(name="redirect_mask", B=400, E=12, e_end=12, k=3)
    mask = np.zeros(12, bool)
    mask[[0, 5]] = True
    _check(w, moe_synth.make_inputs(w), mask=mask)


def test_forward_redirect_skewed_full_size():
    w = moe_synth.WORKLOADS["skewed"]
    say(f"[redirect skewed] {w}")
    _check(w, moe_synth.make_inputs(w), ref_y=False)
