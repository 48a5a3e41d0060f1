"""Unavailable-expert mask and routing-health signals on the GPU, against the
oracle: the mask through moe_dispatch (both slot paths: the fused count
scan and the separate scan launch) and moe_forward, bit-exact on every
integer output and within 2e-2 on y; the statistics at the edges of the
router's lane geometry (1, 300 and 1024 experts) and for an empty batch.

"Expert Parallelism" (inferensys.com glossary), "Risk and Threat
Considerations": an expert can become unavailable; "Practitioner Guidance":
utilisation and routing entropy as health signals."""
import numpy as np
import pytest

import moe_synth
import oracle
from _helpers import (assert_bf16_close, packed_weights_for_gpu, problem_for, say, to_dev,
                      to_np)

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="health", B=64, d=32, E=8, k=2, c=1.25, f=48, act="gelu", x_dtype="bf16",
                n_ranks=1, e_begin=0, e_end=None, router_std=None, zipf_bias=False, tau=1.0,
                seed=11)
    base.update(kw)
    if base["e_end"] is None:
        base["e_end"] = base["E"]
    return moe_synth.Workload(**base)


def _mask(E, frac, seed):
    rng = np.random.default_rng(seed)
    m = rng.random(E) < frac
    return m


MASK_CASES = {
    # fused count scan (E % 4 == 0, small count table)
    "fused_quarter_masked": (dict(B=512, E=16, k=2, c=1.25), 0.25),
    # E % 4 != 0: separate scan launch
    "scan_E6": (dict(B=300, E=6, k=2, c=1.0), 0.34),
    # large count table: separate scan launch, many tiles
    "scan_E300_k4": (dict(B=4000, E=300, k=4, c=1.0, d=16), 0.1),
    "all_masked": (dict(B=64, E=8, k=2), 1.0),
    "none_masked": (dict(B=200, E=12, k=3), 0.0),
}


@pytest.mark.parametrize("case", list(MASK_CASES))
def test_dispatch_with_mask(case):
    import torch
    import expert_token_routing_fp32_amd as moe
    kw, frac = MASK_CASES[case]
    w = _wl(name=case, **kw)
    mask = _mask(w.E, frac, seed=len(case))
    say(f"[mask {case}] {w} masked={np.flatnonzero(mask).tolist()[:12]}")
    inp = moe_synth.make_inputs(w)
    ref = oracle.forward(inp["x"], inp["Wg"], inp["bias"], None, None, None, k=w.k, c=w.c,
                         act=w.act, n_ranks=w.n_ranks, unavailable=mask)
    p = problem_for(w, unavailable=torch.from_numpy(mask.astype(np.uint8)).cuda())
    o = moe.dispatch(p, to_dev(inp["x"]), to_dev(ref["idx"]))
    for key in ("pos", "dest", "expert_load", "expert_count", "expert_offset", "rank_offset"):
        np.testing.assert_array_equal(to_np(o[key]).reshape(np.shape(ref[key])), ref[key],
                                      err_msg=key)
    np.testing.assert_array_equal(to_np(o["keep"]).astype(bool), ref["keep"])
    K = int(ref["expert_offset"][-1])
    np.testing.assert_array_equal(to_np(o["pack_src"])[:K], ref["pack_src"])
    np.testing.assert_array_equal(to_np(o["packed"])[:K], ref["packed"])
    assert (ref["expert_count"][mask] == 0).all()
    say(f"  kept {K} of {w.B * w.k}")


def test_forward_with_mask():
    import torch
    import expert_token_routing_fp32_amd as moe
    w = _wl(name="fwd_mask", B=256, d=64, E=8, k=2, c=1.25, f=96)
    mask = np.zeros(8, bool)
    mask[[2, 5]] = True
    inp = moe_synth.make_inputs(w)
    ref = oracle.forward(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                         k=w.k, c=w.c, act=w.act, unavailable=mask)
    p = problem_for(w, unavailable=torch.from_numpy(mask.astype(np.uint8)).cuda())
    wp = packed_weights_for_gpu(p, inp)
    y, o = moe.forward(p, to_dev(inp["x"]), to_dev(inp["Wg"]), None, wp, outputs=True)
    for key in ("dest", "expert_count", "expert_offset"):
        np.testing.assert_array_equal(to_np(o[key]).reshape(np.shape(ref[key])), ref[key],
                                      err_msg=key)
    got = oracle.bf16_bits_to_f64(to_np(y))
    assert_bf16_close(got, ref["y"], what="forward y with experts 2 and 5 unavailable")
    # no token routed only to unavailable experts gets anything but 0
    only_masked = mask[ref["idx"]].all(axis=1)
    if only_masked.any():
        assert (got[only_masked] == 0).all()


@pytest.mark.parametrize("E,k,B", [(1, 1, 77), (300, 5, 1500), (1024, 16, 700), (37, 3, 1)])
def test_routing_stats_lane_geometries(E, k, B):
    import expert_token_routing_fp32_amd as moe
    rng = np.random.default_rng(E + B)
    logits = (rng.normal(size=(B, E)) * 2.0).astype(np.float32)
    idx, _ = oracle.route(logits, k)
    C = oracle.capacity(B, k, E, 1.0)
    _, _, load, count = oracle.assign_slots(idx, E, C)
    p = moe.make_problem(B=B, d=8, E=E, k=k, c=1.0, tau=1.3)
    s = moe.routing_stats(p, to_dev(logits), to_dev(load), to_dev(count))
    exp = oracle.routing_stats(logits, load, count, C, k, 1.3)
    np.testing.assert_allclose(to_np(s["prob_mean"]), exp["prob_mean"], rtol=1e-5, atol=1e-7)
    sm = to_np(s["summary"])
    np.testing.assert_allclose(sm[:3], [exp["aux_loss"], exp["entropy"], exp["load_entropy"]],
                               rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(to_np(s["dropped"]), exp["dropped"])


def test_routing_stats_empty_batch():
    import torch
    import expert_token_routing_fp32_amd as moe
    p = moe.make_problem(B=0, d=8, E=6, k=2)
    z = torch.zeros(6, dtype=torch.int32, device="cuda")
    s = moe.routing_stats(p, None, z, z)
    assert not to_np(s["summary"]).any() and not to_np(s["prob_mean"]).any()
