"""Edge cases and random small shapes, every step fed the oracle's inputs for
it and compared at the same bar as the full workloads: empty batch, zero
capacity, k = 1, k = E, E = 1, ragged d and f, experts with more rows than one
256-row tile, float32 activations, temperature, bias, residual, a subset of
local experts, the largest E and k, and hypothesis-drawn shapes."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import moe_synth
import oracle
from _helpers import (assert_bf16_close, assert_f32_close, packed_weights_for_gpu, problem_for,
                      say, to_dev, to_np)

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="edge", B=64, d=32, E=8, k=2, c=1.25, f=48, act="gelu", x_dtype="bf16",
                n_ranks=1, e_begin=0, e_end=None, router_std=None, zipf_bias=False, tau=1.0,
                seed=3)
    base.update(kw)
    if base["e_end"] is None:
        base["e_end"] = base["E"]
    return moe_synth.Workload(**base)


def check_stages(w, C=None, residual=False, ffn=True):
    """route <- oracle logits, dispatch <- oracle idx, ffn <- oracle packed,
    combine <- oracle ret (bf16-rounded by the oracle), forward end to end."""
    import torch
    import expert_token_routing_fp32_amd as moe
    inp = moe_synth.make_inputs(w)
    ref = oracle.forward(inp["x"], inp["Wg"], inp["bias"], None, None, None, k=w.k, c=w.c,
                         act=w.act, n_ranks=w.n_ranks, e_begin=w.e_begin, e_end=w.e_end,
                         tau=w.tau, C=C)
    p = problem_for(w, C=-1 if C is None else C, add_residual=residual)
    assert moe.problem_capacity(p) == ref["C"]
    x = to_dev(inp["x"]) if w.B else torch.empty(
        (0, w.d), dtype=torch.int16 if w.x_dtype == "bf16" else torch.float32, device="cuda")
    # gate
    if w.B:
        lg = moe.gate(p, x, to_dev(inp["Wg"]), None if inp["bias"] is None else to_dev(inp["bias"]))
        assert_f32_close(to_np(lg), ref["logits"], what="logits")
    # route
    lt = to_dev(ref["logits"]) if w.B else torch.empty((0, w.E), device="cuda")
    idx, wt = moe.route(p, lt)
    if w.B:
        np.testing.assert_array_equal(to_np(idx), ref["idx"])
        assert_f32_close(to_np(wt), ref["w"], what="topk_w")
    # dispatch
    it = to_dev(ref["idx"]) if w.B else torch.empty((0, w.k), dtype=torch.int32, device="cuda")
    o = moe.dispatch(p, x, it)
    for key in ("pos", "dest", "expert_load", "expert_count", "expert_offset", "rank_offset"):
        np.testing.assert_array_equal(to_np(o[key]).reshape(np.shape(ref[key])), ref[key], err_msg=key)
    K = int(ref["expert_offset"][-1])
    if w.B:
        np.testing.assert_array_equal(to_np(o["keep"]).astype(bool), ref["keep"])
        np.testing.assert_array_equal(to_np(o["pack_src"])[:K], ref["pack_src"])
        np.testing.assert_array_equal(to_np(o["packed"][:K]), ref["packed"])
    if not ffn or w.B == 0:
        return
    # expert ffn on the oracle's packed rows
    wp = packed_weights_for_gpu(p, inp)
    km = moe.max_kept(p)
    pk = torch.zeros((max(km, 1), w.d), dtype=torch.int16, device="cuda")
    if K:
        pk[:K] = to_dev(ref["packed"])
    ret = moe.expert_ffn(p, pk, to_dev(ref["expert_offset"]), wp)
    exp = oracle.expert_ffn(inp["x"], ref["pack_src"], ref["expert_offset"], w.e_begin, w.e_end,
                            inp["W1"], inp["W2"], inp["W3"], w.act)
    if K:
        got = oracle.bf16_bits_to_f64(to_np(ret[:K]))
        assert_bf16_close(got, exp, what="ret")
    # combine on the oracle's ret, rounded to bf16 by the oracle
    rb = oracle.f32_to_bf16_bits_rne(exp.astype(np.float32)) if K else np.zeros((0, w.d), np.uint16)
    rk = torch.zeros((max(km, 1), w.d), dtype=torch.int16, device="cuda")
    if K:
        rk[:K] = to_dev(rb)
    y = moe.combine(p, rk, to_dev(ref["dest"]), to_dev(ref["w"].astype(np.float32)),
                    x_residual=x if residual else None)
    yexp = oracle.combine(oracle.bf16_bits_to_f64(rb), ref["dest"], ref["w"],
                          x_residual=inp["x"] if residual else None)
    yg = to_np(y)
    got = oracle.bf16_bits_to_f64(yg) if yg.dtype == np.uint16 else yg.astype(np.float64)
    assert_bf16_close(got, yexp, what="y")
    if not ref["keep"].any(axis=1).all() and not residual:
        assert (got[~ref["keep"].any(axis=1)] == 0).all()
    # and the whole layer
    yf = moe.forward(p, x, to_dev(inp["Wg"]), None if inp["bias"] is None else to_dev(inp["bias"]),
                     wp)
    yfe = oracle.combine(exp, ref["dest"], ref["w"], x_residual=inp["x"] if residual else None)
    yfg = to_np(yf)
    gotf = oracle.bf16_bits_to_f64(yfg) if yfg.dtype == np.uint16 else yfg.astype(np.float64)
    assert_bf16_close(gotf, yfe, what="forward y")


CASES = {
    "empty_batch": dict(w=dict(B=0)),
    "zero_capacity": dict(w=dict(B=50), C=0),
    "top1": dict(w=dict(k=1, B=100)),
    "k_equals_E": dict(w=dict(E=4, k=4, e_end=4, B=40)),
    "single_expert": dict(w=dict(E=1, k=1, e_end=1, B=33)),
    "ragged_dims": dict(w=dict(B=300, d=40, f=72, E=5, e_end=5, c=2.0)),
    "multi_tile_rows": dict(w=dict(B=700, d=64, f=96, E=2, e_end=2, k=1, c=1.5)),
    "big_tiles_swiglu": dict(w=dict(B=1100, d=520, f=264, E=3, e_end=3, k=2, c=1.0, act="swiglu")),
    "f32_activations": dict(w=dict(x_dtype="f32", B=77, d=24, f=40, router_std=0.5)),
    "temperature": dict(w=dict(tau=0.7, B=90)),
    "bias": dict(w=dict(zipf_bias=True, E=16, e_end=16, B=128)),
    "residual": dict(w=dict(B=64), residual=True),
    "residual_f32": dict(w=dict(B=64, x_dtype="f32"), residual=True),
    "local_subset": dict(w=dict(E=8, n_ranks=4, e_begin=2, e_end=4, B=96, act="swiglu")),
    "no_local_experts": dict(w=dict(E=8, n_ranks=2, e_begin=4, e_end=4, B=40)),
    "max_E_k": dict(w=dict(E=1024, k=16, e_end=1024, B=2048, d=64, f=16), ffn=False),
    "E_not_pow2_many": dict(w=dict(E=300, k=5, e_end=300, B=1500, d=48, f=32)),
    "drop_heavy": dict(w=dict(E=16, e_end=16, B=512, c=0.25, zipf_bias=True)),
    # >= 384 rows per expert: the matrix-core tile schedule (per-XCD blocks)
    "rows_1024_gelu": dict(w=dict(B=2048, d=72, E=4, e_end=4, k=2, c=1.0, f=520)),
    "rows_1024_swiglu": dict(w=dict(B=2048, d=136, E=4, e_end=4, k=2, c=1.25, f=264,
                                    act="swiglu")),
    # ~1050 rows per expert: five row slices of 6-7 blocks each, not four full
    # slices and a thin remainder
    "rows_1050_five_slices": dict(w=dict(B=2100, d=72, E=4, e_end=4, k=2, c=1.25, f=264,
                                         act="swiglu")),
}


@pytest.mark.parametrize("case", list(CASES))
def test_edge(case):
    spec = CASES[case]
    w = _wl(name=case, **spec["w"])
    say(f"[edge {case}] {w}")
    check_stages(w, C=spec.get("C"), residual=spec.get("residual", False), ffn=spec.get("ffn", True))


@settings(max_examples=25, deadline=None, suppress_health_check=list(HealthCheck))
@given(B=st.integers(1, 260), d8=st.integers(1, 12), f8=st.integers(1, 20), E=st.integers(1, 40),
       data=st.data())
def test_random_shapes(B, d8, f8, E, data):
    k = data.draw(st.integers(1, min(E, 8)))
    c = data.draw(st.sampled_from([0.3, 1.0, 1.25, 2.0]))
    act = data.draw(st.sampled_from(["gelu", "swiglu"]))
    xdt = data.draw(st.sampled_from(["bf16", "f32"]))
    seed = data.draw(st.integers(0, 1000))
    w = _wl(name="random", B=B, d=8 * d8, f=8 * f8, E=E, e_end=E, k=k, c=c, act=act,
            x_dtype=xdt, seed=seed)
    say(f"[random] {w}")
    check_stages(w)


def test_pack_combine_past_the_grid_cap():
    """B = 262147 tokens of d = 8192: the pack and the combine then need more
    than 65535 groups of 4 rows, the grid's y extent is capped and the
    kernels loop over the rest.  With one expert, k = 1 and C = B nothing
    is dropped, every packed row r is token r and its weight is 1, so the
    packed rows and y must equal x bit for bit (a property at any size; the
    oracle is not needed)."""
    import torch
    import expert_token_routing_fp32_amd as moe
    B, d = 262147, 8192
    p = moe.make_problem(B=B, d=d, E=1, k=1, c=1.0, f=8, act="gelu", x_dtype="bf16")
    assert moe.problem_capacity(p) == B
    say(f"[grid cap] B={B} d={d}")
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(B, d, device="cuda", generator=g).to(torch.bfloat16)
    idx = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    o = moe.dispatch(p, x, idx)
    assert int(o["expert_offset"][1]) == B
    assert torch.equal(o["dest"].view(-1), torch.arange(B, dtype=torch.int32, device="cuda"))
    assert torch.equal(o["packed"][:B], x.view(torch.int16))
    w = torch.ones(B, 1, dtype=torch.float32, device="cuda")
    y = moe.combine(p, o["packed"], o["dest"], w)
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("shape", [dict(B=0), dict(B=96), dict(B=96, x_dtype="f32"),
                                   dict(B=16384, E=128, e_end=128, d=128, f=64),
                                   dict(B=96, E=8, n_ranks=2, e_begin=4, e_end=4)])
def test_stage_events_follow_the_kernels(shape):
    """moe_forward's stage events come from the dispatch timestamps of each
    stage's kernels, in stream order, so every consecutive pair is ordered
    (the gate's split copy, a forward with no local experts and an empty
    batch, where every event is a marker, included), and the output is the
    same as without events."""
    import torch
    import expert_token_routing_fp32_amd as moe
    w = _wl(name="events", **shape)
    inp = moe_synth.make_inputs(w)
    p = problem_for(w)
    x = to_dev(inp["x"]) if w.B else torch.empty((0, w.d), dtype=torch.int16, device="cuda")
    Wg = to_dev(inp["Wg"])
    wp = packed_weights_for_gpu(p, inp)
    say(f"[stage events] {w}")
    y0 = moe.forward(p, x, Wg, None, wp)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.N_STAGE_EVENTS)]
    y1 = moe.forward(p, x, Wg, None, wp, stage_events=evs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(y1), to_np(y0))
    for i in range(moe.N_STAGE_EVENTS - 1):
        assert evs[i].elapsed_time(evs[i + 1]) >= -1e-3, i
    assert evs[0].elapsed_time(evs[-1]) >= 0
