"""Shared expert on the GPU against the oracle ("Expert Parallelism",
narrativegoldmine.com, "Major Variants and Families", shared expert routing:
one expert processes every token beside the routed ones).

moe_shared_ffn on all rows (weight-streaming and matrix-core-bound row
counts, GELU and SwiGLU) and on sampled rows of the EP-share shape (32768
tokens, 7168 -> 2048 -> 7168 SwiGLU); moe_combine_shared and
moe_forward_shared end to end.  bf16 outputs within 2e-2 (max|d| / max|ref|),
integer outputs bit-exact."""
import numpy as np
import pytest

import moe_synth
import oracle
from _helpers import (assert_bf16_close, packed_weights_for_gpu, problem_for, say, to_dev,
                      to_np)

pytestmark = pytest.mark.gpu


def _shared_weights(rng, d, f, swiglu):
    """bf16 bits of W1s [1, d, f], W3s, W2s [1, f, d] with std 1/sqrt(fan_in)."""
    def bf(a):
        return oracle.f32_to_bf16_bits_rne(a.astype(np.float32))
    W1 = bf(rng.normal(scale=d ** -0.5, size=(1, d, f)))
    W3 = bf(rng.normal(scale=d ** -0.5, size=(1, d, f))) if swiglu else None
    W2 = bf(rng.normal(scale=f ** -0.5, size=(1, f, d)))
    return W1, W3, W2


def _pack_shared(ps, W1, W3, W2):
    import expert_token_routing_fp32_amd as moe
    return moe.pack_weights(ps, to_dev(W1), None if W3 is None else to_dev(W3), to_dev(W2))


@pytest.mark.parametrize("B,d,f,act", [(300, 64, 96, "gelu"), (300, 72, 40, "swiglu"),
                                       (1000, 256, 520, "gelu"), (1000, 136, 264, "swiglu")])
def test_shared_ffn_all_rows(B, d, f, act):
    import expert_token_routing_fp32_amd as moe
    rng = np.random.default_rng(B + d + f)
    x = oracle.f32_to_bf16_bits_rne(rng.normal(size=(B, d)).astype(np.float32))
    W1, W3, W2 = _shared_weights(rng, d, f, act == "swiglu")
    p = moe.make_problem(B=B, d=d, E=4, k=2, f=f, act=act)
    ps = moe.shared_problem(p, f, act)
    say(f"[shared {B}x{d} f={f} {act}]")
    out = moe.shared_ffn(ps, to_dev(x), _pack_shared(ps, W1, W3, W2))
    exp = oracle.shared_ffn(x, W1[0], W2[0], None if W3 is None else W3[0], act)
    assert_bf16_close(oracle.bf16_bits_to_f64(to_np(out)), exp, what="shared out")


def test_shared_ffn_ep_share_shape_sampled_rows():
    import torch
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.WORKLOADS["ep_share"]
    rng = np.random.default_rng(5)
    inp = moe_synth.make_inputs(w)
    W1, W3, W2 = _shared_weights(rng, w.d, w.f, True)
    p = problem_for(w)
    ps = moe.shared_problem(p, w.f, "swiglu")
    out = moe.shared_ffn(ps, to_dev(inp["x"]), _pack_shared(ps, W1, W3, W2))
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.B - 1],
                                     rng.integers(0, w.B, 59)]))
    exp = oracle.shared_ffn(inp["x"], W1[0], W2[0], W3[0], "swiglu", tokens=rows)
    got = to_np(out[torch.from_numpy(rows).cuda()])
    assert_bf16_close(oracle.bf16_bits_to_f64(got), exp, what=f"ep_share shared ({rows.size} rows)")


def test_combine_shared():
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.Workload(name="cs", B=200, d=64, E=8, k=2, c=1.0, f=48, act="gelu",
                           x_dtype="bf16", n_ranks=1, e_begin=0, e_end=8, router_std=None,
                           zipf_bias=False, tau=1.0, seed=2)
    inp = moe_synth.make_inputs(w)
    ref = oracle.forward(inp["x"], inp["Wg"], None, None, None, None, k=w.k, c=w.c, act=w.act)
    rng = np.random.default_rng(0)
    K = int(ref["expert_offset"][-1])
    ret = oracle.f32_to_bf16_bits_rne(rng.normal(size=(K, w.d)).astype(np.float32))
    sh = oracle.f32_to_bf16_bits_rne(rng.normal(size=(w.B, w.d)).astype(np.float32))
    p = problem_for(w)
    full = np.zeros((max(moe.max_kept(p), 1), w.d), np.uint16)  # the binding wants Kmax rows
    full[:K] = ret
    y = moe.combine(p, to_dev(full), to_dev(ref["dest"]), to_dev(ref["w"].astype(np.float32)),
                    shared_out=to_dev(sh))
    exp = oracle.combine(oracle.bf16_bits_to_f64(ret), ref["dest"], ref["w"],
                         shared=oracle.bf16_bits_to_f64(sh))
    assert_bf16_close(oracle.bf16_bits_to_f64(to_np(y)), exp, what="combine + shared")


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_forward_shared(act):
    import torch
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.Workload(name="fs", B=256, d=64, E=8, k=2, c=1.0, f=96, act=act,
                           x_dtype="bf16", n_ranks=1, e_begin=0, e_end=8, router_std=None,
                           zipf_bias=False, tau=1.0, seed=4)
    inp = moe_synth.make_inputs(w)
    rng = np.random.default_rng(9)
    fs = 128
    S1, S3, S2 = _shared_weights(rng, w.d, fs, act == "swiglu")
    ref = oracle.forward(inp["x"], inp["Wg"], None, inp["W1"], inp["W3"], inp["W2"], k=w.k,
                         c=w.c, act=act, shared=(S1[0], None if S3 is None else S3[0], S2[0]))
    p = problem_for(w)
    ps = moe.shared_problem(p, fs, act)
    wp = packed_weights_for_gpu(p, inp)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.N_STAGE_EVENTS)]
    y, o = moe.forward(p, to_dev(inp["x"]), to_dev(inp["Wg"]), None, wp, outputs=True,
                       stage_events=evs, shared=(ps, _pack_shared(ps, S1, S3, S2)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o["dest"]), ref["dest"])
    assert_bf16_close(oracle.bf16_bits_to_f64(to_np(y)), ref["y"], what=f"forward+shared {act}")
    a, b = moe.STAGE_EVENTS["expert_ffn"]
    assert evs[a].elapsed_time(evs[b]) > 0
