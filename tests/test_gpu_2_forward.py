"""End-to-end moe_forward against the oracle, with the launch configuration
bench.py times (one stream, in-place expert outputs, workspace outputs).

The GPU computes the router logits in fp32 and the oracle rounds an exact
float64 sum, so a token whose top-(k+1) logits are closer than the logit
tolerance may legitimately be routed differently.  Such tokens are found from
the oracle's logits alone ("undecided"); every other token must be routed
identically.  When all tokens agree, every integer output must match bit for
bit.  Outputs y are compared on tokens whose choices and drop flags agree
(all of them, normally) -- y of a token depends only on its own choices,
weights and drop flags.  The forward's choices and weights must also equal,
bit for bit, what moe_route makes of the forward's own logits."""
import numpy as np
import pytest

import oracle
from moe_synth import ORDER
from _helpers import (TOL_F32, assert_bf16_close, assert_f32_close, problem_for, say, to_dev,
                      to_np, packed_weights_for_gpu, workload)

pytestmark = pytest.mark.gpu


def undecided_tokens(logits: np.ndarray, k: int, tol: float = TOL_F32) -> np.ndarray:
    """Tokens whose ordered top-(k+1) logits have a gap within twice the
    tolerance (so the fp32 gate may order them either way)."""
    l = np.sort(logits.astype(np.float64), axis=1)[:, ::-1]
    m = min(k + 1, l.shape[1])
    top = l[:, :m]
    gaps = top[:, :-1] - top[:, 1:]
    band = 2 * tol * np.maximum(1.0, np.abs(top[:, :-1]))
    return np.nonzero((gaps <= band).any(axis=1))[0] if m > 1 else np.zeros(0, dtype=np.int64)


def run_forward(w, inp, ref, name, n_sample=48):
    import torch
    import expert_token_routing_fp32_amd as moe
    p = problem_for(w)
    x = to_dev(inp["x"])
    wp = packed_weights_for_gpu(p, inp)
    y, o = moe.forward(p, x, to_dev(inp["Wg"]), None if inp["bias"] is None else to_dev(inp["bias"]),
                       wp, outputs=True)
    torch.cuda.synchronize()
    assert_f32_close(to_np(o["logits"]), ref["logits"], what=f"{name} logits")
    gi = to_np(o["topk_idx"])
    # the forward's routing is the route kernel's on the forward's own logits
    idx2, w2 = moe.route(p, o["logits"])
    np.testing.assert_array_equal(to_np(idx2), gi)
    np.testing.assert_array_equal(to_np(w2).view(np.uint32), to_np(o["topk_w"]).view(np.uint32))
    und = undecided_tokens(ref["logits"], w.k)
    diff = np.nonzero((gi != ref["idx"]).any(axis=1))[0]
    say(f"  {name}: undecided tokens {und.size}, tokens routed differently {diff.size}")
    assert np.isin(diff, und).all(), "a decided token was routed differently"
    assert_f32_close(to_np(o["topk_w"])[np.setdiff1d(np.arange(w.B), diff)],
                     ref["w"][np.setdiff1d(np.arange(w.B), diff)], what=f"{name} topk_w")
    gkeep = to_np(o["keep"]).astype(bool)
    if diff.size == 0:
        for key in ("pos", "dest", "expert_load", "expert_count", "expert_offset",
                    "rank_offset"):
            np.testing.assert_array_equal(to_np(o[key]), ref[key], err_msg=key)
        np.testing.assert_array_equal(gkeep, ref["keep"])
        K = int(ref["expert_offset"][-1])
        np.testing.assert_array_equal(to_np(o["pack_src"])[:K], ref["pack_src"])
    # a moved choice shifts at most one keep decision in each of two experts
    kdiff = np.nonzero((gkeep != ref["keep"]).any(axis=1) | (gi != ref["idx"]).any(axis=1))[0]
    assert kdiff.size <= 3 * diff.size
    agree = np.setdiff1d(np.arange(w.B), kdiff)
    # y on every agreeing token for the small workloads; otherwise on
    # sampled agreeing tokens that reach every local expert (the tokens of
    # its first and last row and of one random row), plus random ones
    K_all = int(ref["expert_offset"][-1])
    if K_all * w.f <= 4096 * 8192 and w.B * w.d <= 16384 * 2048:
        tokens = agree
    else:
        rng = np.random.default_rng(2)
        eo, ps = ref["expert_offset"], ref["pack_src"]
        pick = []
        for e in range(w.e_begin, w.e_end):
            a, b = int(eo[e]), int(eo[e + 1])
            if b > a:
                pick += [int(ps[a]), int(ps[b - 1]), int(ps[int(rng.integers(a, b))])]
        pick += list(rng.choice(agree, size=min(n_sample, agree.size), replace=False))
        tokens = np.intersect1d(np.unique(np.array(pick, dtype=np.int64)), agree)
        reached = np.unique(ref["idx"][tokens][ref["keep"][tokens]])
        local = reached[(reached >= w.e_begin) & (reached < w.e_end)]
        say(f"  {name}: {tokens.size} sampled tokens reach {local.size} local experts")
    dsub = ref["dest"][tokens]
    rows = np.unique(dsub[dsub >= 0])
    ret = oracle.expert_ffn(inp["x"], ref["pack_src"], ref["expert_offset"], w.e_begin, w.e_end,
                            inp["W1"], inp["W2"], inp["W3"], w.act, rows=rows)
    exp = oracle.combine(ret, ref["dest"], ref["w"], tokens=tokens, ret_rows=rows)
    yg = to_np(y[torch.from_numpy(tokens).to(y.device)])
    got = oracle.bf16_bits_to_f64(yg) if yg.dtype == np.uint16 else yg.astype(np.float64)
    assert_bf16_close(got, exp, what=f"{name} y ({tokens.size} tokens)")
    return y, o


@pytest.mark.parametrize("name", ORDER)
def test_forward(name):
    say(f"[forward {name}]")
    w, inp, ref = workload(name)
    run_forward(w, inp, ref, name)


def test_forward_is_deterministic():
    import torch
    import expert_token_routing_fp32_amd as moe
    w, inp, ref = workload("uniform")
    p = problem_for(w)
    args = (to_dev(inp["x"]), to_dev(inp["Wg"]), None, packed_weights_for_gpu(p, inp))
    y1 = moe.forward(p, *args)
    y2 = moe.forward(p, *args)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("B,d,E", [(8192, 320, 128), (16384, 328, 100), (16384, 512, 256),
                                   (8192, 512, 160), (32768, 512, 256), (32768, 328, 200)])
def test_forward_gate_matches_moe_gate(B, d, E):
    """Where that fills the CUs (the first four shapes) the forward splits
    the router weights once into a copy of bf16 parts before the gate; on
    large gates whose grid is full already (the last two) it copies them in
    the lanes' order as fp32 and splits in the kernel; moe_gate loads Wg
    directly and splits inside its kernel.
    The MFMAs see the same three parts in the same order, so the logits must
    be bit-identical.  Shapes: a K range whose last 64-k stage lies past d
    (d = 320 over two K ranges), d not a multiple of 16 with E not a multiple
    of 32, 256 experts in one workgroup, and 160 and 200 experts (5 or 7
    blocks of 32 over workgroups of 4: the second row of workgroups has
    blocks past the last one, which must read only inside the copy)."""
    import torch
    import expert_token_routing_fp32_amd as moe
    p = moe.make_problem(B=B, d=d, E=E, k=2, c=1.25, f=16, act="gelu", x_dtype="bf16")
    g = torch.Generator(device="cuda").manual_seed(B + d + E)
    x = torch.randn(B, d, device="cuda", generator=g).to(torch.bfloat16)
    Wg = torch.randn(d, E, device="cuda", generator=g) * d ** -0.5
    W1 = (torch.randn(E, d, 16, device="cuda", generator=g) * d ** -0.5).to(torch.bfloat16)
    W2 = (torch.randn(E, 16, d, device="cuda", generator=g) * 0.25).to(torch.bfloat16)
    wp = moe.pack_weights(p, W1, None, W2)
    say(f"[gate copy] B={B} d={d} E={E}")
    lg = moe.gate(p, x, Wg)
    _, o = moe.forward(p, x, Wg, None, wp, outputs=True)
    torch.cuda.synchronize()
    assert torch.equal(o["logits"].view(torch.int32), lg.view(torch.int32))
