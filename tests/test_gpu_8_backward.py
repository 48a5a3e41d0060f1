"""Backward pass on the GPU against the oracle's float64 backward ("Expert
Parallelism", narrativegoldmine.com, "About": training by backpropagation
with an auxiliary load-balancing loss; "Formal Algorithm": the auxiliary
loss joins the training loss).

Bars (the pages fix no backward precision; these follow the forward's):
* bf16 outputs (dx, the packed-row gradient) and every gradient that passes
  through a bf16 matrix-core operand (the experts' weight gradients: dret,
  the recomputed Z, dZ and H are bf16): max|d| / max|ref| <= 2e-2, per
  expert as well as per tensor;
* fp32 outputs computed from the same inputs in fp32 (dw = <dy, ret>, the
  router's dlogits, the dispatch sum): |d| <= 1e-5 max(1, |ref|) when fed
  the oracle's inputs; dWg and the bias gradient, sums over all B tokens:
  that, or the forward error bound of an n-term fp32 sum, gamma_n times the
  sum of the terms' magnitudes, whichever is larger; end to end, where dw
  differs from the float64 dot by fp32 rounding, max|d| / max|ref| <= 1e-4.

Stage tests feed each step the oracle's inputs for it (bf16-rounded where
the GPU takes bf16); the chain (moe_backward) runs on the GPU forward's own
outputs and is compared with the oracle on the same routing and ret."""
import numpy as np
import pytest

import moe_synth
import oracle
from _helpers import (assert_bf16_close, assert_f32_close, assert_sum_close,
                      packed_weights_for_gpu, problem_for, rel_err, say, to_dev, to_np,
                      weights_for_gpu, workload)

pytestmark = pytest.mark.gpu

AUX = 0.05


def _bf(a64):
    """float64 -> the bf16 values the GPU would hold (RNE) and their bits."""
    bits = oracle.f32_to_bf16_bits_rne(np.asarray(a64, np.float32))
    return oracle.bf16_bits_to_f64(bits), bits


def _x_vals(x):
    return oracle.bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def _dy(w, seed=5):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((w.B, w.d)).astype(np.float32)
    return moe_synth.f32_to_bf16_bits(a) if w.x_dtype == "bf16" else a


def _wpb(p, inp):
    import expert_token_routing_fp32_amd as moe
    W1, W3, W2 = weights_for_gpu(inp)
    return moe.pack_weights_bwd(p, to_dev(W1), None if W3 is None else to_dev(W3), to_dev(W2))


def _per_expert(got, ref, rows, eo, experts, what, tol=2e-2):
    worst = 0.0
    for e in experts:
        m = (rows >= eo[e]) & (rows < eo[e + 1])
        if m.any():
            r = rel_err(got[m], ref[m])
            worst = max(worst, r)
            assert r <= tol, f"{what}: expert {e}: {r}"
    say(f"  {what}: worst expert {worst:.3e}")


def _rel_close(got, ref, tol, what):
    e = rel_err(got, ref)
    say(f"  {what}: max|d|/max|ref| = {e:.3e} (tol {tol:g})")
    assert e <= tol, f"{what}: {e} > {tol}"


SMALL = {
    "toy": moe_synth.WORKLOADS["toy"],
    "gelu_drops_residual": moe_synth.Workload("bwd_gelu", B=600, d=96, E=12, k=3, c=0.8, f=136,
                                              act="gelu", x_dtype="bf16", n_ranks=3, e_begin=0,
                                              e_end=12, router_std=None, zipf_bias=True, seed=3),
    "swiglu_remote": moe_synth.Workload("bwd_swiglu", B=512, d=128, E=16, k=2, c=1.25, f=200,
                                        act="swiglu", x_dtype="bf16", n_ranks=4, e_begin=4,
                                        e_end=8, router_std=None, seed=4),
    "swiglu_f32_x": moe_synth.Workload("bwd_f32", B=300, d=64, E=8, k=2, c=1.0, f=96,
                                       act="swiglu", x_dtype="f32", n_ranks=1, e_begin=0,
                                       e_end=8, router_std=0.3, seed=6),
    # whole 256 x 256 tiles of the weight-gradient GEMM with fp32 tokens: the
    # router dx epilogue's vector path storing fp32 (B, d >= 256)
    "swiglu_f32_x_wide": moe_synth.Workload("bwd_f32_wide", B=640, d=512, E=16, k=2, c=1.25,
                                            f=256, act="swiglu", x_dtype="f32", n_ranks=1,
                                            e_begin=0, e_end=16, router_std=0.3, seed=8),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_backward_stages(case):
    """Each backward step fed the oracle's inputs, all rows and experts."""
    import torch
    import expert_token_routing_fp32_amd as moe
    w = SMALL[case]
    res = case == "gelu_drops_residual"
    say(f"[backward stages {case}] B={w.B} d={w.d} E={w.E} k={w.k} f={w.f} {w.act}")
    inp = moe_synth.make_inputs(w)
    ref = oracle.forward(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                         k=w.k, c=w.c, act=w.act, n_ranks=w.n_ranks, e_begin=w.e_begin,
                         e_end=w.e_end, tau=w.tau, add_residual=res)
    p = problem_for(w, add_residual=res)
    dy = _dy(w)
    dyv = _x_vals(dy)
    dest, eo, ps = ref["dest"], ref["expert_offset"], ref["pack_src"]
    K = int(eo[-1])
    km = moe.max_kept(p)
    w32 = ref["w"].astype(np.float32)
    # combine backward, on the oracle's ret as the GPU holds it (bf16)
    ret_v, ret_bits = _bf(ref["ret"])
    ret_d = torch.zeros((km, w.d), dtype=torch.int16, device="cuda")
    ret_d[:K] = to_dev(ret_bits)
    dret_g, dw_g = moe.combine_backward(p, to_dev(dy), ret_d, to_dev(dest), to_dev(w32))
    dret_r, dw_r = oracle.combine_backward(dyv, ret_v, dest, w32)
    assert_bf16_close(oracle.bf16_bits_to_f64(to_np(dret_g)[:K]), dret_r, what="dret")
    assert_f32_close(to_np(dw_g), dw_r, what="dw")
    assert (to_np(dw_g)[~ref["keep"]] == 0).all()
    # route backward with the auxiliary term, fed the oracle's dw
    dwf = dw_r.astype(np.float32)
    dl_g = moe.route_backward(p, to_dev(ref["logits"]), to_dev(ref["idx"]), to_dev(dwf),
                              to_dev(ref["expert_load"]), AUX)
    dl_r = oracle.route_backward(ref["logits"], ref["idx"], dwf, w.tau, AUX, ref["expert_load"])
    assert_f32_close(to_np(dl_g), dl_r, what="dlogits")
    # expert FFN backward, fed the oracle's dret rounded to bf16
    dret_v, dret_bits = _bf(dret_r)
    dret_d = torch.zeros((km, w.d), dtype=torch.int16, device="cuda")
    dret_d[:K] = to_dev(dret_bits)
    before = dret_d.clone()
    wp = packed_weights_for_gpu(p, inp)
    wpb = _wpb(p, inp)
    ps_d = torch.zeros(max(km, 1), dtype=torch.int32, device="cuda")
    ps_d[:K] = to_dev(ps)
    o = moe.expert_ffn_backward(p, to_dev(inp["x"]), ps_d, to_dev(eo), wp, wpb, dret_d)
    dXp_r, gr = oracle.expert_ffn_backward(inp["x"], ps, eo, w.e_begin, w.e_end, inp["W1"],
                                           inp["W2"], inp["W3"], w.act, dret_v)
    lo, hi = int(eo[w.e_begin]), int(eo[w.e_end])
    rows = np.arange(lo, hi)
    got = oracle.bf16_bits_to_f64(to_np(o["dxp"])[lo:hi])
    assert_bf16_close(got, dXp_r[lo:hi], what="dXp (local rows)")
    _per_expert(got, dXp_r[lo:hi], rows, eo, range(w.e_begin, w.e_end), "dXp")
    if lo > 0:
        assert torch.equal(o["dxp"][:lo], before[:lo])
    if K > hi:
        assert torch.equal(o["dxp"][hi:K], before[hi:K])
    for name, gi in (("dW1", 0), ("dW2", 1), ("dW3", 2)):
        if gr[w.e_begin][gi] is None:
            continue
        G = to_np(o[name])
        for e in range(w.e_begin, w.e_end):
            R = gr[e][gi]
            gg = G[e - w.e_begin]
            if np.abs(R).max() == 0:
                assert np.abs(gg).max() == 0, f"{name} expert {e} should be zero"
            else:
                assert rel_err(gg, R) <= 2e-2, (name, e, rel_err(gg, R))
        say(f"  {name}: every local expert within 2e-2")
    # dispatch backward on bf16 packed-row gradients
    dxp_v, dxp_bits = _bf(dXp_r)
    dxp_d = torch.zeros((km, w.d), dtype=torch.int16, device="cuda")
    dxp_d[:K] = to_dev(dxp_bits)
    acc_g = moe.dispatch_backward(p, dxp_d, to_dev(dest), to_dev(dy) if res else None)
    acc_r = oracle.dispatch_backward(dxp_v, dest) + (dyv if res else 0.0)
    assert_f32_close(to_np(acc_g), acc_r, what="dispatch backward")
    # gate backward, fed the oracle's dlogits and the dispatch sum
    dlf = dl_r.astype(np.float32)
    accf = acc_r.astype(np.float32)
    dx_g, dWg_g, db_g = moe.gate_backward(p, to_dev(inp["x"]), to_dev(inp["Wg"]), to_dev(dlf),
                                          to_dev(accf))
    dxg_r, dWg_r, db_r = oracle.gate_backward(inp["x"], inp["Wg"], dlf)
    dxg = to_np(dx_g)
    dxv = oracle.bf16_bits_to_f64(dxg) if dxg.dtype == np.uint16 else dxg.astype(np.float64)
    assert_bf16_close(dxv, dxg_r + accf.astype(np.float64), what="dx (gate + dispatch)")
    # dWg and the bias gradient are sums over the B tokens (of 3 products per
    # token with bf16 x, 6 with fp32 x, then at most 64 partials)
    n = (3 if w.x_dtype == "bf16" else 6) * w.B + 64
    dla = np.abs(dlf.astype(np.float64))
    assert_sum_close(to_np(dWg_g), dWg_r, np.abs(_x_vals(inp["x"])).T @ dla, n, what="dWg")
    assert_sum_close(to_np(db_g), db_r, dla.sum(axis=0), n, what="dbias")


def _chain(w, tokens_n=None, experts=None, res=False):
    """moe_backward on the GPU forward's outputs against the oracle on the
    same routing and ret: everything (tokens_n None) or sampled tokens and
    the weight gradients of the listed experts."""
    import torch
    import expert_token_routing_fp32_amd as moe
    inp = moe_synth.make_inputs(w)
    p = problem_for(w, add_residual=res)
    x = to_dev(inp["x"])
    Wg = to_dev(inp["Wg"])
    bias = None if inp["bias"] is None else to_dev(inp["bias"])
    wp = packed_weights_for_gpu(p, inp)
    wpb = _wpb(p, inp)
    y, o = moe.forward(p, x, Wg, bias, wp, outputs=True)
    dy = _dy(w, seed=7)
    g = moe.backward(p, x, Wg, wp, wpb, o, to_dev(dy), aux_coef=AUX)
    torch.cuda.synchronize()
    logits = to_np(o["logits"])
    idx, dest = to_np(o["topk_idx"]), to_np(o["dest"])
    w32 = to_np(o["topk_w"])
    eo, ps, load = to_np(o["expert_offset"]), to_np(o["pack_src"]), to_np(o["expert_load"])
    K = int(eo[-1])
    dyv = _x_vals(dy)
    B = w.B
    full = tokens_n is None
    if full:
        tokens = np.arange(B)
    else:
        rng = np.random.default_rng(11)
        tokens = np.sort(rng.choice(B, size=min(tokens_n, B), replace=False))
    if experts is None:
        experts = list(range(w.e_begin, w.e_end)) if full else []
    # rows: those of the sampled tokens, and every row of the sampled experts
    dsub = dest[tokens]
    rows = set(dsub[dsub >= 0].tolist())
    for e in experts:
        rows.update(range(int(eo[e]), int(eo[e + 1])))
    rows = np.array(sorted(rows), dtype=np.int64)
    say(f"  {len(tokens)} tokens, {rows.size} of {K} rows, {len(experts)} experts' weight grads")
    ret_bits = to_np(o["packed"][torch.from_numpy(rows).to("cuda")]) if rows.size else \
        np.zeros((0, w.d), np.uint16)
    ret_v = oracle.bf16_bits_to_f64(ret_bits)
    dret_r, dw_r = oracle.combine_backward(dyv, ret_v, dest, w32, rows=rows)
    dw_g = to_np(g["dw"])
    _rel_close(dw_g[tokens], dw_r[tokens], 1e-4, "dw")
    dl_r = oracle.route_backward(logits[tokens], idx[tokens], dw_r[tokens], w.tau, AUX, load,
                                 batch=B)
    dl_g = to_np(g["dlogits"])
    _rel_close(dl_g[tokens], dl_r, 1e-4, "dlogits")
    dXp_r, gr = oracle.expert_ffn_backward(inp["x"], ps, eo, w.e_begin, w.e_end, inp["W1"],
                                           inp["W2"], inp["W3"], w.act, dret_r, rows=rows,
                                           experts=experts)
    dx_r = oracle.dispatch_backward(dXp_r, dest, tokens=tokens, rows=rows)
    dx_r += oracle.gate_backward(inp["x"][tokens], inp["Wg"], dl_r)[0]
    if res:
        dx_r += dyv[tokens]
    dxg = to_np(g["dx"])[tokens]
    dxv = oracle.bf16_bits_to_f64(dxg) if dxg.dtype == np.uint16 else dxg.astype(np.float64)
    assert_bf16_close(dxv, dx_r, what=f"dx ({len(tokens)} tokens)")
    for e in experts:
        for name, gi in (("dW1", 0), ("dW2", 1), ("dW3", 2)):
            R = gr[e][gi]
            if R is None:
                continue
            G = to_np(g[name][e - w.e_begin])
            if np.abs(R).max() == 0:
                assert np.abs(G).max() == 0
            else:
                assert rel_err(G, R) <= 2e-2, (name, e, rel_err(G, R))
    if experts:
        say(f"  dW of experts {experts[:4]}{'...' if len(experts) > 4 else ''}: within 2e-2")
    if full:
        _, dWg_r, db_r = oracle.gate_backward(inp["x"], inp["Wg"], dl_r)
        _rel_close(to_np(g["dWg"]), dWg_r, 1e-4, "dWg")
        _rel_close(to_np(g["dbias"]), db_r, 1e-4, "dbias")
    return g


@pytest.mark.parametrize("name", ["toy", "uniform", "skewed"])
def test_backward_chain_full(name):
    w = moe_synth.WORKLOADS[name]
    say(f"[backward chain {name}] all tokens, all experts")
    _chain(w)


def test_backward_chain_residual():
    w = SMALL["gelu_drops_residual"]
    say("[backward chain residual]")
    _chain(w, res=True)


@pytest.mark.parametrize("name,ntok,experts", [("mixtral", 48, [3]),
                                               ("ep_share", 48, [0, 17, 31])])
def test_backward_chain_sampled(name, ntok, experts):
    """Full-size matrix-core-bound workloads: sampled tokens' dx, dw and
    dlogits, and the weight gradients of a few experts (every row of
    theirs)."""
    w = moe_synth.WORKLOADS[name]
    say(f"[backward chain {name}] sampled")
    _chain(w, tokens_n=ntok, experts=experts)


def test_backward_empty_batch():
    import torch
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.Workload("bwd_empty", B=0, d=64, E=8, k=2, c=1.0, f=96, act="swiglu",
                           x_dtype="bf16", n_ranks=1, e_begin=0, e_end=8, router_std=None)
    p = problem_for(w)
    inp = moe_synth.make_inputs(moe_synth.scaled(w, B=4))
    wp = packed_weights_for_gpu(p, inp)
    wpb = _wpb(p, inp)
    e0 = torch.empty(0, dtype=torch.int16, device="cuda")
    saved = dict(logits=torch.empty(0, device="cuda"), topk_idx=torch.empty(0, dtype=torch.int32,
                 device="cuda"), topk_w=torch.empty(0, device="cuda"),
                 dest=torch.empty(0, dtype=torch.int32, device="cuda"),
                 expert_load=torch.zeros(8, dtype=torch.int32, device="cuda"),
                 expert_offset=torch.zeros(9, dtype=torch.int32, device="cuda"),
                 pack_src=torch.empty(0, dtype=torch.int32, device="cuda"), packed=e0)
    g = moe.backward(p, e0, to_dev(inp["Wg"]), wp, wpb, saved, e0, aux_coef=AUX)
    torch.cuda.synchronize()
    for key in ("dWg", "dbias", "dW1", "dW2", "dW3"):
        assert float(g[key].abs().max()) == 0.0, key


@pytest.mark.parametrize("name", ["gelu_drops_residual", "swiglu_remote", "swiglu_f32_x",
                                  "uniform", "ep_share"])
def test_backward_saved_z_matches_recompute(name):
    """The forward's saved pre-activations (save_z) are the bits the
    backward's recompute produces (the same kernel, the same order), so
    every gradient is bit-identical either way, and saving them leaves the
    forward's outputs unchanged."""
    import torch
    import expert_token_routing_fp32_amd as moe
    w = SMALL[name] if name in SMALL else moe_synth.WORKLOADS[name]
    res = name == "gelu_drops_residual"
    say(f"[saved z {name}]")
    inp = moe_synth.make_inputs(w)
    p = problem_for(w, add_residual=res)
    x, Wg = to_dev(inp["x"]), to_dev(inp["Wg"])
    bias = None if inp["bias"] is None else to_dev(inp["bias"])
    wp = packed_weights_for_gpu(p, inp)
    wpb = _wpb(p, inp)
    y0, o0 = moe.forward(p, x, Wg, bias, wp, outputs=True)
    y1, o1 = moe.forward(p, x, Wg, bias, wp, outputs=True, save_z=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    K = int(o0["expert_offset"][-1])  # rows past the kept ones are not written
    for key in ("dest", "expert_offset", "pack_src", "packed"):
        a, b = (o0[key], o1[key]) if key in ("dest", "expert_offset") else \
            (o0[key][:K], o1[key][:K])
        assert torch.equal(a, b), key
    dy = to_dev(_dy(w, seed=9))
    g0 = moe.backward(p, x, Wg, wp, wpb, o0, dy, aux_coef=AUX)
    g1 = moe.backward(p, x, Wg, wp, wpb, o1, dy, aux_coef=AUX)
    torch.cuda.synchronize()
    for key, v in g0.items():
        if v is not None:
            assert torch.equal(v, g1[key]), key
    say(f"  {len(g0)} gradients bit-identical with the saved pre-activations "
        f"({moe.saved_z_bytes(p) / 1e6:.1f} MB)")


def _shared_weights(rng, d, f, swiglu):
    """bf16 bits of a shared expert's W1s [1, d, f], W3s, W2s [1, f, d]."""
    def bf(a):
        return oracle.f32_to_bf16_bits_rne(a.astype(np.float32))
    W1 = bf(rng.normal(scale=d ** -0.5, size=(1, d, f)))
    W3 = bf(rng.normal(scale=d ** -0.5, size=(1, d, f))) if swiglu else None
    W2 = bf(rng.normal(scale=f ** -0.5, size=(1, f, d)))
    return W1, W3, W2


@pytest.mark.parametrize("B,d,f,E,act,fs,sact", [(256, 64, 96, 8, "gelu", 128, "gelu"),
                                                 (300, 72, 40, 8, "swiglu", 200, "swiglu"),
                                                 (4096, 1024, 1024, 64, "gelu", 1024, "swiglu")])
def test_backward_shared(B, d, f, E, act, fs, sact):
    """moe_backward_shared: the routed gradients are moe_backward's bit for
    bit (the shared expert changes only dx); the shared expert's weight
    gradients and its part of dx against the oracle's expert FFN backward
    with every token as the one expert's rows and dy as its output
    gradient; and every gradient bit-identical when the forward saved both
    experts' pre-activations."""
    import torch
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.Workload(name="bshared", B=B, d=d, E=E, k=2, c=1.0, f=f, act=act,
                           x_dtype="bf16", n_ranks=1, e_begin=0, e_end=E, router_std=None,
                           zipf_bias=False, tau=1.0, seed=4)
    say(f"[backward shared] B={B} d={d} f={f} E={E} {act}, shared f={fs} {sact}")
    inp = moe_synth.make_inputs(w)
    S1, S3, S2 = _shared_weights(np.random.default_rng(9), d, fs, sact == "swiglu")
    p = problem_for(w)
    ps = moe.shared_problem(p, fs, sact)
    x, Wg = to_dev(inp["x"]), to_dev(inp["Wg"])
    wp = packed_weights_for_gpu(p, inp)
    wpb = _wpb(p, inp)
    d3 = None if S3 is None else to_dev(S3)
    wps = moe.pack_weights(ps, to_dev(S1), d3, to_dev(S2))
    wpsb = moe.pack_weights_bwd(ps, to_dev(S1), d3, to_dev(S2))
    y, o = moe.forward(p, x, Wg, None, wp, outputs=True, shared=(ps, wps))
    dy = _dy(w, seed=7)
    g = moe.backward(p, x, Wg, wp, wpb, o, to_dev(dy), aux_coef=AUX, shared=(ps, wps, wpsb))
    g0 = moe.backward(p, x, Wg, wp, wpb, o, to_dev(dy), aux_coef=AUX)
    torch.cuda.synchronize()
    for key in ("dW1", "dW2", "dW3", "dWg", "dbias", "dlogits", "dw"):
        if g0[key] is not None:
            assert torch.equal(g[key], g0[key]), key
    dXs, grs = oracle.expert_ffn_backward(inp["x"], np.arange(B), np.array([0, B]), 0, 1, S1, S2,
                                          S3, sact, _x_vals(dy))
    for name, gi in (("dW1s", 0), ("dW2s", 1), ("dW3s", 2)):
        if grs[0][gi] is None:
            assert g[name] is None
            continue
        e = rel_err(to_np(g[name]), grs[0][gi])
        say(f"  {name}: max|d|/max|ref| = {e:.3e}")
        assert e <= 2e-2, (name, e)
    dx_s = oracle.bf16_bits_to_f64(to_np(g["dx"]))
    dx_0 = oracle.bf16_bits_to_f64(to_np(g0["dx"]))
    assert_bf16_close(dx_s, dx_0 + dXs, what="dx with the shared expert")
    # with both experts' pre-activations saved by the forward: the same bits
    y1, o1 = moe.forward(p, x, Wg, None, wp, outputs=True, shared=(ps, wps), save_z=True)
    g1 = moe.backward(p, x, Wg, wp, wpb, o1, to_dev(dy), aux_coef=AUX, shared=(ps, wps, wpsb))
    torch.cuda.synchronize()
    assert torch.equal(y, y1)
    for key, v in g.items():
        if v is not None:
            assert torch.equal(v, g1[key]), key
