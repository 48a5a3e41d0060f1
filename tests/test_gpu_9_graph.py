"""moe_forward and moe_backward captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed.

The library enqueues kernels only (no memset or copy nodes, no host reads of
device data), so a caller can capture the whole layer once and replay it.
Every replay must reproduce the eager forward bit for bit: the outputs are
overwritten between replays (eager work of the program's own, with an eager
forward and a synchronisation in between), so a replay that skipped or reused
a stage would show.  The shapes cover the toy layer (fp32 activations), the
weight-streaming expert GEMMs (uniform routing) and the matrix-core-bound
ones with rank segments and local experts (an EP-share shape scaled down);
the backward, a small uniform layer and the scaled EP share with the saved
pre-activations."""
import numpy as np
import pytest

import moe_synth
from _helpers import say, to_dev, to_np

pytestmark = pytest.mark.gpu

SHAPES = {
    "toy": dict(),
    "uniform": dict(),
    "ep_share_small": dict(B=4096, d=512, E=32, k=8, f=512, n_ranks=8, e_begin=0, e_end=4),
}
BASE = {"toy": "toy", "uniform": "uniform", "ep_share_small": "ep_share"}
# outputs compared in full (rows of pack_src / packed past the kept count are
# not written by the forward)
FULL = ("logits", "topk_idx", "topk_w", "pos", "keep", "dest", "expert_load",
        "expert_count", "expert_offset", "rank_offset")


def _bits(t):
    a = to_np(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_graph_replays_match_eager(name):
    import torch
    import expert_token_routing_fp32_amd as moe
    w = moe_synth.WORKLOADS[BASE[name]]
    if SHAPES[name]:
        w = moe_synth.scaled(w, **SHAPES[name])
    inp = moe_synth.make_inputs(w)
    p = moe.make_problem(B=w.B, d=w.d, E=w.E, k=w.k, c=w.c, f=w.f, act=w.act,
                         x_dtype=w.x_dtype, n_ranks=w.n_ranks, e_begin=w.e_begin,
                         e_end=w.e_end, tau=w.tau)
    bf16 = w.x_dtype == "bf16"
    x = to_dev(inp["x"])
    Wg = to_dev(inp["Wg"])
    bias = None if inp["bias"] is None else to_dev(inp["bias"])
    W1 = to_dev(inp["W1"] if bf16 else inp["W1_bits"])
    W2 = to_dev(inp["W2"] if bf16 else inp["W2_bits"])
    W3 = None if w.act != "swiglu" else to_dev(inp["W3"] if bf16 else inp["W3_bits"])
    wp = moe.pack_weights(p, W1, W3, W2)
    ws = torch.empty(moe.workspace_bytes(p, "forward"), dtype=torch.uint8, device="cuda")

    y_e, o_e = moe.forward(p, x, Wg, bias, wp, outputs=True, ws=ws)
    torch.cuda.synchronize()
    K = int(to_np(o_e["expert_offset"])[-1])
    say(f"  {name}: B={w.B} d={w.d} E={w.E} k={w.k} kept {K}")

    # capture (one eager call on the side stream first, as torch requires)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(p, x, Wg, bias, wp, outputs=True, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_g, o_g = moe.forward(p, x, Wg, bias, wp, outputs=True, ws=ws)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between the replays: clobber the graph's outputs and run
        # an eager forward on the shared workspace
        y_g.fill_(0)
        for key in o_g:
            o_g[key].fill_(-1 if o_g[key].dtype != torch.uint8 else 255)
        moe.forward(p, x, Wg, bias, wp, ws=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y_g), _bits(y_e), err_msg=f"replay {rep}: y")
        for key in FULL:
            np.testing.assert_array_equal(_bits(o_g[key]), _bits(o_e[key]),
                                          err_msg=f"replay {rep}: {key}")
        np.testing.assert_array_equal(to_np(o_g["pack_src"])[:K], to_np(o_e["pack_src"])[:K],
                                      err_msg=f"replay {rep}: pack_src")
        np.testing.assert_array_equal(to_np(o_g["packed"])[:K], to_np(o_e["packed"])[:K],
                                      err_msg=f"replay {rep}: packed")
    say(f"  {name}: 4 replays equal the eager forward bit for bit")


BWD_SHAPES = {
    "uniform_small": ("uniform", dict(B=1024, d=256, E=16, k=2, f=512, e_end=16), False),
    "ep_share_small_saved_z": ("ep_share", SHAPES["ep_share_small"], True),
}


@pytest.mark.parametrize("name", list(BWD_SHAPES))
def test_backward_graph_replays_match_eager(name):
    """moe_backward captured once and replayed: every gradient bit-identical
    to the eager backward's on the same saved forward outputs."""
    import torch
    import expert_token_routing_fp32_amd as moe
    base, change, save_z = BWD_SHAPES[name]
    w = moe_synth.scaled(moe_synth.WORKLOADS[base], **change)
    inp = moe_synth.make_inputs(w)
    p = moe.make_problem(B=w.B, d=w.d, E=w.E, k=w.k, c=w.c, f=w.f, act=w.act,
                         x_dtype=w.x_dtype, n_ranks=w.n_ranks, e_begin=w.e_begin,
                         e_end=w.e_end, tau=w.tau)
    x = to_dev(inp["x"])
    Wg = to_dev(inp["Wg"])
    W1, W2 = to_dev(inp["W1"]), to_dev(inp["W2"])
    W3 = None if w.act != "swiglu" else to_dev(inp["W3"])
    wp = moe.pack_weights(p, W1, W3, W2)
    wpb = moe.pack_weights_bwd(p, W1, W3, W2)
    _, o = moe.forward(p, x, Wg, None, wp, outputs=True, save_z=save_z)
    rng = np.random.default_rng(7)
    dy = to_dev(moe_synth.f32_to_bf16_bits(rng.standard_normal((w.B, w.d), dtype=np.float32)))
    ws = torch.empty(moe.workspace_bytes(p, "backward"), dtype=torch.uint8, device="cuda")
    g_e = moe.backward(p, x, Wg, wp, wpb, o, dy, aux_coef=0.01, ws=ws)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.backward(p, x, Wg, wp, wpb, o, dy, aux_coef=0.01, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_g = moe.backward(p, x, Wg, wp, wpb, o, dy, aux_coef=0.01, ws=ws)
    torch.cuda.synchronize()
    keys = [k_ for k_ in g_e if g_e[k_] is not None]
    say(f"  {name}: gradients {keys}")
    for rep in range(3):
        for k_ in keys:
            g_g[k_].fill_(-1)
        moe.backward(p, x, Wg, wp, wpb, o, dy, aux_coef=0.01, ws=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k_ in keys:
            np.testing.assert_array_equal(_bits(g_g[k_]), _bits(g_e[k_]),
                                          err_msg=f"replay {rep}: {k_}")
    say(f"  {name}: 3 replays equal the eager backward bit for bit")
