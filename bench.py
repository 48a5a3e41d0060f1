#!/usr/bin/env python3
"""Throughput of the MoE-layer forward on one MI355X.

A step is one moe_forward over the batch: fp32 gate, softmax + top-k,
capacity-limited slot assignment with drops, pack into per-expert (per-rank)
segments, grouped expert MLP on bf16 MFMA, weighted combine.  Inputs are
seeded synthetic tensors of the workload's shape, resident in HBM before the
timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload ep_share] [--cold]
                  [--no-cpu-baseline] [--gpus 1]

The default workload is the largest one that fits one GPU: one rank's share
of a 256-expert top-8 expert-parallel layer (32768 tokens, d = 7168, 32
local SwiGLU experts of 2048), whose expert GEMM is matrix-core bound.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "MoE-layer tokens/s on 1 MI355X; expert GEMM % MFMA peak; dispatch % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
# fp32 FMA without packed-math forms: 256 CU x 4 SIMD x 16 lanes x 2 FLOP x 2.4 GHz
VALU_FP32_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ep_share")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MB buffer before every step (flushes L2 and MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-tokens", type=int, default=0, metavar="N",
                    help="tokens of the CPU oracle's sample (default: the whole batch up to "
                         "4096 tokens, else the first 1024 tokens as a batch of their own)")
    ap.add_argument("--no-cold-pass", action="store_true",
                    help="skip the extra cold-cache pass of the default run")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times: the "
                         "kernel of known traffic that HBM byte counters are scaled by")
    ap.add_argument("--routing", default="token", choices=["token", "expert_choice"],
                    help="expert_choice: every expert picks its top-C tokens "
                         "(moe_forward_expert_choice; all experts local)")
    ap.add_argument("--overflow", default="drop", choices=["drop", "next"],
                    help="next: assignments past capacity are redirected to the token's "
                         "next-best experts (moe_problem_t.overflow)")
    ap.add_argument("--shared-expert", type=int, default=0, metavar="F",
                    help="add a shared expert of hidden size F (same activation) on every "
                         "token: moe_forward_shared (bf16 workloads)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward captured once in a HIP graph and replayed "
                         "(torch.cuda.CUDAGraph; token-choice routing): the rate without the "
                         "host's per-launch cost, reported beside the eager one")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's backward pass (moe_backward, for a seeded output "
                         "gradient, on one forward's saved outputs) instead of the forward")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: the forward does not save the first expert GEMM's "
                         "pre-activations, and the backward recomputes them")
    ap.add_argument("--aux-coef", type=float, default=0.01,
                    help="auxiliary load-balancing loss coefficient of --backward")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only time the HBM streaming probes (libmoe_probe.so): read-only, "
                         "write-only and copy over 4 GiB buffers")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only time the matrix-core ceiling probe (libmoe_probe.so) with random "
                         "and with near-constant bf16 operands")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor library's dense bf16 GEMM (torch.matmul) at the "
                         "expert FFN's shapes, for comparison with the grouped expert GEMM")
    return ap.parse_args()


def mfma_probe(torch) -> dict:
    """What the matrix cores sustain with the expert GEMM's inner-loop mix and no
    memory traffic, one workgroup per CU.  After about a second of untimed
    launches (clocks settle), the two operand cases alternate, 5 launches per
    round, 3 rounds each; reported per case: mean over the rounds and the
    slowest and fastest round."""
    import ctypes
    here = os.path.dirname(os.path.abspath(__file__))
    lib = ctypes.CDLL(os.path.join(here, "expert_token_routing_fp32_amd", "libmoe_probe.so"))
    lib.moe_probe_mfma.restype = ctypes.c_int
    lib.moe_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.moe_probe_mfma_flop.restype = ctypes.c_double
    lib.moe_probe_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4000
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def call(rnd):
        assert lib.moe_probe_mfma(ctypes.c_void_p(out.data_ptr()), grid, iters, rnd,
                                  ctypes.c_void_p(stream.cuda_stream)) == 0

    for i in range(200):
        call(i & 1)
    torch.cuda.synchronize()
    cases = (("random_bf16", 1), ("constant_bf16", 0))
    rounds = {name: [] for name, _ in cases}
    for _ in range(3):
        for name, rnd in cases:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                call(rnd)
            e1.record(stream)
            torch.cuda.synchronize()
            rounds[name].append(e0.elapsed_time(e1) / 5 * 1e-3)
    flop = lib.moe_probe_mfma_flop(grid, iters)
    res = {}
    for name, sec in rounds.items():
        mean = sum(sec) / len(sec)
        res[name] = {"us_per_launch": round(mean * 1e6, 1),
                     "us_rounds": [round(x * 1e6, 1) for x in sec],
                     "tflops": round(flop / mean / 1e12, 1),
                     "frac_of_2500": round(flop / mean / 1e12 / 2500.0, 4)}
    return {"mfma_probe": res, "grid": grid, "iters": iters, "tflop_per_launch": round(flop / 1e12, 3),
            "warmup_launches": 200, "rounds": 3, "launches_per_round": 5}


def library_gemm(torch) -> dict:
    """The vendor library's dense bf16 GEMM (torch.matmul, which dispatches
    to hipBLASLt on this image) at the expert FFN's shapes: the kept local
    rows of the EP-share and mixtral workloads as one dense matrix (a single
    large GEMM, easier than the grouped one), and one EP-share expert's
    rows.  Random normal bf16 operands, the right operand contiguous
    [K][N]; 5 untimed calls, then 20 timed between HIP events.  A
    comparison point for the grouped expert GEMM, not part of the layer."""
    shapes = [("ep_share GEMM1 (W1 and W3), all kept local rows", 32976, 7168, 4096),
              ("ep_share GEMM2 (W2), all kept local rows", 32976, 2048, 7168),
              ("ep_share GEMM1, one expert's rows", 1031, 7168, 4096),
              ("mixtral GEMM1 (W1 and W3), all kept rows", 16264, 4096, 28672),
              ("mixtral GEMM2 (W2), all kept rows", 16264, 14336, 4096)]
    g = torch.Generator(device="cuda:0")
    g.manual_seed(0)
    res = []
    for name, M, K, N in shapes:
        a = torch.randn(M, K, device="cuda:0", dtype=torch.bfloat16, generator=g)
        b = torch.randn(K, N, device="cuda:0", dtype=torch.bfloat16, generator=g).contiguous()
        for _ in range(5):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 20 * 1e3
        tf = 2.0 * M * N * K / us / 1e6
        res.append({"shape": name, "M": M, "K": K, "N": N, "us": round(us, 1),
                    "tflops": round(tf, 1), "frac_of_2500": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        del a, b, c
    return {"library_gemm": res, "calls": 20, "warmup_calls": 5, "dtype": "bf16",
            "operands": "random normal"}


def hbm_probe(torch) -> dict:
    """What HBM sustains for plain streams on this part: read-only (each
    16-byte chunk loaded once, folded into a register), write-only and copy
    kernels over 4 GiB buffers (far past the 256 MB MALL), one grid of 8
    workgroups per CU.  After 5 untimed launches of each, 3 rounds of 5
    launches per kind; reported: mean over the rounds in GB/s (bytes moved:
    read, written, or read + written)."""
    import ctypes
    here = os.path.dirname(os.path.abspath(__file__))
    lib = ctypes.CDLL(os.path.join(here, "expert_token_routing_fp32_amd", "libmoe_probe.so"))
    lib.moe_probe_hbm.restype = ctypes.c_int
    lib.moe_probe_hbm.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    nbytes = 4 << 30
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    grid = torch.cuda.get_device_properties(0).multi_processor_count * 8
    out = torch.empty(grid * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def call(mode):
        rc = lib.moe_probe_hbm(mode, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                               nbytes, ctypes.c_void_p(out.data_ptr()), grid,
                               ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, rc

    kinds = (("read", 0, 1), ("write", 1, 1), ("copy", 2, 2))
    for _, mode, _ in kinds:
        for _ in range(5):
            call(mode)
    torch.cuda.synchronize()
    res = {}
    for name, mode, mult in kinds:
        rounds = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                call(mode)
            e1.record(stream)
            torch.cuda.synchronize()
            rounds.append(e0.elapsed_time(e1) / 5 * 1e-3)
        mean = sum(rounds) / len(rounds)
        res[name] = {"us_per_launch": round(mean * 1e6, 1),
                     "gbs": round(mult * nbytes / mean / 1e9, 1),
                     "gbs_rounds": [round(mult * nbytes / r / 1e9, 1) for r in rounds],
                     "frac_of_8000": round(mult * nbytes / mean / 1e9 / HBM_PEAK_GBS, 4)}
    return {"hbm_probe": res, "bytes": nbytes, "grid": grid, "rounds": 3,
            "launches_per_round": 5}


def algorithmic(w, keep: np.ndarray, eo: np.ndarray, dest: np.ndarray) -> dict:
    """Bytes / FLOPs the method must move / compute for one forward, per step.
    With bf16 tokens the forward's first GEMM reads the local rows from x
    itself (counted in the FFN's bytes), so the pack reads the tokens with a
    kept choice on another rank and writes only those rows."""
    B, d, E, k, f = w.B, w.d, w.E, w.k, w.f
    sx = 2 if w.x_dtype == "bf16" else 4
    K = int(eo[-1])
    lo, hi = int(eo[w.e_begin]), int(eo[w.e_end])
    Kloc = hi - lo
    nmat = 3 if w.act == "swiglu" else 2
    active_local = int(sum(1 for e in range(w.e_begin, w.e_end) if eo[e + 1] > eo[e]))
    t_act = int(keep.any(axis=1).sum())
    gather = w.x_dtype == "bf16" and B * d * 2 < (1 << 32) and w.e_end > w.e_begin
    if gather:
        remote = (dest >= 0) & ((dest < lo) | (dest >= hi))
        pack_bytes = int(remote.any(axis=1).sum()) * d * sx + 2.0 * d * int(remote.sum())
    else:
        pack_bytes = t_act * d * sx + 2.0 * d * K
    return dict(
        gate_flop=2.0 * B * d * E,
        gate_bytes=B * d * sx + 4.0 * d * E + 4.0 * B * E,
        route_bytes=B * (4.0 * E + 8.0 * k),
        slot_bytes=B * k * (4 + 4 + 1 + 4) + 4.0 * K,
        pack_bytes=pack_bytes,
        ffn_flop=2.0 * d * f * nmat * Kloc,
        ffn_bytes=active_local * 2.0 * d * f * nmat + 4.0 * d * Kloc,
        combine_bytes=2.0 * d * K + B * d * sx + 8.0 * k * B,
        K=K, Kloc=Kloc, t_act=t_act, active_local=active_local,
    )


def algorithmic_ec(w, sel_t: np.ndarray, R: int) -> dict:
    """The same accounting for expert-choice routing (R = E * min(C, B)
    rows): the router writes the probabilities and reads them once per
    choice pass; the pack reads each chosen token once and writes R rows;
    the combine reads R rows, the token's sel entries and writes y."""
    B, d, E, f = w.B, w.d, w.E, w.f
    sx = 2 if w.x_dtype == "bf16" else 4
    nmat = 3 if w.act == "swiglu" else 2
    t_act = int((sel_t >= 0).any(axis=0).sum())
    active = int((sel_t >= 0).any(axis=1).sum())
    return dict(
        gate_flop=2.0 * B * d * E,
        gate_bytes=B * d * sx + 4.0 * d * E + 4.0 * B * E,
        route_bytes=B * E * (4.0 + 4.0 + 4.0) + R * 8.0,
        slot_bytes=0.0,
        pack_bytes=t_act * d * sx + 2.0 * d * R,
        ffn_flop=2.0 * d * f * nmat * R,
        ffn_bytes=active * 2.0 * d * f * nmat + 4.0 * d * R,
        combine_bytes=2.0 * d * R + B * d * sx + 4.0 * B * E,
        K=R, Kloc=R, t_act=t_act, active_local=active,
    )


def measured_traffic(workload: str):
    """HBM bytes per expert-FFN call from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by a plain copy's reading), or None when there is
    no record for this workload or the GEMM sources changed since it was
    taken (the record keeps a hash of them)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if rec is None:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    return rec["expert_ffn_bytes"] if h.hexdigest()[:16] == rec["src_sha256_16"] else None


def cpu_baseline(w, inp, budget_s: float, shared=None, ec: bool = False,
                 overflow: str = "drop", n_tokens: int = 0) -> dict:
    """The oracle as it stands, timed on the host on a bounded sample: the
    first n_tokens tokens of the batch as a batch of their own (same weights,
    capacity from their own count), whole forward, repeated for about
    budget_s seconds; tokens/s = sample tokens x runs / time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    if n_tokens <= 0:
        n_tokens = w.B if w.B <= 4096 else 1024
    n_tokens = min(n_tokens, w.B)
    xs = inp["x"][:n_tokens]
    sh = None
    if shared is not None:
        sh = shared
    reps, t_tot = 0, 0.0
    while reps == 0 or (t_tot < budget_s and reps < 20):
        t0 = time.perf_counter()
        if ec:
            oracle.forward_expert_choice(xs, inp["Wg"], inp["bias"], inp["W1"], inp["W3"],
                                         inp["W2"], k=w.k, c=w.c, act=w.act, tau=w.tau)
        else:
            oracle.forward(xs, inp["Wg"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                           k=w.k, c=w.c, act=w.act, n_ranks=w.n_ranks, e_begin=w.e_begin,
                           e_end=w.e_end, tau=w.tau, shared=sh, overflow=overflow)
        t_tot += time.perf_counter() - t0
        reps += 1
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    what = (f"the whole {w.name} batch ({w.B} tokens)" if n_tokens == w.B else
            f"the first {n_tokens} of the {w.B} tokens of the {w.name} batch as a batch of "
            f"their own (same weights and shape, capacity from {n_tokens} tokens)")
    return {"value": round(n_tokens * reps / t_tot, 1), "unit": "tokens/s",
            "cores": int(threads), "kind": "oracle", "cpu_model": model,
            "sample": f"{what}, oracle forward run {reps} times ({t_tot:.1f} s), float64 NumPy, "
                      "input generation excluded"}


def graph_replay(args, p, x, Wg, bias, wp, y, ws, shared, w, torch, moe):
    """The same forward captured once in a HIP graph (the library enqueues
    kernels only) and replayed: warmup replays, then the timed ones between
    synchronisations, as the eager steps.  Only the host's launch cost
    differs, which is what bounds the small workloads."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(p, x, Wg, bias, wp, y=y, ws=ws, shared=shared)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(p, x, Wg, bias, wp, y=y, ws=ws, shared=shared)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    log(f"[bench] graph replay: {sec * 1e3:.4f} ms/step")
    return {"ms_per_step": round(sec * 1e3, 4), "tokens_per_s": round(w.B / sec, 1),
            "timing": f"{args.steps} replays of one captured forward between two "
                      "synchronisations (wall clock)"}


def bench_backward(args, w, inp, p, x, Wg, bias, wp, wpb, torch, moe, dev, shared=None):
    """The backward pass: one forward (outputs kept, and the first expert
    GEMM's pre-activations unless --recompute), then moe_backward on those
    outputs and a seeded output gradient, W untimed + K timed calls
    bracketed by synchronizations; then the same number of calls of the
    stage entry points with events between them for the breakdown.  With a
    shared expert (``shared`` = (ps, packed, packed backward copy)) the
    chain is moe_backward_shared, and the shared expert's FFN backward is a
    stage of its own in the breakdown."""
    bf16 = w.x_dtype == "bf16"
    y, o = moe.forward(p, x, Wg, bias, wp, outputs=True, save_z=not args.recompute,
                       shared=None if shared is None else shared[:2])
    rs = np.random.default_rng(w.seed + 7)
    dy_np = rs.standard_normal((w.B, w.d)).astype(np.float32)
    if bf16:
        import moe_synth
        dy = torch.from_numpy(moe_synth.f32_to_bf16_bits(dy_np).view(np.int16)).to(dev)
    else:
        dy = torch.from_numpy(dy_np).to(dev)
    if shared is None:
        nws = moe.workspace_bytes(p, "backward")
    else:
        nws = moe.lib().moe_backward_shared_workspace_bytes(ctypes.byref(p),
                                                           ctypes.byref(shared[0]))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        return moe.backward(p, x, Wg, wp, wpb, o, dy, aux_coef=args.aux_coef, ws=ws,
                            shared=shared)
    log(f"[bench] backward: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] backward: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps

    # breakdown: the stage calls of the same chain, events between them
    keys = ("combine", "route", "expert_ffn", "dispatch") + \
        (("shared_ffn",) if shared is not None else ()) + ("gate",)
    per = {k_: [] for k_ in keys}
    km = moe.max_kept(p)
    dret = torch.empty((max(km, 1), w.d), dtype=torch.int16, device=dev)
    dwb = torch.empty((w.B, w.k), dtype=torch.float32, device=dev)
    dlb = torch.empty((w.B, w.E), dtype=torch.float32, device=dev)
    accb = torch.empty((w.B, w.d), dtype=torch.float32, device=dev)
    ws_f = torch.empty(max(moe.workspace_bytes(p, "expert_ffn_backward"), 1), dtype=torch.uint8,
                       device=dev)
    ws_g = torch.empty(max(moe.workspace_bytes(p, "gate_backward"), 1), dtype=torch.uint8,
                       device=dev)
    if shared is not None:
        ps_ = shared[0]
        s_src = torch.arange(w.B, dtype=torch.int32, device=dev)
        s_eo = torch.tensor([0, w.B], dtype=torch.int32, device=dev)
        s_dret = torch.empty((w.B, w.d), dtype=torch.int16, device=dev)
        ws_s = torch.empty(max(moe.workspace_bytes(ps_, "expert_ffn_backward"), 1),
                           dtype=torch.uint8, device=dev)
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(keys) + 1)]
        ev[0].record()
        moe.combine_backward(p, dy, o["packed"], o["dest"], o["topk_w"], dret=dret, dw=dwb)
        ev[1].record()
        moe.route_backward(p, o["logits"], o["topk_idx"], dwb, o["expert_load"], args.aux_coef,
                           dlogits=dlb)
        ev[2].record()
        moe.expert_ffn_backward(p, x, o["pack_src"], o["expert_offset"], wp, wpb, dret, ws=ws_f,
                                z=o.get("z"))
        ev[3].record()
        moe.dispatch_backward(p, dret, o["dest"], dy if p.add_residual else None, dx_acc=accb)
        ev[4].record()
        if shared is not None:
            s_dret.copy_(dy)
            moe.expert_ffn_backward(ps_, x, s_src, s_eo, shared[1], shared[2], s_dret, ws=ws_s,
                                    z=o.get("z_shared"))
            ev[5].record()
        moe.gate_backward(p, x, Wg, dlb, dx_acc=accb, ws=ws_g)
        ev[len(keys)].record()
        torch.cuda.synchronize()
        for i, k_ in enumerate(keys):
            per[k_].append(ev[i].elapsed_time(ev[i + 1]) * 1e-3)
    med = {k_: float(np.median(v)) for k_, v in per.items()}
    keep = o["keep"].cpu().numpy().astype(bool)
    eo = o["expert_offset"].cpu().numpy()
    alg = algorithmic(w, keep, eo, o["dest"].cpu().numpy())
    # the expert backward's algorithmic work: dX and the weight gradients,
    # twice the forward's FLOPs (recomputed pre-activations, with
    # --recompute, are extra)
    ffn_flop = 2.0 * alg["ffn_flop"]
    t_ffn = med["expert_ffn"]
    tfl = ffn_flop / t_ffn / 1e12
    sx = 2 if bf16 else 4
    K, B, d, E, k = alg["K"], w.B, w.d, w.E, w.k
    # combine backward: dy once, ret and dret rows once each, dw; dispatch
    # backward: dXp rows once, dx_acc written (fp32)
    comb_bytes = B * d * sx + 2.0 * 2 * d * K + 8.0 * B * k
    disp_bytes = 2.0 * d * K + 4.0 * B * d
    out = {
        "metric": "MoE-layer backward tokens/s on 1 MI355X (moe_backward)",
        "value": round(w.B / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} d={w.d} E={w.E} top-{w.k} c={w.c} "
                               f"{w.act} f={w.f} x={w.x_dtype} D={w.n_ranks} "
                               f"local experts [{w.e_begin},{w.e_end}), backward, "
                               f"aux_coef={args.aux_coef}",
                   "global_batch": w.B,
                   "pre_activations": "recomputed" if args.recompute else
                                      "saved by the forward (moe_forward_out_t.z)",
                   **({"shared_expert_f": shared[0].f} if shared is not None else {})},
        "roofline": {"bound": "mfma", "achieved": round(tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None,
                     "kernel": "expert FFN backward (moe_expert_ffn_backward: dH with the "
                               "activation derivative, dX, weight gradients, re-layouts"
                               + (", and the recomputed pre-activations)" if args.recompute
                                  else ")"),
                     "algorithmic_flop": ffn_flop, "avg_launch_us": round(t_ffn * 1e6, 2),
                     "timing": "HIP events around the stage call, median over the steps"},
        "breakdown": {
            **{f"{k_}_backward_us": round(v * 1e6, 2) for k_, v in med.items()},
            "combine_backward_hbm_frac": round(comb_bytes / med["combine"] / 1e9 / HBM_PEAK_GBS,
                                               4),
            "dispatch_backward_hbm_frac": round(disp_bytes / med["dispatch"] / 1e9
                                                / HBM_PEAK_GBS, 4),
            "gate_backward_mfma_frac": round(
                4.0 * B * d * E * 3 / med["gate"] / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "timing": "stage calls with events between them (host enqueue gaps included), "
                      "median over the steps",
            "kept": K, "kept_local": alg["Kloc"],
        },
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on one GPU's share of tokens; it has no cross-GPU step)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))
        return

    if args.mfma_probe:
        print(json.dumps(mfma_probe(torch)))
        return

    if args.hbm_probe:
        print(json.dumps(hbm_probe(torch)))
        return

    if args.library_gemm:
        print(json.dumps(library_gemm(torch)))
        return

    import expert_token_routing_fp32_amd as moe
    import moe_synth

    w = moe_synth.WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: generating inputs")
    inp = moe_synth.make_inputs(w)
    dev = torch.device("cuda:0")

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    bf16 = w.x_dtype == "bf16"
    x = d16(inp["x"]) if bf16 else torch.from_numpy(inp["x"]).to(dev)
    Wg = torch.from_numpy(inp["Wg"]).to(dev)
    bias = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(dev)
    W1 = d16(inp["W1"] if bf16 else inp["W1_bits"])
    W2 = d16(inp["W2"] if bf16 else inp["W2_bits"])
    W3 = None
    if w.act == "swiglu":
        W3 = d16(inp["W3"] if bf16 else inp["W3_bits"])
    p = moe.make_problem(B=w.B, d=w.d, E=w.E, k=w.k, c=w.c, f=w.f, act=w.act, x_dtype=w.x_dtype,
                         n_ranks=w.n_ranks, e_begin=w.e_begin, e_end=w.e_end, tau=w.tau,
                         overflow=args.overflow)
    # expert weights in the library's blocked layout: a one-time conversion at
    # load, like reading a checkpoint -- not part of the timed step
    wp = moe.pack_weights(p, W1, W3, W2)
    del W1, W2, W3
    ws = torch.empty(moe.workspace_bytes(p, "forward"), dtype=torch.uint8, device=dev)
    ec = args.routing == "expert_choice"
    if ec:
        if w.e_begin != 0 or w.e_end != w.E:
            raise SystemExit("--routing expert_choice needs every expert local "
                             f"({w.name} runs experts [{w.e_begin},{w.e_end}) of {w.E})")
        if args.shared_expert or args.overflow != "drop":
            raise SystemExit("--shared-expert and --overflow go with token-choice routing")
        ws = torch.empty(moe.workspace_bytes(p, "forward_expert_choice"), dtype=torch.uint8,
                         device=dev)
    shared = None
    fs = args.shared_expert
    if fs > 0:
        if not bf16:
            raise SystemExit("--shared-expert needs a bf16 workload")
        # seeded bf16 weights of std 1/sqrt(fan_in), like the routed experts
        rs = np.random.default_rng(w.seed + 1000)

        def bw(shape, fan_in):
            a = rs.normal(scale=fan_in ** -0.5, size=shape).astype(np.float32)
            return d16(moe_synth.f32_to_bf16_bits(a))
        S1 = bw((1, w.d, fs), w.d)
        S3 = bw((1, w.d, fs), w.d) if w.act == "swiglu" else None
        S2 = bw((1, fs, w.d), fs)
        ps = moe.shared_problem(p, fs, w.act)
        shared = (ps, moe.pack_weights(ps, S1, S3, S2))
        shared_bwd = (ps, shared[1], moe.pack_weights_bwd(ps, S1, S3, S2)) if args.backward \
            else None
        shared_np = (S1.cpu().numpy().view(np.uint16)[0],
                     None if S3 is None else S3.cpu().numpy().view(np.uint16)[0],
                     S2.cpu().numpy().view(np.uint16)[0])
        del S1, S2, S3
        ws = torch.empty(moe.lib().moe_forward_shared_workspace_bytes(
            ctypes.byref(p), ctypes.byref(ps)), dtype=torch.uint8, device=dev)
    y = torch.empty((w.B, w.d), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    if args.backward:
        if ec or args.overflow != "drop":
            raise SystemExit("--backward goes with token-choice routing and the drop policy")
        W1 = d16(inp["W1"] if bf16 else inp["W1_bits"])
        W2 = d16(inp["W2"] if bf16 else inp["W2_bits"])
        W3 = d16(inp["W3"] if bf16 else inp["W3_bits"]) if w.act == "swiglu" else None
        wpb = moe.pack_weights_bwd(p, W1, W3, W2)
        del W1, W2, W3
        bench_backward(args, w, inp, p, x, Wg, bias, wp, wpb, torch, moe, dev,
                       shared_bwd if shared is not None else None)
        return
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None

    # HIP events recorded by the library on its stream.  moe_forward takes
    # every one from the dispatch timestamps of a stage's own kernels (start
    # of its first, end of its last: no marker packets), so each stage's
    # time is its kernels' and the gaps between launches are measured apart.
    # A launch that carries an event gets a gap of a few microseconds on
    # each side (the runtime's timestamping); launches without events follow
    # each other with none.  So the timed steps carry events only on every
    # `stride`-th step (at least 10 sampled steps), and those time one GEMM
    # of the expert FFN each, by its own start and end: GEMM1 on the even
    # sampled steps, GEMM2 on the odd ones; the FFN's time is the sum of the
    # two means.  A second run of as many steps records every event on every
    # step for the breakdown (there too the FFN is the sum of its GEMMs).
    # The expert-choice forward records marker events at its stage
    # boundaries, except around the expert FFN (one pair).
    if ec:
        n_ev = 6
        ffn_parts = [(3, 4)]
        pairs = {"gate": (0, 1), "route": (1, 2), "dispatch": (2, 3), "expert_ffn": (3, 4),
                 "combine": (4, 5)}
        gaps = {}
    else:
        n_ev = moe.N_STAGE_EVENTS
        ffn_parts = [moe.FFN_GEMM_EVENTS["gemm1"], moe.FFN_GEMM_EVENTS["gemm2"]]
        pairs, gaps = moe.STAGE_EVENTS, moe.LAUNCH_GAPS
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    stride = max(1, args.steps // 10)
    sampled = list(range(0, args.steps, stride))
    # which FFN part each sampled step times (all parts on one step when
    # there are fewer sampled steps than parts)
    part_of = {i: [ffn_parts[n % len(ffn_parts)]] if len(sampled) >= len(ffn_parts) else ffn_parts
               for n, i in enumerate(sampled)}
    ffn_only = [[r[j] if any(j in ab for ab in part_of[i]) else None for j in range(n_ev)]
                if i in part_of else None for i, r in enumerate(evs)]

    def step(ev=None):
        if flush is not None:
            flush.fill_(1)
        if ec:
            moe.forward_expert_choice(p, x, Wg, bias, wp, y=y, ws=ws, stage_events=ev)
        else:
            moe.forward(p, x, Wg, bias, wp, y=y, ws=ws, stage_events=ev, shared=shared)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ffn_only[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / args.steps
    flush_s = 0.0
    if flush is not None:
        # the cold protocol's 512 MB write runs before every step, inside the
        # timed loop: time the same number of writes alone and take them out
        f0 = time.perf_counter()
        for _ in range(args.steps):
            flush.fill_(1)
        torch.cuda.synchronize()
        flush_s = (time.perf_counter() - f0) / args.steps
        sec_per_step -= flush_s
    t_ffn_live = 0.0
    for ab in ffn_parts:
        on = [i for i in sampled if ab in part_of[i]]
        t_ffn_live += sum(evs[i][ab[0]].elapsed_time(evs[i][ab[1]]) for i in on) / len(on) * 1e-3
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    def mean_s(ab):
        return sum(r[ab[0]].elapsed_time(r[ab[1]]) for r in evs) / len(evs) * 1e-3

    stage_s = {name: mean_s(ab) for name, ab in pairs.items()}
    stage_s["expert_ffn"] = sum(mean_s(ab) for ab in ffn_parts)
    gap_s = {name: mean_s(ab) for name, ab in gaps.items()}
    # per-step device time of the breakdown run: first kernel's start to the
    # last kernel's end (events from the dispatches), median over the steps
    last_ev = n_ev - 1
    warm_med = float(np.median([r[0].elapsed_time(r[last_ev]) for r in evs])) * 1e-3
    cold_med = None
    if not args.cold and not args.no_cold_pass:
        # the same steps after a 512 MB write each (flushes L2 and the MALL);
        # the write runs before the first event, so it is not in the time
        fl = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for i in range(args.steps):
            fl.fill_(1)
            if ec:
                moe.forward_expert_choice(p, x, Wg, bias, wp, y=y, ws=ws, stage_events=evs[i])
            else:
                moe.forward(p, x, Wg, bias, wp, y=y, ws=ws, stage_events=evs[i], shared=shared)
        torch.cuda.synchronize()
        cold_med = float(np.median([r[0].elapsed_time(r[last_ev]) for r in evs])) * 1e-3
        del fl
    t_gate, t_route, t_disp, t_comb = (stage_s[k] for k in ("gate", "route", "dispatch", "combine"))
    log(f"[bench] {sec_per_step * 1e3:.3f} ms/step; " +
        ", ".join(f"{k} {v * 1e6:.1f} us" for k, v in stage_s.items()))

    if ec:
        _, o = moe.forward_expert_choice(p, x, Wg, bias, wp, outputs=True)
        torch.cuda.synchronize()
        alg = algorithmic_ec(w, o["sel_t"].cpu().numpy(), moe.expert_choice_rows(p))
    else:
        _, o = moe.forward(p, x, Wg, bias, wp, outputs=True, shared=shared)
        torch.cuda.synchronize()
        keep = o["keep"].cpu().numpy().astype(bool)
        eo = o["expert_offset"].cpu().numpy()
        alg = algorithmic(w, keep, eo, o["dest"].cpu().numpy())
    if shared is not None:
        # the shared expert on every token: its weights once, x read, its
        # output rows written (FFN stage) and read again by the combine
        nmat_s = 3 if w.act == "swiglu" else 2
        alg["ffn_flop"] += 2.0 * w.B * w.d * fs * nmat_s
        alg["ffn_bytes"] += 2.0 * w.d * fs * nmat_s + 4.0 * w.B * w.d
        alg["combine_bytes"] += 2.0 * w.B * w.d

    # routing-health signals of the same batch (an optional call after the
    # forward, not part of the timed step): timed alone with events
    health = {}
    if not ec:
        ws_stats = torch.empty(max(moe.workspace_bytes(p, "routing_stats"), 1),
                               dtype=torch.uint8, device=dev)
        for _ in range(3):
            hs = moe.routing_stats(p, o["logits"], o["expert_load"], o["expert_count"],
                                   ws=ws_stats)
        # events around each call (the three launches of one call are
        # enqueued back to back by the library; between calls the host
        # allocates the outputs), median of 20
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(20)]
        for e0, e1 in pairs:
            e0.record()
            hs = moe.routing_stats(p, o["logits"], o["expert_load"], o["expert_count"],
                                   ws=ws_stats)
            e1.record()
        torch.cuda.synchronize()
        t_stats = float(np.median([a.elapsed_time(b) for a, b in pairs])) * 1e-3
        hsum = hs["summary"].cpu().numpy()
        # algorithmic bytes: the logits once, the counts, the per-expert outputs
        stats_bytes = w.B * w.E * 4 + w.E * (2 * 4 + 4 * 4) + 5 * 8
        health = {
            "routing_stats_us": round(t_stats * 1e6, 2),
            "routing_stats_hbm_frac": round(stats_bytes / t_stats / 1e9 / HBM_PEAK_GBS, 4),
            "routing_health": {"aux_loss": round(float(hsum[0]), 6),
                               "entropy_nats": round(float(hsum[1]), 5),
                               "load_entropy_nats": round(float(hsum[2]), 5),
                               "dropped": int(hsum[3]), "kept": int(hsum[4])},
        }

    ffn_gbs = alg["ffn_bytes"] / t_ffn_live / 1e9
    ffn_tflops = alg["ffn_flop"] / t_ffn_live / 1e12
    ffn_bound = "hbm" if alg["ffn_bytes"] / (HBM_PEAK_GBS * 1e9) >= \
        alg["ffn_flop"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    if ffn_bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(ffn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ffn_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(ffn_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ffn_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    if ffn_bound == "mfma":
        # the attainable ceiling measured live, after the timed steps: the same
        # MFMA instruction mix with random bf16 operands and no memory traffic
        probe = mfma_probe(torch)["mfma_probe"]["random_bf16"]
        roof["attainable"] = {"achieved_frac": round(ffn_tflops / probe["tflops"], 4),
                              "ceiling_tflops": probe["tflops"],
                              "ceiling": "the expert GEMM's MFMA mix (libmoe_probe.so) with "
                                         "random bf16 operands and no memory traffic, one "
                                         "workgroup per CU, timed in this run"}
    roof["traffic"] = measured_traffic(w.name) if shared is None and not ec else None
    roof["kernel"] = "expert FFN: grouped_gemm_kernel GEMM1 (act) + GEMM2, one moe_expert_ffn call"
    roof["algorithmic_bytes"] = alg["ffn_bytes"]
    roof["algorithmic_flop"] = alg["ffn_flop"]
    roof["avg_launch_us"] = round(t_ffn_live * 1e6, 2)
    roof["timing"] = (("HIP events from the start and end of the expert FFN's kernels" if ec else
                       "HIP events from the start and end of each of the expert FFN's two GEMM "
                       "kernels (GEMM1 on half the sampled steps, GEMM2 on the other half; the "
                       "FFN is the sum of their means)") +
                      " (hipExtLaunchKernelGGL on the forward's stream), sampled on "
                      f"{len(sampled)} of the {args.steps} timed steps "
                      f"({'all' if stride == 1 else f'every {stride}th'})")

    rpc_bytes = alg["route_bytes"] + alg["slot_bytes"] + alg["pack_bytes"] + alg["combine_bytes"]
    rpc_t = t_route + t_disp + t_comb
    breakdown = {
        "step_ms_median": {
            "warm": round(warm_med * 1e3, 4),
            **({"cold": round(cold_med * 1e3, 4)} if cold_med is not None else {}),
            "timing": ("first kernel's dispatch start to the last kernel's end, median over "
                       f"{args.steps} steps; warm: the breakdown run; cold: the same steps, "
                       "each after a 512 MB write that flushes L2 and the MALL")},
        "timing": ("stage events over a second run of the same number of steps"
                   + ("" if ec else ": each stage from its own kernels' dispatch start and end")),
        "expert_ffn_us_breakdown_run": round(stage_s["expert_ffn"] * 1e6, 2),
        "gate_us": round(t_gate * 1e6, 2),
        # bf16 activations: three bf16 MFMA products per fp32 multiply-add
        # (exact split of the fp32 weights); fp32 activations: vector ALUs
        "gate_frac": round(alg["gate_flop"] * 3 / t_gate / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        if bf16 else round(alg["gate_flop"] / t_gate / 1e12 / VALU_FP32_PEAK_TFLOPS, 4),
        "gate_peak": "bf16 MFMA x3" if bf16 else "fp32 VALU",
        "route_us": round(t_route * 1e6, 2),
        "dispatch_us": round(t_disp * 1e6, 2),
        "expert_ffn_us": round(t_ffn_live * 1e6, 2),
        "combine_us": round(t_comb * 1e6, 2),
        **({"launch_gaps_us": {k: round(v * 1e6, 2) for k, v in gap_s.items()}} if gap_s else {}),
        "expert_gemm_tflops": round(ffn_tflops, 1),
        "expert_gemm_mfma_frac": round(ffn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "expert_gemm_hbm_frac": round(ffn_gbs / HBM_PEAK_GBS, 4),
        "route_pack_combine_gbs": round(rpc_bytes / rpc_t / 1e9, 1),
        "route_pack_combine_hbm_frac": round(rpc_bytes / rpc_t / 1e9 / HBM_PEAK_GBS, 4),
        "kept": alg["K"], "kept_local": alg["Kloc"],
        "dropped": None if ec else int(w.B * w.k - alg["K"]),
        **health,
    }
    if args.graph and not ec:
        breakdown["graph_replay"] = graph_replay(args, p, x, Wg, bias, wp, y, ws, shared, w,
                                                 torch, moe)
    if ec:
        breakdown["expert_choice"] = {"rows": alg["K"], "tokens_chosen": alg["t_act"],
                                      "route_us_is": "router probabilities + the choice",
                                      "dispatch_us_is": "gather pack"}

    out = {
        "metric": METRIC,
        "value": round(w.B / sec_per_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} d={w.d} E={w.E} top-{w.k} c={w.c} "
                               f"{w.act} f={w.f} x={w.x_dtype} D={w.n_ranks} "
                               f"local experts [{w.e_begin},{w.e_end})"
                               + (f" + shared expert f={fs}" if shared is not None else "")
                               + (", expert-choice routing" if ec else "")
                               + (", overflow to the next-best expert"
                                  if args.overflow == "next" else ""),
                   "global_batch": w.B, "cache": "cold" if args.cold else "warm",
                   **({"cold_flush_ms_excluded": round(flush_s * 1e3, 4)} if args.cold else {})},
        "roofline": roof,
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds,
                                           shared_np if shared is not None else None, ec,
                                           args.overflow, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
