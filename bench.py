#!/usr/bin/env python3
"""Throughput of the MoE-layer forward on one MI355X.

A step is one moe_forward over the batch: fp32 gate, softmax + top-k,
capacity-limited slot assignment with drops, pack into per-expert (per-rank)
segments, grouped expert MLP on bf16 MFMA, weighted combine.  Inputs are
seeded synthetic tensors of the workload's shape, resident in HBM before the
timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload uniform] [--cold]
                  [--no-cpu-baseline] [--gpus 1]
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
    ap.add_argument("--workload", default="uniform")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MB buffer before every step (flushes L2 and MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only time the matrix-core ceiling probe (libmoe_probe.so) with random "
                         "and with near-constant bf16 operands")
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


def algorithmic(w, keep: np.ndarray, eo: np.ndarray) -> dict:
    """Bytes / FLOPs the method must move / compute for one forward, per step."""
    B, d, E, k, f = w.B, w.d, w.E, w.k, w.f
    sx = 2 if w.x_dtype == "bf16" else 4
    K = int(eo[-1])
    lo, hi = int(eo[w.e_begin]), int(eo[w.e_end])
    Kloc = hi - lo
    nmat = 3 if w.act == "swiglu" else 2
    active_local = int(sum(1 for e in range(w.e_begin, w.e_end) if eo[e + 1] > eo[e]))
    t_act = int(keep.any(axis=1).sum())
    return dict(
        gate_flop=2.0 * B * d * E,
        gate_bytes=B * d * sx + 4.0 * d * E + 4.0 * B * E,
        route_bytes=B * (4.0 * E + 8.0 * k),
        slot_bytes=B * k * (4 + 4 + 1 + 4) + 4.0 * K,
        pack_bytes=t_act * d * sx + 2.0 * d * K,
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
                 overflow: str = "drop") -> dict:
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    reps, t_tot = 0, 0.0
    while reps == 0 or (t_tot < budget_s and reps < 20):
        t0 = time.perf_counter()
        if ec:
            oracle.forward_expert_choice(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W3"],
                                         inp["W2"], k=w.k, c=w.c, act=w.act, tau=w.tau)
        else:
            oracle.forward(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                           k=w.k, c=w.c, act=w.act, n_ranks=w.n_ranks, e_begin=w.e_begin,
                           e_end=w.e_end, tau=w.tau, shared=shared, overflow=overflow)
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
    return {"value": round(w.B * reps / t_tot, 1), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model,
            "sample": f"the whole {w.name} batch ({w.B} tokens), oracle forward run {reps} times "
                      f"({t_tot:.1f} s), float64 NumPy, input generation excluded"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer has no cross-GPU step in this build)", file=sys.stderr)
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
        S1 = bw((1, fs, w.d), w.d)
        S3 = bw((1, fs, w.d), w.d) if w.act == "swiglu" else None
        S2 = bw((1, w.d, fs), fs)
        ps = moe.shared_problem(p, fs, w.act)
        shared = (ps, moe.pack_weights(ps, S1, S3, S2))
        shared_np = (S1.cpu().numpy().view(np.uint16)[0],
                     None if S3 is None else S3.cpu().numpy().view(np.uint16)[0],
                     S2.cpu().numpy().view(np.uint16)[0])
        del S1, S2, S3
        ws = torch.empty(moe.lib().moe_forward_shared_workspace_bytes(
            ctypes.byref(p), ctypes.byref(ps)), dtype=torch.uint8, device=dev)
    y = torch.empty((w.B, w.d), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None

    # HIP events recorded by the library on its stream.  moe_forward takes
    # every one from the dispatch timestamps of a stage's own kernels (start
    # of its first, end of its last: no marker packets), so each stage's
    # time is its kernels' and the gaps between launches are measured apart.
    # The expert-choice forward records marker events at its stage
    # boundaries, except around the expert FFN.  The timed steps record only
    # the FFN pair, and only on every `stride`-th step (at least 10 sampled
    # steps); a second run of as many steps records them all on every step
    # for the breakdown.
    if ec:
        n_ev, ffn_ev = 6, (3, 4)
        pairs = {"gate": (0, 1), "route": (1, 2), "dispatch": (2, 3), "expert_ffn": (3, 4),
                 "combine": (4, 5)}
        gaps = {}
    else:
        n_ev, ffn_ev = moe.N_STAGE_EVENTS, moe.STAGE_EVENTS["expert_ffn"]
        pairs, gaps = moe.STAGE_EVENTS, moe.LAUNCH_GAPS
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    stride = max(1, args.steps // 10)
    sampled = list(range(0, args.steps, stride))
    ffn_only = [[r[j] if j in ffn_ev else None for j in range(n_ev)] if i % stride == 0 else None
                for i, r in enumerate(evs)]

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
    a, b = ffn_ev
    t_ffn_live = sum(evs[i][a].elapsed_time(evs[i][b]) for i in sampled) / len(sampled) * 1e-3
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    def mean_s(ab):
        return sum(r[ab[0]].elapsed_time(r[ab[1]]) for r in evs) / len(evs) * 1e-3

    stage_s = {name: mean_s(ab) for name, ab in pairs.items()}
    gap_s = {name: mean_s(ab) for name, ab in gaps.items()}
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
        alg = algorithmic(w, keep, eo)
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
    roof["traffic"] = measured_traffic(w.name) if shared is None and not ec else None
    roof["kernel"] = "expert FFN: grouped_gemm_kernel GEMM1 (act) + GEMM2, one moe_expert_ffn call"
    roof["algorithmic_bytes"] = alg["ffn_bytes"]
    roof["algorithmic_flop"] = alg["ffn_flop"]
    roof["avg_launch_us"] = round(t_ffn_live * 1e6, 2)
    roof["timing"] = ("HIP events taken from the start of the expert FFN's first kernel and "
                      "the end of its last (hipExtLaunchKernelGGL on the forward's stream), "
                      f"averaged over {len(sampled)} of the {args.steps} timed steps "
                      f"({'all' if stride == 1 else f'every {stride}th'})")

    rpc_bytes = alg["route_bytes"] + alg["slot_bytes"] + alg["pack_bytes"] + alg["combine_bytes"]
    rpc_t = t_route + t_disp + t_comb
    breakdown = {
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
                                           args.overflow)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
