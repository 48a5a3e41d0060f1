"""Shared plumbing for the GPU parity tests: device transfers, tolerances,
per-workload cached inputs and oracle results.  The expected values come from
``oracle`` only; the HIP path's outputs are only ever compared, never fed
back into the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np

import moe_synth
import oracle

# tolerances of the parity tests: fp32 logits and gate weights |d| <= 1e-5 max(1, |ref|);
# bf16 tensors max|d| / max|ref| <= 2e-2
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def dev():
    return torch().device("cuda:0")


def to_dev(a: np.ndarray):
    t = torch()
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_np(t, dtype=None):
    a = t.detach().cpu()
    if a.dtype in (torch().bfloat16,):
        a = a.view(torch().int16)
    a = a.numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.astype(dtype)


def bf16_np(a_bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f64(a_bits)


def assert_f32_close(got, ref, tol=TOL_F32, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    m = float(err.max()) if err.size else 0.0
    say(f"  {what}: max |d|/max(1,|ref|) = {m:.3e} (tol {tol:g})")
    assert m <= tol, f"{what}: {m} > {tol}"


def assert_sum_close(got, ref, abs_sum, n, what=""):
    """fp32 results that are sums of n products: within TOL_F32 max(1, |ref|)
    or within the standard forward error bound of an n-term fp32 sum,
    gamma_n = n u / (1 - n u) (u = 2^-24) times the sum of the terms'
    magnitudes (abs_sum, same shape), whichever is larger -- a fixed bound
    does not scale with the length of the contraction."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    u = 2.0 ** -24
    gamma = n * u / (1.0 - n * u)
    tol = np.maximum(TOL_F32 * np.maximum(1.0, np.abs(ref)), gamma * np.asarray(abs_sum))
    r = np.abs(got - ref) / tol
    m = float(r.max()) if r.size else 0.0
    say(f"  {what}: max |d| / bound = {m:.3f} (n = {n})")
    assert m <= 1.0, f"{what}: {m} of the bound"


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.abs(ref).max()) if ref.size else 0.0
    num = float(np.abs(got - ref).max()) if ref.size else 0.0
    return num / den if den > 0 else num


def assert_bf16_close(got, ref, tol=TOL_BF16, what=""):
    e = rel_err(got, ref)
    say(f"  {what}: max|d|/max|ref| = {e:.3e} (tol {tol:g})")
    assert e <= tol, f"{what}: {e} > {tol}"


def problem_for(w: moe_synth.Workload, **over):
    import expert_token_routing_fp32_amd as moe
    kw = dict(B=w.B, d=w.d, E=w.E, k=w.k, c=w.c, f=w.f, act=w.act, x_dtype=w.x_dtype,
              n_ranks=w.n_ranks, e_begin=w.e_begin, e_end=w.e_end, tau=w.tau)
    kw.update(over)
    return moe.make_problem(**kw)


def weights_for_gpu(inp: dict):
    """bf16 weights as the GEMM consumes them (toy: rounded copies)."""
    w = inp["workload"]
    if w.x_dtype == "bf16":
        return inp["W1"], inp["W3"], inp["W2"]
    return inp["W1_bits"], inp["W3_bits"], inp["W2_bits"]


def packed_weights_for_gpu(p, inp: dict):
    """Upload the bf16 expert weights and put them in the library's blocked
    layout (moe_pack_weights), as a model would once at load time."""
    import expert_token_routing_fp32_amd as moe
    W1, W3, W2 = weights_for_gpu(inp)
    return moe.pack_weights(p, to_dev(W1), None if W3 is None else to_dev(W3), to_dev(W2))


@functools.lru_cache(maxsize=2)
def workload(name: str, **scale):
    """Inputs plus the oracle's routing/dispatch results (no FFN)."""
    w = moe_synth.WORKLOADS[name]
    if scale:
        w = moe_synth.scaled(w, **scale)
    inp = moe_synth.make_inputs(w)
    ref = oracle.forward(inp["x"], inp["Wg"], inp["bias"], None, None, None, k=w.k, c=w.c,
                         act=w.act, n_ranks=w.n_ranks, e_begin=w.e_begin, e_end=w.e_end,
                         tau=w.tau)
    return w, inp, ref


def sample_rows(eo: np.ndarray, e_begin: int, e_end: int, n: int, seed: int = 0) -> np.ndarray:
    """Packed rows of local experts: first and last row of every local expert
    with rows, plus random ones (at most ~n)."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(e_begin, e_end):
        a, b = int(eo[e]), int(eo[e + 1])
        if b > a:
            rows += [a, b - 1]
    lo, hi = int(eo[e_begin]), int(eo[e_end])
    if hi > lo:
        rows += list(rng.integers(lo, hi, size=max(0, n - len(rows))))
    rows = np.unique(np.array(rows, dtype=np.int64))
    if rows.size > n:
        rows = np.sort(rng.choice(rows, size=n, replace=False))
    return rows


def row_slices(M: int, bm: int = 256):
    """The row slices the grouped expert GEMM cuts an expert's M rows into:
    ceil(M / bm) slices over which the ceil(M / 32) row blocks of 32 are
    dealt as evenly as possible (the first nb % nsl slices take one block
    more).  Returns [(first_row, n_rows)], relative to the expert's first
    row.  Used only to choose which rows a test compares."""
    if M <= 0:
        return []
    nsl = (M + bm - 1) // bm
    nb = (M + 31) // 32
    q, r = divmod(nb, nsl)
    out = []
    for m in range(nsl):
        m0 = 32 * (m * q + min(m, r))
        span = 32 * (q + (1 if m < r else 0))
        out.append((m0, min(M - m0, span)))
    return out


def tile_rows(eo: np.ndarray, e_begin: int, e_end: int, seed: int = 0):
    """Packed rows that hit every tile of the grouped expert GEMM: for every
    local expert, the first and last row of each of its row slices and one
    random row of each of its 32-row blocks (every sampled row is compared
    over all output columns, so every output tile of that slice is hit).
    Returns (rows, stats) with the counts of experts, slices and blocks."""
    rng = np.random.default_rng(seed)
    rows = []
    n_exp = n_sl = n_blk = 0
    for e in range(e_begin, e_end):
        a, b = int(eo[e]), int(eo[e + 1])
        M = b - a
        if M <= 0:
            continue
        n_exp += 1
        for m0, n in row_slices(M):
            n_sl += 1
            rows += [a + m0, a + m0 + n - 1]
        for b0 in range(0, M, 32):
            n_blk += 1
            rows.append(a + b0 + int(rng.integers(0, min(32, M - b0))))
    rows = np.unique(np.array(rows, dtype=np.int64))
    return rows, dict(experts=n_exp, slices=n_sl, blocks=n_blk, rows=int(rows.size))


def assert_bf16_close_per_expert(got, ref, rows, eo, e_begin, e_end, tol=TOL_BF16, what=""):
    """The bf16 tolerance on the whole tensor and on each expert's rows alone
    (a small-magnitude expert cannot hide behind a large one)."""
    assert_bf16_close(got, ref, tol, what)
    worst, we = 0.0, -1
    for e in range(e_begin, e_end):
        m = (rows >= int(eo[e])) & (rows < int(eo[e + 1]))
        if m.any():
            r = rel_err(got[m], ref[m])
            if r > worst:
                worst, we = r, e
            assert r <= tol, f"{what}: expert {e}: {r} > {tol}"
    say(f"  {what}: worst expert {we}: max|d|/max|ref| = {worst:.3e}")
