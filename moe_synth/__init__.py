"""Seeded synthetic workloads for one mixture-of-experts layer.

This module only *draws inputs*: it holds the five workload shapes and the
seeded random generators that fill them.  It computes nothing that the MoE
layer itself computes (no logits, no softmax, no capacity, no routing), so the
CPU oracle (``oracle/``) and the HIP path can both be fed from it without
sharing any of the method's arithmetic.

Shapes and value distributions follow the workloads the pages describe:

* ``toy``      -- the worked example of "Expert Parallelism" (theinfinity.ai,
                  capacity paragraph and its figure): 6 tokens, 8 experts on 4
                  devices, top-2, capacity factor 1.25.
* ``uniform``  -- 64 experts as in the 8-GPU / 64-expert trace of "Expert
                  Parallelism and the All-to-All Bottleneck" (section "The
                  All-to-All Communication Pattern").
* ``mixtral``  -- 8 experts, top-2 (narrativegoldmine.com, "Major Variants and
                  Families", top-k routing).
* ``skewed``   -- 128 experts, top-2 (inferensys.com glossary, first example)
                  with a Zipf routing bias so that a few hot experts overflow.
* ``ep_share`` -- 256 experts, top-8 (narrativegoldmine.com, "Major Variants
                  and Families", fine-grained routing); one rank's share of an
                  8-rank expert-parallel layer.

Storage conventions (the layout in memory, shared by both sides because it is
the *input format*, not arithmetic):

* ``x``   [B, d]: float32 for the toy workload, bf16 bits (uint16) otherwise.
* ``Wg``  [d, E] float32; router logits are ``x @ Wg (+ bias)``.
* ``W1``, ``W3`` [E_loc, d, f] and ``W2`` [E_loc, f, d]: each expert matrix is
  stored [in, out] row-major, as the workloads print them (``W1[d x f]``,
  ``W2[f x d]``), so one expert computes ``act(x @ W1) @ W2`` on a row x.
  bf16 bits, except the toy workload, which keeps float32 originals in ``W*``
  and their bf16 round-to-nearest-even copies in ``W*_bits``.
* ``bias`` [E] float32 or None.

Random numbers: NumPy PCG64 streams derived from ``SeedSequence(seed)``; one
child stream per tensor and, for expert weights, one grandchild stream per
expert, so an expert's weights do not depend on how many experts are drawn.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get_workload", "make_inputs",
           "f32_to_bf16_bits", "scaled"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # tokens on this GPU
    d: int                 # hidden size
    E: int                 # experts in the layer
    k: int                 # experts per token
    c: float               # capacity factor
    f: int                 # expert FFN inner size
    act: str               # "gelu" or "swiglu"
    x_dtype: str           # "f32" or "bf16" (x and y)
    n_ranks: int           # D: ranks the experts are spread over
    e_begin: int           # experts whose FFN runs on this GPU: [e_begin, e_end)
    e_end: int
    router_std: Optional[float]   # None -> 1/sqrt(d)
    zipf_bias: bool = False       # per-expert bias 1.5*ln(Zipf(s=1.2) prob of rank e+1)
    tau: float = 1.0
    seed: int = 0

    @property
    def n_local(self) -> int:
        return self.e_end - self.e_begin


WORKLOADS = {
    "toy": Workload("toy", B=6, d=16, E=8, k=2, c=1.25, f=32, act="gelu",
                    x_dtype="f32", n_ranks=4, e_begin=0, e_end=8, router_std=0.5),
    "uniform": Workload("uniform", B=4096, d=1024, E=64, k=2, c=1.25, f=4096,
                        act="gelu", x_dtype="bf16", n_ranks=1, e_begin=0,
                        e_end=64, router_std=0.02),
    "mixtral": Workload("mixtral", B=8192, d=4096, E=8, k=2, c=1.0, f=14336,
                        act="swiglu", x_dtype="bf16", n_ranks=1, e_begin=0,
                        e_end=8, router_std=None),
    "skewed": Workload("skewed", B=16384, d=2048, E=128, k=2, c=1.0, f=1408,
                       act="gelu", x_dtype="bf16", n_ranks=1, e_begin=0,
                       e_end=128, router_std=None, zipf_bias=True),
    "ep_share": Workload("ep_share", B=32768, d=7168, E=256, k=8, c=1.25, f=2048,
                         act="swiglu", x_dtype="bf16", n_ranks=8, e_begin=0,
                         e_end=32, router_std=None),
}

ORDER = ["toy", "uniform", "mixtral", "skewed", "ep_share"]


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller test shapes)."""
    return dataclasses.replace(w, **changes)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits.

    Used only to *store* drawn inputs as bf16.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _normal_rows(ss: np.random.SeedSequence, rows: int, cols: int, std: float,
                 to_bf16: bool, block: int = 4096) -> np.ndarray:
    """[rows, cols] normals, drawn in row blocks (one grandchild stream per
    block) on a thread pool; optionally stored as bf16 bits."""
    nblk = (rows + block - 1) // block
    kids = ss.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.uint16 if to_bf16 else np.float32)

    def one(i):
        r0, r1 = i * block, min(rows, (i + 1) * block)
        a = _normal(kids[i], (r1 - r0, cols), std)
        out[r0:r1] = f32_to_bf16_bits(a) if to_bf16 else a

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(nblk)))
    return out


def _expert_weights(ss: np.random.SeedSequence, w: Workload, rows: int,
                    cols: int, std: float, to_bf16: bool) -> np.ndarray:
    """[n_local, rows, cols]; expert e (global index) uses grandchild stream e."""
    kids = ss.spawn(w.E)
    out = np.empty((w.n_local, rows, cols), dtype=np.uint16 if to_bf16 else np.float32)

    def one(i):
        a = _normal(kids[w.e_begin + i], (rows, cols), std)
        out[i] = f32_to_bf16_bits(a) if to_bf16 else a

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(w.n_local)))
    return out


def zipf_bias(E: int, s: float = 1.2, scale: float = 1.5) -> np.ndarray:
    """b_e = scale * ln(p_{e+1}), p_r = r^-s / sum_{r'=1..E} r'^-s (float32)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return (scale * np.log(p)).astype(np.float32)


def make_inputs(w: Workload, with_weights: bool = True) -> dict:
    """Draw every input of workload ``w`` (deterministic in ``w.seed``)."""
    ss = np.random.SeedSequence(w.seed)
    s_x, s_g, s_w1, s_w3, s_w2 = ss.spawn(5)
    bf16 = w.x_dtype == "bf16"
    inp = {"workload": w}
    inp["x"] = _normal_rows(s_x, w.B, w.d, 1.0, to_bf16=bf16)
    rstd = w.router_std if w.router_std is not None else 1.0 / math.sqrt(w.d)
    inp["Wg"] = _normal(s_g, (w.d, w.E), rstd)
    inp["bias"] = zipf_bias(w.E) if w.zipf_bias else None
    if with_weights:
        sd1 = 1.0 / math.sqrt(w.d)
        sd2 = 1.0 / math.sqrt(w.f)
        inp["W1"] = _expert_weights(s_w1, w, w.d, w.f, sd1, to_bf16=bf16)
        inp["W3"] = (_expert_weights(s_w3, w, w.d, w.f, sd1, to_bf16=bf16)
                     if w.act == "swiglu" else None)
        inp["W2"] = _expert_weights(s_w2, w, w.f, w.d, sd2, to_bf16=bf16)
        if not bf16:
            # the expert GEMM consumes bf16 operands: keep rounded copies
            for n in ("W1", "W3", "W2"):
                inp[n + "_bits"] = None if inp[n] is None else f32_to_bf16_bits(inp[n])
    return inp
