"""MI355X (gfx950) forward pass of one mixture-of-experts layer.

A thin Python face of the C ABI in include/moe.h (libmoe.so, built from
csrc/ by ``build.py``).  Tensors are torch tensors on a ROCm device; this
module only checks shapes and passes pointers and the current HIP stream --
every step of the layer runs in the library's kernels.  bf16 tensors may be
``torch.bfloat16`` or raw 16-bit patterns (``torch.int16``).

Steps ("Expert Parallelism", narrativegoldmine.com, "Formal Algorithm";
"Expert Parallelism and the All-to-All Bottleneck", "The Mechanism of Expert
Parallelism"): gate -> route -> dispatch (capacity, slots, pack) ->
expert_ffn -> combine; ``forward`` runs them back to back.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib as L
from ._lib import MoEError, Problem  # noqa: F401

__all__ = ["make_problem", "capacity", "problem_capacity", "max_kept", "validate",
           "workspace_bytes", "weights_bytes", "pack_weights", "gate", "route", "dispatch",
           "dispatch_noalloc",
           "expert_ffn", "combine", "unpack", "forward", "routing_stats", "shared_problem",
           "shared_ffn", "router_probs", "expert_choice", "expert_choice_pack",
           "expert_choice_combine", "forward_expert_choice", "expert_choice_rows",
           "combine_backward", "route_backward", "weights_bwd_bytes", "pack_weights_bwd",
           "expert_ffn_backward", "dispatch_backward", "gate_backward", "backward", "MoEError",
           "saved_z_bytes",
           "Problem", "lib", "FFN_GEMM_EVENTS"]


def lib():
    return L.load()


def make_problem(B: int, d: int, E: int, k: int, c: float = 1.0, f: int = 8,
                 act: str = "gelu", x_dtype: str = "bf16", C: int = -1, n_ranks: int = 1,
                 e_begin: int = 0, e_end: Optional[int] = None, tau: float = 1.0,
                 add_residual: bool = False, unavailable=None,
                 overflow: str = "drop") -> Problem:
    """``unavailable``: optional device tensor of E uint8 (or bool); a
    nonzero entry gives that expert capacity 0.  The problem keeps a
    reference to it.  ``overflow``: "drop", or "next" (forward only: dropped
    choices are redirected to the token's next-best experts)."""
    p = Problem(B=B, d=d, E=E, k=k, c=c, C=C, n_ranks=n_ranks, e_begin=e_begin,
                e_end=E if e_end is None else e_end, f=f,
                act={"gelu": L.MOE_GELU, "swiglu": L.MOE_SWIGLU}[act],
                x_dtype={"f32": L.MOE_F32, "bf16": L.MOE_BF16}[x_dtype], tau=tau,
                add_residual=int(bool(add_residual)),
                overflow={"drop": L.MOE_OVERFLOW_DROP, "next": L.MOE_OVERFLOW_NEXT}[overflow])
    set_unavailable(p, unavailable)
    return p


def set_unavailable(p: Problem, mask) -> None:
    """Attach (or with None, clear) the per-expert unavailable mask."""
    if mask is None:
        p.expert_unavailable = None
        p._mask = None
        return
    if mask.dtype == torch.bool:
        mask = mask.to(torch.uint8)
    if mask.dtype != torch.uint8 or not mask.is_cuda or mask.numel() != p.E:
        raise ValueError("unavailable must be a device uint8/bool tensor of E entries")
    mask = mask.contiguous()
    p._mask = mask
    p.expert_unavailable = mask.data_ptr()


def capacity(B: int, k: int, E: int, c: float) -> int:
    return lib().moe_capacity(B, k, E, c)


def problem_capacity(p: Problem) -> int:
    return lib().moe_problem_capacity(ctypes.byref(p))


def max_kept(p: Problem) -> int:
    return lib().moe_max_kept(ctypes.byref(p))


def validate(p: Problem) -> int:
    return lib().moe_validate(ctypes.byref(p))


def shared_problem(p: Problem, f: int, act: str = "swiglu") -> Problem:
    """The problem of a shared expert beside the routed layer p: same B and
    d, one expert that every token uses, its own f and activation."""
    return make_problem(B=p.B, d=p.d, E=1, k=1, c=1.0, f=f, act=act, x_dtype="bf16")


def workspace_bytes(p: Problem, op: str = "forward") -> int:
    o = {"dispatch": L.MOE_OP_DISPATCH, "ffn": L.MOE_OP_FFN, "forward": L.MOE_OP_FORWARD,
         "routing_stats": L.MOE_OP_ROUTING_STATS, "shared_ffn": L.MOE_OP_SHARED_FFN,
         "forward_expert_choice": L.MOE_OP_FORWARD_EXPERT_CHOICE,
         "expert_ffn_backward": L.MOE_OP_EXPERT_FFN_BACKWARD,
         "gate_backward": L.MOE_OP_GATE_BACKWARD, "backward": L.MOE_OP_BACKWARD}[op]
    return lib().moe_workspace_bytes(ctypes.byref(p), o)


def weights_bytes(p: Problem) -> int:
    return lib().moe_weights_bytes(ctypes.byref(p))


# ---------------------------------------------------------------------------
def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, numel: int, itemsize: int, dev=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != itemsize:
        raise ValueError(f"{name}: element size {t.element_size()} != {itemsize}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements < {numel}")


def _xsize(p: Problem) -> int:
    return 2 if p.x_dtype == L.MOE_BF16 else 4


def _ws(p: Problem, op: str, ws: Optional[torch.Tensor], device) -> torch.Tensor:
    n = workspace_bytes(p, op)
    if ws is None:
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    _need(ws, "ws", n, 1)
    return ws


def _check(p: Problem):
    st = validate(p)
    L.check(st, "problem")


def gate(p: Problem, x, Wg, bias=None, logits=None):
    _check(p)
    B, d, E = p.B, p.d, p.E
    _need(x, "x", B * d, _xsize(p))
    _need(Wg, "Wg", d * E, 4)
    if bias is not None:
        _need(bias, "bias", E, 4)
    if logits is None:
        logits = torch.empty((B, E), dtype=torch.float32, device=x.device)
    _need(logits, "logits", B * E, 4)
    L.check(lib().moe_gate(ctypes.byref(p), _p(x), _p(Wg), _p(bias), _p(logits), _stream()),
            "moe_gate")
    return logits


def route(p: Problem, logits, topk_idx=None, topk_w=None):
    _check(p)
    B, E, k = p.B, p.E, p.k
    _need(logits, "logits", B * E, 4)
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((B, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", B * k, 4)
    _need(topk_w, "topk_w", B * k, 4)
    L.check(lib().moe_route(ctypes.byref(p), _p(logits), _p(topk_idx), _p(topk_w), _stream()),
            "moe_route")
    return topk_idx, topk_w


def routing_stats(p: Problem, logits, expert_load, expert_count, ws=None) -> dict:
    """Routing-health signals from the logits and the dispatch counts:
    prob_mean, token_frac, utilization [E] float32, dropped [E] int32 and
    summary [5] float64 (aux loss, routing entropy, load entropy, dropped
    total, kept total), all device tensors."""
    _check(p)
    B, E = p.B, p.E
    dev = expert_load.device
    if B > 0:
        _need(logits, "logits", B * E, 4)
    _need(expert_load, "expert_load", E, 4)
    _need(expert_count, "expert_count", E, 4)
    o = dict(prob_mean=torch.empty(E, dtype=torch.float32, device=dev),
             token_frac=torch.empty(E, dtype=torch.float32, device=dev),
             utilization=torch.empty(E, dtype=torch.float32, device=dev),
             dropped=torch.empty(E, dtype=torch.int32, device=dev),
             summary=torch.empty(5, dtype=torch.float64, device=dev))
    out = L.RoutingStats(**{n: o[n].data_ptr() for n in o})
    ws = _ws(p, "routing_stats", ws, dev)
    L.check(lib().moe_routing_stats(ctypes.byref(p), _p(logits) if B > 0 else None,
                                    _p(expert_load), _p(expert_count), ctypes.byref(out), _p(ws),
                                    ws.numel(), _stream()), "moe_routing_stats")
    return o


def dispatch(p: Problem, x, topk_idx, ws=None) -> dict:
    """Slots, drops and the pack.  Returns every output as a device tensor;
    ``packed`` has max_kept(p) rows, of which expert_offset[E] are written."""
    _check(p)
    B, d, E, k, D = p.B, p.d, p.E, p.k, p.n_ranks
    dev = topk_idx.device
    _need(x, "x", B * d, _xsize(p))
    _need(topk_idx, "topk_idx", B * k, 4)
    km = max_kept(p)
    i32 = dict(dtype=torch.int32, device=dev)
    o = dict(pos=torch.empty((B, k), **i32), keep=torch.empty((B, k), dtype=torch.uint8, device=dev),
             dest=torch.empty((B, k), **i32), expert_load=torch.empty(E, **i32),
             expert_count=torch.empty(E, **i32), expert_offset=torch.empty(E + 1, **i32),
             rank_offset=torch.empty(D + 1, **i32), pack_src=torch.empty(max(km, 1), **i32),
             packed=torch.empty((max(km, 1), d), dtype=torch.int16, device=dev))
    ws = _ws(p, "dispatch", ws, dev)
    L.check(lib().moe_dispatch(ctypes.byref(p), _p(x), _p(topk_idx), _p(o["pos"]), _p(o["keep"]),
                               _p(o["dest"]), _p(o["expert_load"]), _p(o["expert_count"]),
                               _p(o["expert_offset"]), _p(o["rank_offset"]), _p(o["pack_src"]),
                               _p(o["packed"]), _p(ws), ws.numel(), _stream()), "moe_dispatch")
    return o


def _shape(t, name: str, shape: tuple) -> None:
    """Exact shape check (the library sees only pointers, so a matrix given
    transposed would have the right size and the wrong meaning)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def dispatch_noalloc(p: Problem, x, topk_idx, out: Optional[dict] = None) -> dict:
    """``dispatch`` through moe_dispatch_noalloc: the library's own
    device-resident table instead of a workspace (for callers that cannot
    allocate).  ``out``: optional dict of preallocated output tensors (the
    keys ``dispatch`` returns); missing ones are allocated here, by the
    caller's side, never by the library."""
    _check(p)
    B, d, E, k, D = p.B, p.d, p.E, p.k, p.n_ranks
    dev = topk_idx.device
    _need(x, "x", B * d, _xsize(p))
    _need(topk_idx, "topk_idx", B * k, 4)
    km = max_kept(p)
    i32 = dict(dtype=torch.int32, device=dev)
    make = dict(pos=lambda: torch.empty((B, k), **i32),
                keep=lambda: torch.empty((B, k), dtype=torch.uint8, device=dev),
                dest=lambda: torch.empty((B, k), **i32),
                expert_load=lambda: torch.empty(E, **i32),
                expert_count=lambda: torch.empty(E, **i32),
                expert_offset=lambda: torch.empty(E + 1, **i32),
                rank_offset=lambda: torch.empty(D + 1, **i32),
                pack_src=lambda: torch.empty(max(km, 1), **i32),
                packed=lambda: torch.empty((max(km, 1), d), dtype=torch.int16, device=dev))
    o = dict(out or {})
    for key, fn in make.items():
        if key not in o:
            o[key] = fn()
    for key, n, sz in [("pos", B * k, 4), ("keep", B * k, 1), ("dest", B * k, 4),
                       ("expert_load", E, 4), ("expert_count", E, 4),
                       ("expert_offset", E + 1, 4), ("rank_offset", D + 1, 4),
                       ("pack_src", km, 4), ("packed", km * d, 2)]:
        _need(o[key], key, n, sz)
    L.check(lib().moe_dispatch_noalloc(ctypes.byref(p), _p(x), _p(topk_idx), _p(o["pos"]),
                                       _p(o["keep"]), _p(o["dest"]), _p(o["expert_load"]),
                                       _p(o["expert_count"]), _p(o["expert_offset"]),
                                       _p(o["rank_offset"]), _p(o["pack_src"]), _p(o["packed"]),
                                       _stream()), "moe_dispatch_noalloc")
    return o


def pack_weights(p: Problem, W1, W3, W2, out=None):
    """The local experts' weights in the blocked layout the expert GEMM
    streams; done once per model.  [in, out] matrices as the layer's
    configurations print them: W1, W3 [n_local, d, f], W2 [n_local, f, d]
    (bf16), so that an expert computes act(x @ W1) @ W2."""
    _check(p)
    d, f = p.d, p.f
    nl = p.e_end - p.e_begin
    if nl > 0:
        _shape(W1, "W1", (nl, d, f))
        _shape(W2, "W2", (nl, f, d))
        if p.act == L.MOE_SWIGLU:
            _shape(W3, "W3", (nl, d, f))
    n = weights_bytes(p)
    dev = W2.device if W2 is not None else torch.device("cuda")
    if out is None:
        out = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    _need(out, "wpacked", n, 1)
    if nl > 0:
        _need(W1, "W1", nl * d * f, 2)
        _need(W2, "W2", nl * f * d, 2)
        if p.act == L.MOE_SWIGLU:
            _need(W3, "W3", nl * d * f, 2)
    L.check(lib().moe_pack_weights(ctypes.byref(p), _p(W1), _p(W3 if p.act == L.MOE_SWIGLU else None),
                                   _p(W2), _p(out), out.numel(), _stream()), "moe_pack_weights")
    return out


def expert_ffn(p: Problem, packed, expert_offset, wpacked, ret=None, ws=None):
    """ret = expert MLP of the local experts' rows; other rows copied (or
    left in place when ``ret is packed``).  ``wpacked`` from pack_weights."""
    _check(p)
    d, E = p.d, p.E
    km = max_kept(p)
    _need(packed, "packed", km * d, 2)
    _need(expert_offset, "expert_offset", E + 1, 4)
    if p.e_end > p.e_begin:
        _need(wpacked, "wpacked", weights_bytes(p), 1)
    if ret is None:
        ret = torch.empty_like(packed)
    _need(ret, "ret", km * d, 2)
    ws = _ws(p, "ffn", ws, packed.device)
    L.check(lib().moe_expert_ffn(ctypes.byref(p), _p(packed), _p(expert_offset), _p(wpacked),
                                 _p(ret), _p(ws), ws.numel(), _stream()), "moe_expert_ffn")
    return ret


def shared_ffn(ps: Problem, x, wpacked, out=None, ws=None):
    """A shared expert on every token: out [B, d] bf16 (as int16 bits)."""
    _check(ps)
    B, d = ps.B, ps.d
    _need(x, "x", B * d, 2)
    if out is None:
        out = torch.empty((B, d), dtype=torch.int16, device=x.device)
    _need(out, "out", B * d, 2)
    ws = _ws(ps, "shared_ffn", ws, x.device)
    L.check(lib().moe_shared_ffn(ctypes.byref(ps), _p(x), _p(wpacked), _p(out), _p(ws),
                                 ws.numel(), _stream()), "moe_shared_ffn")
    return out


def combine(p: Problem, ret, dest, topk_w, x_residual=None, y=None, shared_out=None):
    """``shared_out``: a shared expert's rows [B, d] bf16, added with weight 1
    (moe_combine_shared)."""
    _check(p)
    B, d, k = p.B, p.d, p.k
    _need(ret, "ret", max_kept(p) * d, 2)
    _need(dest, "dest", B * k, 4)
    _need(topk_w, "topk_w", B * k, 4)
    if p.add_residual:
        _need(x_residual, "x_residual", B * d, _xsize(p))
    if y is None:
        y = torch.empty((B, d), dtype=torch.bfloat16 if p.x_dtype == L.MOE_BF16 else torch.float32,
                        device=ret.device)
    _need(y, "y", B * d, _xsize(p))
    if shared_out is not None:
        _need(shared_out, "shared_out", B * d, 2)
        L.check(lib().moe_combine_shared(ctypes.byref(p), _p(ret), _p(dest), _p(topk_w),
                                         _p(shared_out),
                                         _p(x_residual if p.add_residual else None), _p(y),
                                         _stream()), "moe_combine_shared")
        return y
    L.check(lib().moe_combine(ctypes.byref(p), _p(ret), _p(dest), _p(topk_w),
                              _p(x_residual if p.add_residual else None), _p(y), _stream()),
            "moe_combine")
    return y


def unpack(p: Problem, ret, dest, out=None):
    _check(p)
    B, d, k = p.B, p.d, p.k
    _need(ret, "ret", max_kept(p) * d, 2)
    _need(dest, "dest", B * k, 4)
    if out is None:
        out = torch.empty((B, k, d), dtype=torch.int16, device=ret.device)
    _need(out, "out", B * k * d, 2)
    L.check(lib().moe_unpack(ctypes.byref(p), _p(ret), _p(dest), _p(out), _stream()), "moe_unpack")
    return out


_OUT_FIELDS = ("logits", "topk_idx", "topk_w", "pos", "keep", "dest", "expert_load",
               "expert_count", "expert_offset", "rank_offset", "pack_src", "packed")


# forward's stage events: the start and end of each stage's kernels
# (dispatch timestamps); the expert FFN's two GEMMs also have their own
# pairs; the gaps between launches lie between the pairs
N_STAGE_EVENTS = L.MOE_STAGE_EVENTS
STAGE_EVENTS = {"gate": (0, 1), "route": (2, 3), "dispatch": (3, 4), "expert_ffn": (5, 8),
                "combine": (9, 10)}
FFN_GEMM_EVENTS = {"gemm1": (5, 6), "gemm2": (7, 8)}
LAUNCH_GAPS = {"gate_route": (1, 2), "before_ffn": (4, 5), "between_gemms": (6, 7),
               "after_ffn": (8, 9)}
STAGES = tuple(STAGE_EVENTS)


def forward(p: Problem, x, Wg, bias, wpacked, y=None, outputs: bool = False, ws=None,
            stage_events=None, shared=None, save_z: bool = False):
    """The whole layer on the current stream (``wpacked`` from pack_weights).
    With ``outputs`` the intermediate tensors are allocated and returned too
    (``packed`` then holds the expert outputs of the local rows, in place);
    with ``save_z`` as well, ``z``: the first expert GEMM's pre-activations,
    which backward() then reads instead of recomputing them (and with a
    shared expert ``z_shared``, its own).
    ``stage_events``: optional N_STAGE_EVENTS timing-enabled
    ``torch.cuda.Event`` (or None); the library records them from the start
    and end of each stage's own kernels (STAGE_EVENTS gives the pair of each
    stage, LAUNCH_GAPS the pairs around the gaps between launches).
    ``shared`` = (ps, wpacked_shared) adds a shared expert on every token
    (moe_forward_shared; ps from shared_problem)."""
    _check(p)
    B, d, E, k = p.B, p.d, p.E, p.k
    dev = x.device
    _need(x, "x", B * d, _xsize(p))
    _need(Wg, "Wg", d * E, 4)
    if bias is not None:
        _need(bias, "bias", E, 4)
    if p.e_end > p.e_begin:
        _need(wpacked, "wpacked", weights_bytes(p), 1)
    if y is None:
        y = torch.empty((B, d), dtype=torch.bfloat16 if p.x_dtype == L.MOE_BF16 else torch.float32,
                        device=dev)
    _need(y, "y", B * d, _xsize(p))
    o = None
    outp = None
    if outputs:
        km = max(max_kept(p), 1)
        i32 = dict(dtype=torch.int32, device=dev)
        o = dict(logits=torch.empty((B, E), dtype=torch.float32, device=dev),
                 topk_idx=torch.empty((B, k), **i32),
                 topk_w=torch.empty((B, k), dtype=torch.float32, device=dev),
                 pos=torch.empty((B, k), **i32), keep=torch.empty((B, k), dtype=torch.uint8, device=dev),
                 dest=torch.empty((B, k), **i32), expert_load=torch.empty(E, **i32),
                 expert_count=torch.empty(E, **i32), expert_offset=torch.empty(E + 1, **i32),
                 rank_offset=torch.empty(p.n_ranks + 1, **i32), pack_src=torch.empty(km, **i32),
                 packed=torch.empty((km, d), dtype=torch.int16, device=dev))
        outp = L.ForwardOut(**{n: o[n].data_ptr() for n in _OUT_FIELDS})
        if save_z:
            o["z"] = torch.empty(max(saved_z_bytes(p) // 2, 1), dtype=torch.int16, device=dev)
            outp.z = o["z"].data_ptr()
            if shared is not None:
                o["z_shared"] = torch.empty(max(saved_z_bytes(shared[0]) // 2, 1),
                                            dtype=torch.int16, device=dev)
                outp.z_shared = o["z_shared"].data_ptr()
    elif save_z:
        raise ValueError("save_z needs outputs=True")
    if stage_events is not None:
        if len(stage_events) != N_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {N_STAGE_EVENTS} events")
        if outp is None:
            outp = L.ForwardOut()
        for i, ev in enumerate(stage_events):
            if ev is None:
                continue
            if ev.cuda_event == 0:  # torch creates the HIP event on first record
                ev.record()
            outp.events[i] = ev.cuda_event
    if shared is not None:
        ps, wps = shared
        _check(ps)
        n = lib().moe_forward_shared_workspace_bytes(ctypes.byref(p), ctypes.byref(ps))
        if ws is None:
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        _need(ws, "ws", n, 1)
        L.check(lib().moe_forward_shared(ctypes.byref(p), ctypes.byref(ps), _p(x), _p(Wg),
                                         _p(bias), _p(wpacked), _p(wps), _p(y),
                                         ctypes.byref(outp) if outp is not None else None,
                                         _p(ws), ws.numel(), _stream()), "moe_forward_shared")
        return (y, o) if outputs else y
    n = workspace_bytes(p, "forward")
    if ws is None:
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _need(ws, "ws", 1, 1)
    L.check(lib().moe_forward(ctypes.byref(p), _p(x), _p(Wg), _p(bias), _p(wpacked), _p(y),
                              ctypes.byref(outp) if outp is not None else None, _p(ws),
                              ws.numel(), _stream()), "moe_forward")
    return (y, o) if outputs else y


# ---------------------------------------------------------------------------
# expert-choice routing: every expert picks its top-C tokens of the batch
def expert_choice_rows(p: Problem) -> int:
    return lib().moe_expert_choice_rows(ctypes.byref(p))


def router_probs(p: Problem, logits, probs_t=None):
    """p_te = softmax(logits_t / tau), transposed: [E, B] float32."""
    _check(p)
    B, E = p.B, p.E
    _need(logits, "logits", B * E, 4)
    if probs_t is None:
        probs_t = torch.empty((E, B), dtype=torch.float32, device=logits.device)
    _need(probs_t, "probs_t", B * E, 4)
    L.check(lib().moe_router_probs(ctypes.byref(p), _p(logits), _p(probs_t), _stream()),
            "moe_router_probs")
    return probs_t


def expert_choice(p: Problem, probs_t) -> dict:
    """Every expert's top-min(C, B) tokens: sel_t [E, B], expert_offset [E+1],
    pack_src [R], pack_w [R] (R = expert_choice_rows(p))."""
    _check(p)
    B, E = p.B, p.E
    dev = probs_t.device
    _need(probs_t, "probs_t", B * E, 4)
    R = expert_choice_rows(p)
    o = dict(sel_t=torch.empty((E, B), dtype=torch.int32, device=dev),
             expert_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
             pack_src=torch.empty(max(R, 1), dtype=torch.int32, device=dev),
             pack_w=torch.empty(max(R, 1), dtype=torch.float32, device=dev))
    L.check(lib().moe_expert_choice(ctypes.byref(p), _p(probs_t), _p(o["sel_t"]),
                                    _p(o["expert_offset"]), _p(o["pack_src"]), _p(o["pack_w"]),
                                    _stream()), "moe_expert_choice")
    return o


def expert_choice_pack(p: Problem, x, pack_src, packed=None):
    _check(p)
    R = expert_choice_rows(p)
    _need(x, "x", p.B * p.d, _xsize(p))
    if packed is None:
        packed = torch.empty((max(R, 1), p.d), dtype=torch.int16, device=x.device)
    _need(packed, "packed", R * p.d, 2)
    L.check(lib().moe_expert_choice_pack(ctypes.byref(p), _p(x), _p(pack_src), _p(packed),
                                         _stream()), "moe_expert_choice_pack")
    return packed


def expert_choice_combine(p: Problem, ret, sel_t, pack_w, x_residual=None, y=None):
    _check(p)
    B, d = p.B, p.d
    _need(sel_t, "sel_t", B * p.E, 4)
    if y is None:
        y = torch.empty((B, d), dtype=torch.bfloat16 if p.x_dtype == L.MOE_BF16 else torch.float32,
                        device=sel_t.device)
    _need(y, "y", B * d, _xsize(p))
    L.check(lib().moe_expert_choice_combine(ctypes.byref(p), _p(ret), _p(sel_t), _p(pack_w),
                                            _p(x_residual if p.add_residual else None), _p(y),
                                            _stream()), "moe_expert_choice_combine")
    return y


_EC_FIELDS = ("logits", "probs_t", "sel_t", "expert_offset", "pack_src", "pack_w", "packed")


def forward_expert_choice(p: Problem, x, Wg, bias, wpacked, y=None, outputs: bool = False,
                          ws=None, stage_events=None):
    """The layer with expert-choice routing (moe_forward_expert_choice);
    ``stage_events`` as in ``forward``."""
    _check(p)
    B, d, E = p.B, p.d, p.E
    dev = x.device
    if y is None:
        y = torch.empty((B, d), dtype=torch.bfloat16 if p.x_dtype == L.MOE_BF16 else torch.float32,
                        device=dev)
    o = None
    outp = None
    if outputs:
        R = max(expert_choice_rows(p), 1)
        o = dict(logits=torch.empty((B, E), dtype=torch.float32, device=dev),
                 probs_t=torch.empty((E, B), dtype=torch.float32, device=dev),
                 sel_t=torch.empty((E, B), dtype=torch.int32, device=dev),
                 expert_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
                 pack_src=torch.empty(R, dtype=torch.int32, device=dev),
                 pack_w=torch.empty(R, dtype=torch.float32, device=dev),
                 packed=torch.empty((R, d), dtype=torch.int16, device=dev))
        outp = L.ExpertChoiceOut(**{n: o[n].data_ptr() for n in _EC_FIELDS})
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events needs 6 events")
        if outp is None:
            outp = L.ExpertChoiceOut()
        for i, ev in enumerate(stage_events):
            if ev is None:
                continue
            if ev.cuda_event == 0:
                ev.record()
            outp.events[i] = ev.cuda_event
    n = workspace_bytes(p, "forward_expert_choice")
    if ws is None:
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _need(ws, "ws", n, 1)
    L.check(lib().moe_forward_expert_choice(ctypes.byref(p), _p(x), _p(Wg), _p(bias),
                                            _p(wpacked), _p(y),
                                            ctypes.byref(outp) if outp is not None else None,
                                            _p(ws), ws.numel(), _stream()),
            "moe_forward_expert_choice")
    return (y, o) if outputs else y


# ---------------------------------------------------------------------------
# backward pass (training): gradients for an output gradient dy, with the
# routing decisions of the forward held fixed
def combine_backward(p: Problem, dy, ret, dest, topk_w, dret=None, dw=None):
    """dret [max_kept, d] bf16 (as int16 bits; rows of dropped assignments
    untouched) and dw [B, k] float32."""
    _check(p)
    B, d, k = p.B, p.d, p.k
    km = max_kept(p)
    _need(dy, "dy", B * d, _xsize(p))
    _need(ret, "ret", km * d, 2)
    _need(dest, "dest", B * k, 4)
    _need(topk_w, "topk_w", B * k, 4)
    if dret is None:
        dret = torch.zeros((max(km, 1), d), dtype=torch.int16, device=dy.device)
    if dw is None:
        dw = torch.empty((B, k), dtype=torch.float32, device=dy.device)
    _need(dret, "dret", km * d, 2)
    _need(dw, "dw", B * k, 4)
    L.check(lib().moe_combine_backward(ctypes.byref(p), _p(dy), _p(ret), _p(dest), _p(topk_w),
                                       _p(dret), _p(dw), _stream()), "moe_combine_backward")
    return dret, dw


def route_backward(p: Problem, logits, topk_idx, dw, expert_load=None, aux_coef: float = 0.0,
                   dlogits=None):
    """dlogits [B, E] float32 (aux_coef scales the auxiliary load-balancing
    loss sum_e f_e P_e; it needs expert_load)."""
    _check(p)
    B, E, k = p.B, p.E, p.k
    _need(logits, "logits", B * E, 4)
    _need(topk_idx, "topk_idx", B * k, 4)
    _need(dw, "dw", B * k, 4)
    if aux_coef != 0.0:
        _need(expert_load, "expert_load", E, 4)
    if dlogits is None:
        dlogits = torch.empty((B, E), dtype=torch.float32, device=logits.device)
    _need(dlogits, "dlogits", B * E, 4)
    L.check(lib().moe_route_backward(ctypes.byref(p), _p(logits), _p(topk_idx), _p(dw),
                                     _p(expert_load), ctypes.c_float(aux_coef), _p(dlogits),
                                     _stream()), "moe_route_backward")
    return dlogits


def weights_bwd_bytes(p: Problem) -> int:
    return lib().moe_weights_bwd_bytes(ctypes.byref(p))


def saved_z_bytes(p: Problem) -> int:
    """Bytes of the forward's saved pre-activations (moe_saved_z_bytes)."""
    return lib().moe_saved_z_bytes(ctypes.byref(p))


def pack_weights_bwd(p: Problem, W1, W3, W2, out=None):
    """The local experts' weights rearranged for the expert backward (same
    [in, out] inputs as pack_weights)."""
    _check(p)
    d, f = p.d, p.f
    nl = p.e_end - p.e_begin
    if nl > 0:
        _shape(W1, "W1", (nl, d, f))
        _shape(W2, "W2", (nl, f, d))
        if p.act == L.MOE_SWIGLU:
            _shape(W3, "W3", (nl, d, f))
    n = weights_bwd_bytes(p)
    dev = W2.device if W2 is not None else torch.device("cuda")
    if out is None:
        out = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    _need(out, "wpacked_bwd", n, 1)
    if nl > 0:
        _need(W1, "W1", nl * d * f, 2)
        _need(W2, "W2", nl * f * d, 2)
        if p.act == L.MOE_SWIGLU:
            _need(W3, "W3", nl * d * f, 2)
    L.check(lib().moe_pack_weights_bwd(ctypes.byref(p), _p(W1),
                                       _p(W3 if p.act == L.MOE_SWIGLU else None), _p(W2),
                                       _p(out), out.numel(), _stream()), "moe_pack_weights_bwd")
    return out


def expert_ffn_backward(p: Problem, x, pack_src, expert_offset, wpacked, wpacked_bwd, dret,
                        ws=None, z=None):
    """dret [max_kept, d] bf16 is overwritten in place: its local rows
    become the gradient of the packed input rows.  ``z``: the forward's
    saved pre-activations (``forward(..., save_z=True)``) or None to
    recompute them.  Returns dict dxp (= dret), dW1, dW3 (SwiGLU, else None)
    [n_local, d, f] and dW2 [n_local, f, d] float32."""
    _check(p)
    B, d, f = p.B, p.d, p.f
    nl = p.e_end - p.e_begin
    km = max_kept(p)
    dev = dret.device
    _need(x, "x", B * d, _xsize(p))
    _need(pack_src, "pack_src", km, 4)
    _need(expert_offset, "expert_offset", p.E + 1, 4)
    _need(dret, "dret", km * d, 2)
    sw = p.act == L.MOE_SWIGLU
    f32 = dict(dtype=torch.float32, device=dev)
    dW1 = torch.empty((max(nl, 1), d, f), **f32)
    dW2 = torch.empty((max(nl, 1), f, d), **f32)
    dW3 = torch.empty((max(nl, 1), d, f), **f32) if sw else None
    if nl > 0:
        _need(wpacked, "wpacked", weights_bytes(p), 1)
        _need(wpacked_bwd, "wpacked_bwd", weights_bwd_bytes(p), 1)
    if z is not None:
        _need(z, "z", saved_z_bytes(p) // 2, 2)
    ws = _ws(p, "expert_ffn_backward", ws, dev)
    L.check(lib().moe_expert_ffn_backward(ctypes.byref(p), _p(x), _p(pack_src),
                                          _p(expert_offset), _p(wpacked), _p(wpacked_bwd),
                                          _p(z), _p(dret), _p(dW1), _p(dW3), _p(dW2), _p(ws),
                                          ws.numel(), _stream()), "moe_expert_ffn_backward")
    return dict(dxp=dret, dW1=dW1[:nl], dW3=None if dW3 is None else dW3[:nl], dW2=dW2[:nl])


def dispatch_backward(p: Problem, dxp, dest, dy=None, dx_acc=None):
    """dx_acc [B, d] float32 = sum_j dxp[dest[t, j]] (+ dy with the residual)."""
    _check(p)
    B, d, k = p.B, p.d, p.k
    _need(dxp, "dxp", max_kept(p) * d, 2)
    _need(dest, "dest", B * k, 4)
    if p.add_residual:
        _need(dy, "dy", B * d, _xsize(p))
    if dx_acc is None:
        dx_acc = torch.empty((B, d), dtype=torch.float32, device=dxp.device)
    _need(dx_acc, "dx_acc", B * d, 4)
    L.check(lib().moe_dispatch_backward(ctypes.byref(p), _p(dxp), _p(dest),
                                        _p(dy if p.add_residual else None), _p(dx_acc),
                                        _stream()), "moe_dispatch_backward")
    return dx_acc


def gate_backward(p: Problem, x, Wg, dlogits, dx_acc=None, ws=None):
    """dx [B, d] (x dtype) = dlogits Wg^T (+ dx_acc), dWg [d, E] and dbias
    [E] float32."""
    _check(p)
    B, d, E = p.B, p.d, p.E
    dev = dlogits.device
    _need(x, "x", B * d, _xsize(p))
    _need(Wg, "Wg", d * E, 4)
    _need(dlogits, "dlogits", B * E, 4)
    if dx_acc is not None:
        _need(dx_acc, "dx_acc", B * d, 4)
    dx = torch.empty((B, d), dtype=torch.bfloat16 if p.x_dtype == L.MOE_BF16 else torch.float32,
                     device=dev)
    dWg = torch.empty((d, E), dtype=torch.float32, device=dev)
    dbias = torch.empty(E, dtype=torch.float32, device=dev)
    ws = _ws(p, "gate_backward", ws, dev)
    L.check(lib().moe_gate_backward(ctypes.byref(p), _p(x), _p(Wg), _p(dlogits), _p(dx_acc),
                                    _p(dx), _p(dWg), _p(dbias), _p(ws), ws.numel(), _stream()),
            "moe_gate_backward")
    return dx, dWg, dbias


def backward(p: Problem, x, Wg, wpacked, wpacked_bwd, saved: dict, dy, aux_coef: float = 0.0,
             ws=None, shared=None) -> dict:
    """All gradients of the layer (moe_backward).  ``saved``: the dict of
    ``forward(..., outputs=True)`` (logits, topk_idx, topk_w, dest,
    expert_load, expert_offset, pack_src, and packed = the expert outputs;
    with ``save_z=True`` also z, the pre-activations the backward then does
    not recompute).  ``shared`` = (ps, wpacked_shared, wpacked_shared_bwd)
    for the layer of ``forward(..., shared=...)`` (moe_backward_shared): the
    result then also holds dW1s, dW3s (SwiGLU, else None) and dW2s.
    Returns dx, dWg, dbias, dW1, dW3 (SwiGLU, else None), dW2, dlogits, dw."""
    _check(p)
    B, d, E, k, f = p.B, p.d, p.E, p.k, p.f
    nl = p.e_end - p.e_begin
    dev = dy.device
    _need(x, "x", B * d, _xsize(p))
    _need(Wg, "Wg", d * E, 4)
    _need(dy, "dy", B * d, _xsize(p))
    sw = p.act == L.MOE_SWIGLU
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty((B, d), dtype=torch.bfloat16 if p.x_dtype == L.MOE_BF16
                            else torch.float32, device=dev),
             dWg=torch.empty((d, E), **f32), dbias=torch.empty(E, **f32),
             dW1=torch.empty((max(nl, 1), d, f), **f32), dW2=torch.empty((max(nl, 1), f, d), **f32),
             dW3=torch.empty((max(nl, 1), d, f), **f32) if sw else None,
             dlogits=torch.empty((B, E), **f32), dw=torch.empty((B, k), **f32))
    sv = L.Saved(logits=saved["logits"].data_ptr(), topk_idx=saved["topk_idx"].data_ptr(),
                 topk_w=saved["topk_w"].data_ptr(), dest=saved["dest"].data_ptr(),
                 expert_load=saved["expert_load"].data_ptr(),
                 expert_offset=saved["expert_offset"].data_ptr(),
                 pack_src=saved["pack_src"].data_ptr(), ret=saved["packed"].data_ptr(),
                 z=saved["z"].data_ptr() if saved.get("z") is not None else None,
                 z_shared=saved["z_shared"].data_ptr()
                 if shared is not None and saved.get("z_shared") is not None else None)
    gr = L.Grads(**{n: (g[n].data_ptr() if g[n] is not None else None)
                    for n in ("dx", "dWg", "dbias", "dW1", "dW3", "dW2", "dlogits", "dw")})
    if shared is not None:
        ps, wps, wpsb = shared
        _check(ps)
        fs = ps.f
        ssw = ps.act == L.MOE_SWIGLU
        g["dW1s"] = torch.empty((d, fs), **f32)
        g["dW2s"] = torch.empty((fs, d), **f32)
        g["dW3s"] = torch.empty((d, fs), **f32) if ssw else None
        n = lib().moe_backward_shared_workspace_bytes(ctypes.byref(p), ctypes.byref(ps))
        if ws is None:
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        _need(ws, "ws", n, 1)
        L.check(lib().moe_backward_shared(ctypes.byref(p), ctypes.byref(ps), _p(x), _p(Wg),
                                          _p(wpacked), _p(wpacked_bwd), _p(wps), _p(wpsb),
                                          ctypes.byref(sv), _p(dy), ctypes.c_float(aux_coef),
                                          ctypes.byref(gr), _p(g["dW1s"]), _p(g["dW3s"]),
                                          _p(g["dW2s"]), _p(ws), ws.numel(), _stream()),
                "moe_backward_shared")
    else:
        n = workspace_bytes(p, "backward")
        if ws is None:
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        _need(ws, "ws", n, 1)
        L.check(lib().moe_backward(ctypes.byref(p), _p(x), _p(Wg), _p(wpacked),
                                   _p(wpacked_bwd), ctypes.byref(sv), _p(dy),
                                   ctypes.c_float(aux_coef), ctypes.byref(gr), _p(ws),
                                   ws.numel(), _stream()), "moe_backward")
    for key in ("dW1", "dW2", "dW3"):
        if g[key] is not None:
            g[key] = g[key][:nl]
    return g
