"""CPU oracle for the forward pass of one mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this file: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP
library; both are fed from the seeded generators in ``moe_synth``.

It is a plain, slow, obviously correct restatement of what the pages define,
computed in float64 (NumPy) unless the definition itself fixes a precision:

* router logits are float32 values (the router is an fp32 layer): the dot
  product is formed in float64 and rounded once to float32;
* expert choice is a decision on those float32 logits;
* everything else (softmax, expert FFN, combine) stays in float64.

It also holds the layer's backward pass (gradients for a given output
gradient, with the routing decisions held fixed and an optional auxiliary
load-balancing term), in float64, as the steps of the forward in reverse.

Pages followed (cited by page title and section):

[EP-glossary]  "Expert Parallelism", inferensys.com glossary: the gating
               network gives each token a probability distribution over the
               experts and the top-k are selected; capacity limits per expert,
               overflow is skipped.
[EP-notes]     "Expert Parallelism", narrativegoldmine.com:
               section "Components and Architecture" (gating network,
               dispatch tensor, expert GEMM, combine weighted by the gating
               probabilities, capacity factor and token dropping) and section
               "Formal Algorithm: Expert Parallelism Forward Pass" (g_t,
               p_t = softmax(g_t / tau), e(t) = argmax p_t, w_t = p_{t,e(t)},
               dispatch, expert computation, combine, residual).
[EP-infinity]  "Expert Parallelism", theinfinity.ai: the capacity paragraph
               (C = ceil((B*k/D)*c), overflow = max(0, p*B*k - C)) and the
               worked-example figure (6 tokens, 8 experts, 4 devices, top-2,
               capacity 2, two dropped assignments, experts 1 and 8 idle).
[EP-a2a]       "Expert Parallelism and the All-to-All Bottleneck",
               ashishsrivastav.com: section "The Mechanism of Expert
               Parallelism" (routing, dispatch repacks rows per destination
               expert, expert forward, gather back into the original token
               order) and section "The All-to-All Communication Pattern"
               (contiguous expert placement: 64 experts on 8 GPUs, expert 55
               on GPU 6, expert 5 on GPU 0).

Readings where the pages are silent or disagree (each also listed in the
design notes of the repository):

* capacity is per expert, ceil((B*k/E)*c) -- the page's per-device formula
  with E in place of D; it is the only reading that gives the worked example's
  "capacity of 2" (6*2/8*1.25 = 1.875 -> 2);
* tau = 1 unless given; selection uses the key (logit descending, expert index
  ascending), which orders experts exactly as the exact probabilities do and
  breaks ties toward the lower index;
* gate weights are the raw softmax probabilities of the chosen experts (not
  renormalised), as w_t = p_{t,e(t)} in the formal algorithm;
* assignments claim capacity slot-major: all tokens' first choices in token
  order, then all second choices, ...; a dropped assignment contributes zero;
* the packed buffer is compact and expert-major (hence destination-rank
  major), rows of one expert in claim order;
* an expert is act(x W1) W2 on a row x with exact-erf GELU, or
  (silu(x W1) * (x W3)) W2 for SwiGLU, with no biases; the weights are
  [in, out] matrices as the workloads print them (W1, W3 [d, f], W2 [f, d]);
* rows owned by experts that do not run on this GPU come back unchanged (the
  missing collective is the identity).

Pins (what fixes this code other than itself) live in ``tests/test_oracle_*``;
every function below names the pins that cover it.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "capacity", "bf16_bits_to_f64", "f32_to_bf16_bits_rne", "gate_logits",
    "softmax", "route", "assign_slots", "layout", "pack", "gelu", "silu",
    "expert_mlp", "expert_ffn", "combine", "unpack", "forward", "rank_of_expert",
    "expert_capacities", "routing_stats", "shared_ffn", "router_probs", "expert_choice",
    "expert_choice_combine", "forward_expert_choice", "assign_slots_redirect",
    "combine_by_segment", "combine_backward", "route_backward", "expert_mlp_backward",
    "expert_ffn_backward", "dispatch_backward", "gate_backward", "backward",
]


# ----------------------------------------------------------------------------
# capacity
# ----------------------------------------------------------------------------
def capacity(B: int, k: int, E: int, c: float) -> int:
    """Per-expert capacity C = ceil((B*k/E)*c).

    [EP-infinity] capacity paragraph gives ceil((B*k/D)*c) per device; per
    expert (E for D) is the reading that reproduces the worked example's
    capacity of 2.  Evaluated in IEEE double in exactly this operation order.
    Pins: worked-example capacity 2; the five workload capacities; the
    overflow identity max(0, n_e - C) on every expert (test_oracle_capacity,
    test_oracle_worked_example)."""
    if B == 0:
        return 0
    return int(math.ceil((float(B * k) / float(E)) * float(c)))


def rank_of_expert(e: int, E: int, D: int) -> int:
    """Contiguous placement: E/D experts per rank, rank r owns
    [r*E/D, (r+1)*E/D).  [EP-a2a] "The All-to-All Communication Pattern":
    with 64 experts on 8 GPUs expert 55 lives on GPU 6 and expert 5 on GPU 0
    (pinned in test_oracle_special)."""
    return e // (E // D)


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the high half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs).

    Written from the definition: keep the top 16 bits, look at the dropped
    low 16 bits; round up when they exceed half an ulp, or equal half an ulp
    and the kept part is odd.  Pins: hand-made tie/non-tie cases in
    test_oracle_special."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


def _x_values(x: np.ndarray) -> np.ndarray:
    """The defined input values: bf16 bits (uint16) or float32."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# step 1: gate
# ----------------------------------------------------------------------------
def gate_logits(x: np.ndarray, Wg: np.ndarray,
                bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits g_t = x_t . Wg (+ b), float32 [B, E].

    [EP-notes] "Formal Algorithm": g_t in R^E from the routing linear
    projection; "Components and Architecture": a learned linear map, with an
    optional bias term on the routing logits.  The sum is formed in float64
    (each bf16 x fp32 product is exact there) and rounded once to float32.
    Pins: exact rational dot products (fractions.Fraction) on small inputs in
    test_oracle_gate."""
    xv = _x_values(x)
    l = xv @ np.asarray(Wg, dtype=np.float32).astype(np.float64)
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return l.astype(np.float32)


# ----------------------------------------------------------------------------
# step 2: softmax + top-k
# ----------------------------------------------------------------------------
def softmax(logits: np.ndarray, tau: float = 1.0) -> np.ndarray:
    """p_t = softmax(g_t / tau) over the E experts, float64.

    [EP-notes] "Formal Algorithm", gate computation.  Pins: sums to one,
    equal logits give 1/E, shift invariance, closed-form worked-example
    weights (test_oracle_route)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64) / float(tau)
    if z.shape[0] == 0:
        return z
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def route(logits: np.ndarray, k: int, tau: float = 1.0):
    """Top-k experts per token and their raw gate probabilities.

    Selection is decided on the float32 logits with the key
    (logit descending, expert index ascending); j = 0 is the strongest
    choice.  Because softmax is strictly increasing in the logit this is
    the exact-probability order, and logit ties are exactly probability
    ties, broken toward the lower index.  The weight of choice j is the
    softmax probability of that expert, not renormalised
    ([EP-notes] "Formal Algorithm": e(t) = argmax p_t, w_t = p_{t,e(t)};
    [EP-glossary]: top-k of the distribution).

    Returns idx int32 [B, k], w float64 [B, k] (the float32 the GPU
    reports is compared against it within tolerance).  Pins: k = 1 is
    argmax; k = E selects everything; brute-force sort with engineered ties;
    equal logits give 0..k-1 and 1/E (test_oracle_route)."""
    l32 = np.asarray(logits, dtype=np.float32)
    B, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort of -logit: descending value, equal values keep index order
    order = np.argsort(-l32, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    p = softmax(l32, tau)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return idx, w


# ----------------------------------------------------------------------------
# step 3: capacity-limited slot assignment
# ----------------------------------------------------------------------------
def expert_capacities(E: int, C: int, unavailable=None) -> np.ndarray:
    """Capacity of each expert: C, or 0 for an expert marked unavailable.

    [EP-glossary] lists an expert that becomes unavailable among the
    failure modes of routing; [EP-notes] "Components and Architecture":
    tokens routed to a full expert are dropped.  Reading: an unavailable
    expert is one whose capacity is zero, so every assignment to it is
    dropped exactly like overflow.  Pins: masked experts keep nothing,
    an all-false mask changes nothing, claim-queue brute force with
    per-expert capacities (test_oracle_health)."""
    cap = np.full(E, int(C), dtype=np.int64)
    if unavailable is not None:
        m = np.asarray(unavailable).astype(bool).reshape(-1)
        if m.shape[0] != E:
            raise ValueError("unavailable needs E entries")
        cap[m] = 0
    return cap


def assign_slots(idx: np.ndarray, E: int, C: int, unavailable=None):
    """Slot of every assignment inside its expert, and which ones are kept.

    Assignment (t, j) has claim priority q = j*B + t (slot-major: every
    token's first choice in token order, then every second choice, ...).
    pos[t, j] = number of assignments to the same expert with smaller q;
    keep = pos < C_e.  n_e = assignments routed to e; kept_e = min(n_e, C_e);
    dropped_e = max(0, n_e - C_e), the page's overflow with p*B*k = n_e
    ([EP-infinity] capacity paragraph; [EP-notes] "Components and
    Architecture", capacity factor and token dropping).  C_e = C, or 0 for
    experts marked unavailable (``expert_capacities``).

    Uses one library primitive, a stable sort by expert of the assignments
    listed in q order; the rank inside each run of equal experts is pos.
    Pins: a sequential pure-Python claim queue (brute force), the worked
    example fixture, the overflow identity (test_oracle_slots)."""
    idx = np.asarray(idx, dtype=np.int64)
    B, k = idx.shape
    cap = expert_capacities(E, C, unavailable)
    e_q = idx.T.reshape(-1)                     # position q = j*B + t
    order = np.argsort(e_q, kind="stable")      # by expert, q ascending
    sorted_e = e_q[order]
    load = np.bincount(e_q, minlength=E).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(load)[:-1]])
    pos_q = np.empty(B * k, dtype=np.int64)
    pos_q[order] = np.arange(B * k) - start[sorted_e]
    pos = pos_q.reshape(k, B).T.copy()
    keep = pos < cap[idx]
    count = np.minimum(load, cap)
    return pos.astype(np.int32), keep, load.astype(np.int32), count.astype(np.int32)


def assign_slots_redirect(ranked: np.ndarray, k: int, E: int, C: int, unavailable=None):
    """Slot assignment where overflow is redirected to the next-best expert.

    [EP-notes] "Components and Architecture", token dispatch and capacity
    factor: tokens routed to a full expert are dropped or redirected to a
    secondary expert (a fallback routing).  Reading (one fallback round):
    round 1 is ``assign_slots`` on the top-k choices; then the m-th dropped
    choice of a token (m counted in j order) is redirected to the token's
    (k + m)-th ranked expert -- outside its top-k, distinct for each of its
    redirected choices, none if k + m >= the ranks given -- and the
    redirected assignments claim the capacity left, C_e - kept_e, in the
    original claim order q = j*B + t; what does not fit is dropped.

    ``ranked`` [B, K2] are each token's experts by rank (K2 >= k).  Returns
    expert [B, k] (the expert an assignment ends with: its own, its
    fallback, or its own when dropped), rank [B, k] (its column in
    ``ranked``), slot [B, k], keep [B, k], load (n_e of the top-k choices)
    and count (kept per expert, both rounds).  Pins: a sequential claim
    queue, capacity and distinctness invariants, the drop policy when
    nothing overflows (test_oracle_redirect)."""
    ranked = np.asarray(ranked, dtype=np.int64)
    B = ranked.shape[0]
    K2 = ranked.shape[1]
    idx = ranked[:, :k]
    pos1, keep1, load, count1 = assign_slots(idx, E, C, unavailable)
    cap = expert_capacities(E, C, unavailable)
    rank = np.tile(np.arange(k), (B, 1))
    fb = np.full((B, k), -1, dtype=np.int64)
    for t in range(B):
        m = 0
        for j in range(k):
            if not keep1[t, j]:
                if k + m < K2:
                    fb[t, j] = ranked[t, k + m]
                    rank[t, j] = k + m
                m += 1
    rem = cap - count1
    # round 2: redirected assignments in q order claim the remaining slots
    e_q = fb.T.reshape(-1)
    valid = e_q >= 0
    pos2_q = np.full(B * k, -1, dtype=np.int64)
    vq = np.nonzero(valid)[0]
    order = vq[np.argsort(e_q[vq], kind="stable")]
    sorted_e = e_q[order]
    start = np.searchsorted(sorted_e, np.arange(E))
    pos2_q[order] = np.arange(order.size) - start[sorted_e]
    pos2 = pos2_q.reshape(k, B).T
    keep2 = (fb >= 0) & (pos2 < np.where(fb >= 0, rem[np.maximum(fb, 0)], 0))
    expert = np.where(keep1, idx, np.where(keep2, fb, idx))
    rank = np.where(keep1 | ~keep2, np.tile(np.arange(k), (B, 1)), rank)
    slot = np.where(keep1, pos1, np.where(keep2, count1[np.maximum(fb, 0)] + pos2, -1))
    keep = keep1 | keep2
    count = count1 + np.bincount(fb[keep2], minlength=E).astype(count1.dtype)
    return (expert.astype(np.int32), rank.astype(np.int32), slot.astype(np.int32), keep,
            load, count.astype(np.int32))


def layout(idx: np.ndarray, pos: np.ndarray, keep: np.ndarray, E: int, D: int,
           C: int, unavailable=None, count: Optional[np.ndarray] = None):
    """Compact, expert-major packed layout (hence grouped by destination rank).

    expert_offset = exclusive prefix sum of kept_e (E+1 entries);
    rank_offset[r] = expert_offset[r*E/D] (D+1 entries) -- rank r owns the
    contiguous experts [r*E/D, (r+1)*E/D) ([EP-a2a] "The All-to-All
    Communication Pattern"; "The Mechanism of Expert Parallelism": rows are
    repacked per destination expert); dest[t, j] = expert_offset[e] + pos for
    kept assignments, -1 otherwise; pack_src[dest] = t.
    Pins: worked-example fixture; bijection/segment invariants
    (test_oracle_slots)."""
    idx = np.asarray(idx, dtype=np.int64)
    if count is None:
        load = np.bincount(idx.reshape(-1), minlength=E)
        kept = np.minimum(load, expert_capacities(E, C, unavailable))
    else:
        kept = np.asarray(count, dtype=np.int64)
    expert_offset = np.zeros(E + 1, dtype=np.int64)
    expert_offset[1:] = np.cumsum(kept)
    rank_offset = expert_offset[np.arange(D + 1) * (E // D)]
    dest = np.where(keep, expert_offset[idx] + pos, -1)
    K = int(expert_offset[-1])
    pack_src = np.empty(K, dtype=np.int64)
    t_of = np.broadcast_to(np.arange(idx.shape[0])[:, None], idx.shape)
    pack_src[dest[keep]] = t_of[keep]
    return (expert_offset.astype(np.int32), rank_offset.astype(np.int32),
            dest.astype(np.int32), pack_src.astype(np.int32))


# ----------------------------------------------------------------------------
# step 4: pack (on-device stand-in for the dispatch all-to-all)
# ----------------------------------------------------------------------------
def pack(x: np.ndarray, pack_src: np.ndarray) -> np.ndarray:
    """packed[r] = bf16(x[pack_src[r]]) as bf16 bits [K, d].

    [EP-a2a] "The Mechanism of Expert Parallelism", dispatch phase: the
    (tokens, hidden) activations are repacked so that each row is a token
    bound for one expert.  bf16 inputs are copied bit for bit; float32
    inputs are rounded to nearest even.  Pins: round trip with ``unpack``
    and the bf16 rounding cases (test_oracle_special)."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x[np.asarray(pack_src, dtype=np.int64)])
    return f32_to_bf16_bits_rne(np.asarray(x, np.float32)[np.asarray(pack_src, dtype=np.int64)])


def unpack(rows: np.ndarray, dest: np.ndarray) -> np.ndarray:
    """out[t, j] = rows[dest[t, j]] for kept assignments, 0 elsewhere
    ([EP-a2a] "The Mechanism of Expert Parallelism": results return to the
    original token order)."""
    B, k = dest.shape
    out = np.zeros((B, k, rows.shape[1]), dtype=rows.dtype)
    m = dest >= 0
    out[m] = rows[dest[m]]
    return out


# ----------------------------------------------------------------------------
# step 5: expert FFN
# ----------------------------------------------------------------------------
def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2)), float64.
    Pins: Phi(1), Phi(-1) and an independent library GELU
    (test_oracle_ffn)."""
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z), float64 (pinned like ``gelu``)."""
    return z / (1.0 + np.exp(-z))


def _w(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def expert_mlp(xr: np.ndarray, W1: np.ndarray, W2: np.ndarray,
               W3: Optional[np.ndarray], act: str) -> np.ndarray:
    """One expert on rows xr [n, d] (float64): act(xr W1) W2.

    [EP-notes] "Components and Architecture", Expert GEMM: the expert is a
    standard transformer MLP.  W1, W3: [d, f]; W2: [f, d] ([in, out], the
    layout the workloads print), bf16 bits or float32.  GELU is exact-erf;
    SwiGLU is silu(x W1) * (x W3); no biases.  Pins: an independent float64
    library MLP, E = 1 plain-MLP reduction (test_oracle_ffn)."""
    w1 = _w(W1)
    w2 = _w(W2)
    h = xr @ w1
    if act == "gelu":
        h = gelu(h)
    elif act == "swiglu":
        h = silu(h) * (xr @ _w(W3))
    else:
        raise ValueError(act)
    return h @ w2


def expert_ffn(x: np.ndarray, pack_src: np.ndarray, expert_offset: np.ndarray,
               e_begin: int, e_end: int, W1, W2, W3, act: str,
               rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Return buffer ret in float64: [K, d], or [len(rows), d] for the packed
    rows listed in ``rows`` (spot checks at full size).

    Rows of experts in [e_begin, e_end) get that expert's MLP of the token's
    defined input x (bf16 values, or the float32 originals for an f32
    workload); every other row comes back as its packed bf16 value (the
    missing collective is the identity).  [EP-notes] "Formal Algorithm",
    expert computation on received tokens; [EP-a2a] "The Mechanism of
    Expert Parallelism", phase 3."""
    pack_src = np.asarray(pack_src, dtype=np.int64)
    K = pack_src.shape[0]
    r_all = np.arange(K) if rows is None else np.asarray(rows, dtype=np.int64)
    ret = np.empty((r_all.size, x.shape[1]))
    lo, hi = int(expert_offset[e_begin]), int(expert_offset[e_end])
    # rows owned by other ranks: identity loopback of the packed bf16 value
    remote = (r_all < lo) | (r_all >= hi)
    if remote.any():
        ret[remote] = bf16_bits_to_f64(pack(x, pack_src[r_all[remote]]))
    for e in range(e_begin, e_end):
        a, b = int(expert_offset[e]), int(expert_offset[e + 1])
        sel = np.nonzero((r_all >= a) & (r_all < b))[0]
        if sel.size == 0:
            continue
        i = e - e_begin
        ret[sel] = expert_mlp(_x_values(x[pack_src[r_all[sel]]]), W1[i], W2[i],
                              None if W3 is None else W3[i], act)
    return ret


# ----------------------------------------------------------------------------
# step 6: combine
# ----------------------------------------------------------------------------
def shared_ffn(x: np.ndarray, W1, W2, W3, act: str,
               tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Output of a shared expert, float64 [B, d] (or [len(tokens), d]).

    [EP-notes] "Major Variants and Families", shared expert routing: one
    expert processes every token in addition to the routed experts (a dense
    path beside them).  It is an expert like the others (``expert_mlp``,
    W1/W3 [d, f], W2 [f, d]) applied to every token's input, with weight 1.
    Pin: a shared expert equals a routed expert that every token chooses
    with probability 1 (E = 1, k = 1, no drops), computed through route,
    slots, layout, expert_ffn and combine (test_oracle_shared)."""
    rows = x if tokens is None else x[np.asarray(tokens, dtype=np.int64)]
    return expert_mlp(_x_values(rows), W1, W2, W3, act)


def combine(ret: np.ndarray, dest: np.ndarray, w: np.ndarray,
            x_residual: Optional[np.ndarray] = None,
            tokens: Optional[np.ndarray] = None,
            ret_rows: Optional[np.ndarray] = None,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum_j [kept] w[t, j] * ret[dest[t, j]] (+ x[t]), float64.

    [EP-notes] "Components and Architecture", expert combine: the k outputs
    of a token are weighted by the gating probabilities and summed, in the
    original token order ([EP-a2a] gather phase); a dropped assignment
    contributes nothing, so a token with every choice dropped gets 0 (plus
    the residual when it is added).  ``w`` is taken at float32 precision,
    the precision the router reports it in.

    ``tokens`` restricts the output to those tokens ([len(tokens), d]);
    ``ret_rows`` says which packed rows ``ret`` holds (sorted), when it holds
    only some.  ``shared`` (rows for the same tokens) is a shared expert's
    output, added with weight 1 ([EP-notes] "Major Variants and Families",
    shared expert routing).  Pins: dense soft-mixture equivalence without
    drops, C = 0 gives 0 (test_oracle_combine_special); the shared expert
    as a routed expert every token chooses (test_oracle_shared)."""
    B, k = dest.shape
    tt = np.arange(B) if tokens is None else np.asarray(tokens, dtype=np.int64)
    acc = np.zeros((tt.size, ret.shape[1]))
    w32 = np.asarray(w, dtype=np.float32).astype(np.float64)
    for j in range(k):
        dj = dest[tt, j].astype(np.int64)
        m = dj >= 0
        r = dj[m] if ret_rows is None else np.searchsorted(ret_rows, dj[m])
        acc[m] += w32[tt[m], j][:, None] * ret[r]
    if shared is not None:
        acc += np.asarray(shared, dtype=np.float64)
    if x_residual is not None:
        acc += _x_values(x_residual[tt])
    return acc


def combine_by_segment(x: np.ndarray, pack_src: np.ndarray, expert_offset: np.ndarray,
                       e_begin: int, e_end: int, W1, W2, W3, act: str,
                       dest: np.ndarray, w: np.ndarray,
                       x_residual: Optional[np.ndarray] = None,
                       shared: Optional[np.ndarray] = None) -> np.ndarray:
    """The same y as ``combine(expert_ffn(...), dest, w, ...)`` without
    holding the whole return buffer: the packed rows are taken one expert
    segment at a time (its MLP for a local expert, the packed values for a
    remote one, as ``expert_ffn``), and each row's weighted value is added
    to its token's sum at once.  The terms of a token are therefore added in
    expert order rather than in j order; in float64 the two sums differ by a
    few float64 ulps.  For large batches (the return buffer of 262144 rows of
    7168 would take 15 GB in float64).  Pin: equal to the j-order combine
    within 1e-13 on small layers, with and without remote rows, drops and
    the residual (test_oracle_combine_special)."""
    B, k = dest.shape
    d = x.shape[1]
    pack_src = np.asarray(pack_src, dtype=np.int64)
    w32 = np.asarray(w, dtype=np.float32).astype(np.float64)
    # which choice j of its token each packed row is
    j_of = np.empty(pack_src.shape[0], dtype=np.int64)
    for j in range(k):
        m = dest[:, j] >= 0
        j_of[dest[m, j].astype(np.int64)] = j
    acc = np.zeros((B, d))
    E = expert_offset.shape[0] - 1
    for e in range(E):
        a, b = int(expert_offset[e]), int(expert_offset[e + 1])
        if b <= a:
            continue
        rows = np.arange(a, b)
        seg = expert_ffn(x, pack_src, expert_offset, e_begin, e_end, W1, W2, W3, act,
                         rows=rows) if e_begin <= e < e_end else \
            bf16_bits_to_f64(pack(x, pack_src[rows]))
        t = pack_src[rows]
        # a token appears at most once in one expert's segment
        acc[t] += w32[t, j_of[rows]][:, None] * seg
    if shared is not None:
        acc += np.asarray(shared, dtype=np.float64)
    if x_residual is not None:
        acc += _x_values(x_residual)
    return acc


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------
def forward(x, Wg, bias, W1, W3, W2, *, k: int, c: float, act: str,
            n_ranks: int = 1, e_begin: int = 0, e_end: Optional[int] = None,
            tau: float = 1.0, C: Optional[int] = None, add_residual: bool = False,
            logits: Optional[np.ndarray] = None, unavailable=None,
            shared: Optional[tuple] = None, overflow: str = "drop",
            keep_ret: Optional[bool] = None) -> dict:
    """All steps in the pages' order ([EP-notes] "Formal Algorithm";
    [EP-a2a] "The Mechanism of Expert Parallelism"): gate, top-k, capacity
    and slots, pack, expert FFN, unpack + weighted combine (+ residual).

    ``logits`` may be given to skip the gate (routing tests feed the router
    directly); without expert weights only the integer steps and the pack
    run.  ``shared`` = (W1s, W3s, W2s) adds a shared expert's output to every
    token's combine.  ``overflow`` = "next" redirects overflow to the
    token's next-best experts (``assign_slots_redirect``, the router giving
    min(2k, E) ranked choices); idx / w then hold the expert and weight each
    assignment ends with.  ``keep_ret``: hold the whole return buffer and
    return it as ``ret`` (default: when it has at most 2^26 values); without
    it y comes from ``combine_by_segment``."""
    B = x.shape[0]
    E = Wg.shape[1] if Wg is not None else logits.shape[1]
    e_end = E if e_end is None else e_end
    if logits is None:
        logits = gate_logits(x, Wg, bias)
    if C is None:
        C = capacity(B, k, E, c)
    if overflow == "next":
        ranked, pr = route(logits, min(2 * k, E), tau)
        idx, rk, pos, keep, load, count = assign_slots_redirect(ranked, k, E, C, unavailable)
        w = np.take_along_axis(pr, rk.astype(np.int64), axis=1)
        expert_offset, rank_offset, dest, pack_src = layout(idx, pos, keep, E, n_ranks, C,
                                                            unavailable, count=count)
    elif overflow == "drop":
        idx, w = route(logits, k, tau)
        pos, keep, load, count = assign_slots(idx, E, C, unavailable)
        expert_offset, rank_offset, dest, pack_src = layout(idx, pos, keep, E, n_ranks, C,
                                                            unavailable)
    else:
        raise ValueError(overflow)
    packed = pack(x, pack_src)
    out = dict(logits=logits, idx=idx, w=w, C=C, pos=pos, keep=keep,
               expert_load=load, expert_count=count, expert_offset=expert_offset,
               rank_offset=rank_offset, dest=dest, pack_src=pack_src,
               packed=packed)
    if W1 is not None:
        if keep_ret is None:
            keep_ret = pack_src.shape[0] * x.shape[1] <= (1 << 26)
        sh = None
        if shared is not None:
            sh = shared_ffn(x, shared[0], shared[2], shared[1], act)
            out["shared_out"] = sh
        if keep_ret:
            ret = expert_ffn(x, pack_src, expert_offset, e_begin, e_end, W1, W2, W3, act)
            out["ret"] = ret
            out["y"] = combine(ret, dest, w, x if add_residual else None, shared=sh)
        else:
            out["y"] = combine_by_segment(x, pack_src, expert_offset, e_begin, e_end, W1, W2,
                                          W3, act, dest, w, x if add_residual else None,
                                          shared=sh)
    return out


# ----------------------------------------------------------------------------
# routing-health signals
# ----------------------------------------------------------------------------
def routing_stats(logits: np.ndarray, expert_load: np.ndarray, expert_count: np.ndarray,
                  C: int, k: int, tau: float = 1.0) -> dict:
    """Routing-health signals of one batch, float64.

    [EP-glossary] "Practitioner Guidance": expert utilisation and routing
    entropy are first-class health signals; [EP-infinity] figure text: the
    bar of an expert is the share of its capacity used, a dashed bar an
    expert at capacity that drops; [EP-notes] "Components and
    Architecture", auxiliary load-balancing loss, Switch form: here
    sum_e f_e P_e with f_e the share of tokens that chose e and P_e its mean
    router probability (the caller applies the coefficient; the page prints
    no scaling by E).

    Readings (the pages give no formulas):
      prob_mean[e]  P_e = (1/B) sum_t p_te, p_t = softmax(g_t / tau);
      token_frac[e] f_e = n_e / B, the share of the B tokens that chose e
                    (each token counts once per chosen expert; sums to k);
      aux_loss      sum_e f_e P_e;
      entropy       routing entropy, the mean over tokens of
                    -sum_e p_te ln p_te (nats);
      load_entropy  -sum_e a_e ln a_e with a_e = n_e / (B k), the spread of
                    the assignments over the experts (nats; 0 ln 0 = 0);
      utilization[e] kept_e / C (0 when C = 0);
      dropped[e]    n_e - kept_e.
    With B = 0 every float is 0.  Pins: equal logits, one-hot logits, a
    perfectly balanced top-1 batch, a single hot expert, the overflow
    identity (test_oracle_health)."""
    l32 = np.asarray(logits, dtype=np.float32)
    B, E = l32.shape
    n = np.asarray(expert_load, dtype=np.int64).reshape(E)
    kept = np.asarray(expert_count, dtype=np.int64).reshape(E)
    if B == 0:
        z = np.zeros(E)
        return dict(prob_mean=z, token_frac=z.copy(), aux_loss=0.0, entropy=0.0,
                    load_entropy=0.0, utilization=z.copy(), dropped=n - kept)
    p = softmax(l32, tau)
    P = p.mean(axis=0)
    f = n / B
    plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    ent = float(-plogp.sum(axis=1).mean())
    a = n / (B * k)
    alog = np.where(a > 0, a * np.log(np.where(a > 0, a, 1.0)), 0.0)
    util = kept / C if C > 0 else np.zeros(E)
    return dict(prob_mean=P, token_frac=f, aux_loss=float((f * P).sum()), entropy=ent,
                load_entropy=float(-alog.sum()), utilization=util, dropped=n - kept)


# ----------------------------------------------------------------------------
# expert-choice routing (a variant)
# ----------------------------------------------------------------------------
def router_probs(logits: np.ndarray, tau: float = 1.0) -> np.ndarray:
    """The router's probabilities p_t = softmax(g_t / tau), rounded once to
    float32 [B, E]: the scores expert-choice routing ranks tokens by.  The
    choice below is decided on these float32 values (the precision the GPU
    holds them in), so both sides rank the same numbers.  Pins: as
    ``softmax``."""
    return softmax(logits, tau).astype(np.float32)


def expert_choice(probs: np.ndarray, C: int):
    """Every expert chooses its top-C tokens of the batch by score.

    [EP-notes] "Major Variants and Families", expert choice routing: the
    selection runs per expert over the batch's tokens rather than per token
    over the experts; expert e keeps the C tokens scoring highest in its
    column, so all experts get equal row counts and a token may be kept by
    several experts or by none.  Readings: the
    score of (t, e) is the router probability p_te (float32); C is the
    problem's capacity, at most B; among equal scores the lower token index
    wins; an expert's rows are packed in token order, experts one after the
    other; the weight of a chosen pair is p_te.

    Returns sel int32 [B, E] (packed row of (t, e), or -1), expert_offset
    int32 [E + 1] (= e * min(C, B)), pack_src int32 [E * min(C, B)] (token of
    each row) and pack_w float32 (p_te of each row).  Uses one library
    primitive per expert, a lexicographic sort by (-score, token).  Pins: a
    rank-counting brute force, exact balance, ties, C >= B (every expert
    takes every token) (test_oracle_expert_choice)."""
    p = np.asarray(probs, dtype=np.float32)
    B, E = p.shape
    Ce = min(int(C), B)
    sel = np.full((B, E), -1, dtype=np.int32)
    pack_src = np.empty(E * Ce, dtype=np.int32)
    pack_w = np.empty(E * Ce, dtype=np.float32)
    t_idx = np.arange(B)
    for e in range(E):
        order = np.lexsort((t_idx, -p[:, e].astype(np.float64)))  # score desc, token asc
        chosen = np.sort(order[:Ce])
        rows = e * Ce + np.arange(Ce)
        sel[chosen, e] = rows
        pack_src[rows] = chosen
        pack_w[rows] = p[chosen, e]
    expert_offset = (np.arange(E + 1) * Ce).astype(np.int32)
    return sel, expert_offset, pack_src, pack_w


def expert_choice_combine(ret: np.ndarray, sel: np.ndarray, pack_w: np.ndarray,
                          x_residual: Optional[np.ndarray] = None,
                          tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum over experts e that chose t, in expert order, of
    p_te * ret[row(t, e)] (+ x[t]), float64; a token no expert chose gets 0
    (plus the residual) -- [EP-notes] "Components and Architecture", expert
    combine weighted by the gating probabilities.  Pin: with C >= B it is the
    dense soft mixture sum_e p_te E_e(x_t) (test_oracle_expert_choice)."""
    B, E = sel.shape
    tt = np.arange(B) if tokens is None else np.asarray(tokens, dtype=np.int64)
    acc = np.zeros((tt.size, ret.shape[1]))
    w = np.asarray(pack_w, dtype=np.float32).astype(np.float64)
    for e in range(E):
        r = sel[tt, e].astype(np.int64)
        m = r >= 0
        acc[m] += w[r[m]][:, None] * ret[r[m]]
    if x_residual is not None:
        acc += _x_values(x_residual[tt])
    return acc


def forward_expert_choice(x, Wg, bias, W1, W3, W2, *, k: int, c: float, act: str,
                          tau: float = 1.0, C: Optional[int] = None,
                          add_residual: bool = False,
                          probs: Optional[np.ndarray] = None) -> dict:
    """The layer with expert-choice routing: gate, router probabilities,
    every expert's top-C tokens, pack, expert FFN, weighted combine.  C
    defaults to the problem's capacity ceil((B*k/E)*c) (k is the average
    number of experts per token).  ``probs`` may be given (the GPU's float32
    probabilities) so that the choice is taken on the same numbers."""
    B = x.shape[0]
    logits = gate_logits(x, Wg, bias)
    E = logits.shape[1]
    if probs is None:
        probs = router_probs(logits, tau)
    if C is None:
        C = capacity(B, k, E, c)
    sel, eo, src, pw = expert_choice(probs, C)
    out = dict(logits=logits, probs=probs, C=C, sel=sel, expert_offset=eo, pack_src=src,
               pack_w=pw, packed=pack(x, src))
    if W1 is not None:
        ret = expert_ffn(x, src, eo, 0, E, W1, W2, W3, act)
        out["ret"] = ret
        out["y"] = expert_choice_combine(ret, sel, pw, x if add_residual else None)
    return out


# ----------------------------------------------------------------------------
# backward pass (training)
# ----------------------------------------------------------------------------
# [EP-notes] "About": the sparsely gated layer is trained by backpropagation
# together with an auxiliary load-balancing loss; "Formal Algorithm", last
# step: the auxiliary loss is added to the training loss.  The pages give no
# backward formulas; the readings (also in the design notes):
#
# * the loss is L = sum_t <dy_t, y_t> + aux_coef * L_aux for a given output
#   gradient dy, with L_aux = sum_e f_e P_e as in ``routing_stats``: the token
#   shares f_e = n_e / B are counts (constant), P_e = (1/B) sum_t p_te is
#   differentiable;
# * the expert choice (top-k) and the capacity decision are piecewise
#   constant: no gradient flows through them, only through the gate weights
#   w_tj = p_{t, idx_tj} and the expert outputs; a dropped assignment is
#   absent from y, so it gets zero gradient (dw = 0, no expert rows);
# * rows of experts that run on other ranks come back unchanged in the
#   forward (identity return), so their gradient passes back unchanged;
# * everything in float64 on the defined input values (bf16 inputs widened
#   exactly), like the forward.


def combine_backward(dy: np.ndarray, ret: np.ndarray, dest: np.ndarray, w: np.ndarray,
                     rows: Optional[np.ndarray] = None):
    """Gradient of y[t] = sum_j [kept] w[t,j] ret[dest[t,j]] (+ x[t]).

    Returns dret [K, d] (or [len(rows), d] for the packed rows listed in
    ``rows``, sorted) with dret[dest[t,j]] = w[t,j] dy[t], and dw [B, k] with
    dw[t,j] = <dy[t], ret[dest[t,j]]> for kept assignments, 0 for dropped
    ones.  ``ret`` is the full return buffer, or with ``rows`` only those
    rows (the dw of assignments whose row is not listed is then not
    computed: NaN).  w is taken at float32 precision as in ``combine``.
    Pins: central finite differences of ``combine`` and torch float64
    autograd (test_oracle_backward)."""
    B, k = dest.shape
    dyv = np.asarray(dy, dtype=np.float64)
    w32 = np.asarray(w, dtype=np.float32).astype(np.float64)
    d = dyv.shape[1]
    nrow = ret.shape[0] if rows is None else len(rows)
    dret = np.zeros((nrow, d))
    dw = np.zeros((B, k))
    for j in range(k):
        dj = dest[:, j].astype(np.int64)
        kept = dj >= 0
        if rows is None:
            t = np.nonzero(kept)[0]
            r = dj[t]
            dret[r] = w32[t, j][:, None] * dyv[t]
            dw[t, j] = np.einsum("ij,ij->i", dyv[t], ret[r])
        else:
            pos = np.searchsorted(rows, dj)
            pos = np.minimum(pos, max(len(rows) - 1, 0))
            listed = kept & (len(rows) > 0) & (np.asarray(rows)[pos] == dj)
            t = np.nonzero(listed)[0]
            dret[pos[t]] = w32[t, j][:, None] * dyv[t]
            dw[t, j] = np.einsum("ij,ij->i", dyv[t], ret[pos[t]])
            dw[kept & ~listed, j] = np.nan
    return dret, dw


def route_backward(logits: np.ndarray, idx: np.ndarray, dw: np.ndarray, tau: float = 1.0,
                   aux_coef: float = 0.0, expert_load: Optional[np.ndarray] = None,
                   batch: Optional[int] = None):
    """Gradient of the loss with respect to the router logits [B, E].

    The gate weights are w[t,j] = p[t, idx[t,j]] with p_t = softmax(g_t / tau)
    ([EP-notes] "Formal Algorithm": w_t = p_{t,e(t)}), so with
    dp[t,e] = sum_j [idx[t,j] = e] dw[t,j] (+ aux_coef f_e / B from
    L_aux = sum_e f_e P_e, f_e = n_e / B constant):
    dl[t,e] = (1 / tau) p[t,e] (dp[t,e] - sum_e' p[t,e'] dp[t,e']).
    ``expert_load`` (n_e) is needed when aux_coef != 0.  ``batch``: the
    batch size B of the auxiliary term when ``logits`` holds only some of
    the batch's tokens (default: its row count).  Pins: central finite
    differences of softmax + top-k weights with the choice held fixed, and
    of the auxiliary loss (test_oracle_backward)."""
    p = softmax(logits, tau)
    B, E = p.shape
    dp = np.zeros((B, E))
    idx = np.asarray(idx, dtype=np.int64)
    np.add.at(dp, (np.repeat(np.arange(B), idx.shape[1]), idx.reshape(-1)),
              np.asarray(dw, dtype=np.float64).reshape(-1))
    if aux_coef != 0.0:
        Bb = B if batch is None else int(batch)
        f = np.asarray(expert_load, dtype=np.float64) / Bb
        dp += aux_coef * f[None, :] / Bb
    s = (p * dp).sum(axis=1, keepdims=True)
    return p * (dp - s) / float(tau)


def expert_mlp_backward(xr: np.ndarray, W1, W2, W3, act: str, dout: np.ndarray):
    """Gradient of one expert out = act(xr W1) W2 (SwiGLU: (silu(xr W1) *
    (xr W3)) W2) on rows xr [n, d] for the output gradient dout [n, d].

    With z1 = xr W1 (z3 = xr W3), h = gelu(z1) or silu(z1) z3:
    dh = dout W2^T; GELU: dz1 = dh gelu'(z1), gelu'(z) = Phi(z) + z phi(z);
    SwiGLU: dz1 = dh z3 silu'(z1), silu'(z) = s (1 + z (1 - s)), s the
    logistic, dz3 = dh silu(z1); dxr = dz1 W1^T (+ dz3 W3^T);
    dW1 = xr^T dz1, dW3 = xr^T dz3, dW2 = h^T dout.
    Returns (dxr, dW1, dW2, dW3 or None), float64.  Pins: central finite
    differences and torch float64 autograd (test_oracle_backward)."""
    w1 = _w(W1)
    w2 = _w(W2)
    z1 = xr @ w1
    dout = np.asarray(dout, dtype=np.float64)
    dh = dout @ w2.T
    if act == "gelu":
        h = gelu(z1)
        phi = np.exp(-0.5 * z1 * z1) / math.sqrt(2.0 * math.pi)
        Phi = 0.5 * (1.0 + _erf(z1 / math.sqrt(2.0)))
        dz1 = dh * (Phi + z1 * phi)
        dxr = dz1 @ w1.T
        return dxr, xr.T @ dz1, h.T @ dout, None
    if act == "swiglu":
        w3 = _w(W3)
        z3 = xr @ w3
        s = 1.0 / (1.0 + np.exp(-z1))
        h = z1 * s * z3
        dz1 = dh * z3 * s * (1.0 + z1 * (1.0 - s))
        dz3 = dh * z1 * s
        dxr = dz1 @ w1.T + dz3 @ w3.T
        return dxr, xr.T @ dz1, h.T @ dout, xr.T @ dz3
    raise ValueError(act)


def _erf(z):
    from scipy.special import erf
    return erf(z)


def expert_ffn_backward(x: np.ndarray, pack_src: np.ndarray, expert_offset: np.ndarray,
                        e_begin: int, e_end: int, W1, W2, W3, act: str, dret: np.ndarray,
                        rows: Optional[np.ndarray] = None,
                        experts: Optional[list] = None):
    """Backward of ``expert_ffn``: dXp (the gradient of each packed row's
    input) and the local experts' weight gradients.

    dret is [K, d] (or the listed ``rows`` only, sorted).  A local expert's
    rows get ``expert_mlp_backward``; rows of other ranks' experts pass
    dret through unchanged (the identity return).  Weight gradients are
    computed for ``experts`` (default: every local expert), each from all of
    its rows -- so with ``rows`` given they must include every row of those
    experts.  Returns (dXp, {e: (dW1, dW2, dW3)})."""
    pack_src = np.asarray(pack_src, dtype=np.int64)
    K = pack_src.shape[0]
    r_all = np.arange(K) if rows is None else np.asarray(rows, dtype=np.int64)
    dXp = np.array(dret, dtype=np.float64, copy=True)
    grads = {}
    want = list(range(e_begin, e_end)) if experts is None else list(experts)
    for e in range(e_begin, e_end):
        a, b = int(expert_offset[e]), int(expert_offset[e + 1])
        sel = np.nonzero((r_all >= a) & (r_all < b))[0]
        i = e - e_begin
        if sel.size == 0:
            if e in want:
                d, f = _w(W1[i]).shape
                grads[e] = (np.zeros((d, f)), np.zeros((f, d)),
                            None if W3 is None else np.zeros((d, f)))
            continue
        if e in want and sel.size != b - a:
            raise ValueError(f"expert {e}: weight gradients need all of its rows")
        xr = _x_values(x[pack_src[r_all[sel]]])
        dxr, dW1, dW2, dW3 = expert_mlp_backward(xr, W1[i], W2[i],
                                                 None if W3 is None else W3[i], act,
                                                 dret[sel])
        dXp[sel] = dxr
        if e in want:
            grads[e] = (dW1, dW2, dW3)
    return dXp, grads


def dispatch_backward(dXp: np.ndarray, dest: np.ndarray, tokens: Optional[np.ndarray] = None,
                      rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Backward of the pack: packed[r] = x[pack_src[r]], so
    dx[t] = sum_j [kept] dXp[dest[t,j]] ([B, d], or the listed tokens).
    ``rows`` says which packed rows dXp holds (sorted), when only some.
    Pin: the adjoint identity <pack(x), v> = <x, dispatch_backward(v)>
    (test_oracle_backward)."""
    B, k = dest.shape
    tt = np.arange(B) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((tt.size, dXp.shape[1]))
    for j in range(k):
        dj = dest[tt, j].astype(np.int64)
        m = dj >= 0
        r = dj[m] if rows is None else np.searchsorted(rows, dj[m])
        out[m] += dXp[r]
    return out


def gate_backward(x: np.ndarray, Wg: np.ndarray, dlogits: np.ndarray):
    """Backward of g = x Wg + b: dx = dl Wg^T [B, d], dWg = x^T dl [d, E],
    db = sum_t dl [E], float64 (x at its defined values).  Pin: central
    finite differences (test_oracle_backward)."""
    xv = _x_values(x)
    wg = np.asarray(Wg, dtype=np.float32).astype(np.float64)
    dl = np.asarray(dlogits, dtype=np.float64)
    return dl @ wg.T, xv.T @ dl, dl.sum(axis=0)


def backward(x, Wg, bias, W1, W3, W2, fwd: dict, dy, *, act: str, e_begin: int = 0,
             e_end: Optional[int] = None, tau: float = 1.0, aux_coef: float = 0.0,
             add_residual: bool = False) -> dict:
    """All gradients of the layer for the output gradient dy, given the
    forward's results ``fwd`` (``forward``'s dict with ``ret``): the steps of
    the forward in reverse -- combine, expert FFN, pack, route, gate.

    Returns dx [B, d], dWg [d, E], dbias [E], dW1 / dW3 [n_local, d, f],
    dW2 [n_local, f, d], dlogits [B, E], dw [B, k], dret and dXp [K, d]
    (float64).  Pins: torch float64 autograd of the whole layer with the
    routing held fixed, finite differences (test_oracle_backward)."""
    E = fwd["logits"].shape[1]
    e_end = E if e_end is None else e_end
    dest, w = fwd["dest"], fwd["w"]
    dret, dw = combine_backward(dy, fwd["ret"], dest, w)
    dl = route_backward(fwd["logits"], fwd["idx"], dw, tau, aux_coef, fwd["expert_load"])
    dXp, g = expert_ffn_backward(x, fwd["pack_src"], fwd["expert_offset"], e_begin, e_end,
                                 W1, W2, W3, act, dret)
    dx = dispatch_backward(dXp, dest)
    dxg, dWg, db = gate_backward(x, Wg, dl)
    dx += dxg
    if add_residual:
        dx += np.asarray(dy, dtype=np.float64)
    n_local = e_end - e_begin
    dW1 = np.stack([g[e][0] for e in range(e_begin, e_end)]) if n_local else None
    dW2 = np.stack([g[e][1] for e in range(e_begin, e_end)]) if n_local else None
    dW3 = (np.stack([g[e][2] for e in range(e_begin, e_end)])
           if n_local and W3 is not None else None)
    return dict(dx=dx, dWg=dWg, dbias=db, dW1=dW1, dW3=dW3, dW2=dW2, dlogits=dl, dw=dw,
                dret=dret, dXp=dXp)
