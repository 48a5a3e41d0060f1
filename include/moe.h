/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts layer forward.
 *
 * One MoE layer on one GPU's share of tokens, in the steps the pages give
 * ("Expert Parallelism", narrativegoldmine.com, section "Formal Algorithm:
 * Expert Parallelism Forward Pass"; "Expert Parallelism and the All-to-All
 * Bottleneck", ashishsrivastav.com, section "The Mechanism of Expert
 * Parallelism"):
 *
 *   moe_gate       router logits  g = x . Wg (+ b)                 (fp32)
 *   moe_route      softmax over E, top-k choice and gate weights
 *   moe_dispatch   per-expert capacity, slot assignment with drops, and the
 *                  pack that stands in for the dispatch all-to-all
 *   moe_expert_ffn grouped expert MLP on the packed rows (bf16 MFMA)
 *   moe_combine    gate-weighted sum back into token order (the return
 *                  all-to-all becomes the identity on one GPU)
 *   moe_forward    all of the above, enqueued back to back
 *
 * and, beside that path, the variants and signals the pages also describe:
 *
 *   moe_routing_stats   routing-health signals (utilisation, drops,
 *                       auxiliary loss, routing and load entropy)
 *   expert_unavailable  (a moe_problem_t field) experts with capacity 0
 *   overflow            (a moe_problem_t field) overflow redirected to the
 *                       next-best expert instead of dropped
 *   moe_shared_ffn, moe_combine_shared, moe_forward_shared
 *                       a shared expert on every token
 *   moe_router_probs, moe_expert_choice, moe_expert_choice_pack,
 *   moe_expert_choice_combine, moe_forward_expert_choice
 *                       expert-choice routing (experts pick their tokens)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is DEVICE memory unless stated otherwise; the
 *   caller allocates every buffer (and the workspace) and keeps ownership.
 *   The library allocates nothing and keeps no state between calls.
 * - Every call only enqueues work on `stream` and returns; results are valid
 *   once the stream reaches that point.  Nothing synchronizes the host.
 * - All arguments are checked on the host before anything is enqueued; a
 *   failed check returns an error code and enqueues nothing.  After the
 *   launches, a launch failure reported by the HIP runtime returns
 *   MOE_ERR_HIP.  Kernels have no device-side error path: integer inputs
 *   that come from the caller (topk_idx, dest) are treated as "dropped" when
 *   out of range rather than read out of bounds; float inputs are assumed
 *   finite.
 * - Row-major everywhere.  bf16 tensors are passed as raw 16-bit patterns
 *   (moe_bf16_t).  Pointers used with 16-byte vector accesses (x, packed,
 *   weights, y, ret, out) must be 16-byte aligned; d and f must be multiples
 *   of 8.
 * - Sizes: Kmax = min(B*k, E*C) bounds the number of kept assignments K; the
 *   exact K is expert_offset[E], known only on the device.
 * - Expert weights are [in, out] matrices, one per expert, row-major, as the
 *   layer's configurations print them: W1 and W3 are [n_local][d][f] and W2
 *   is [n_local][f][d], where n_local = e_end - e_begin; expert e computes,
 *   on a token row x, act(x . W1) . W2 (GELU) or (silu(x . W1) * (x . W3)) . W2
 *   (SwiGLU), with no biases.  The expert GEMM streams them from a blocked
 *   copy made once by moe_pack_weights (see there); moe_expert_ffn and
 *   moe_forward take that copy.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16_t; /* raw bf16 bits */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* a null required pointer, a bad size or field */
  MOE_ERR_UNSUPPORTED = 2, /* valid, but outside the sizes the kernels handle */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = 4          /* the HIP runtime reported a launch error */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;
typedef enum { MOE_GELU = 0, MOE_SWIGLU = 1 } moe_act_t;
typedef enum { MOE_OVERFLOW_DROP = 0, MOE_OVERFLOW_NEXT = 1 } moe_overflow_t;

/* Which call a workspace is sized for (moe_workspace_bytes). */
typedef enum {
  MOE_OP_DISPATCH = 0,
  MOE_OP_FFN = 1,
  MOE_OP_FORWARD = 2,
  MOE_OP_ROUTING_STATS = 3,
  MOE_OP_SHARED_FFN = 4,
  MOE_OP_FORWARD_EXPERT_CHOICE = 5,
  MOE_OP_EXPERT_FFN_BACKWARD = 6,
  MOE_OP_GATE_BACKWARD = 7,
  MOE_OP_BACKWARD = 8
} moe_op_t;

/* The problem statement: B tokens of hidden size d, E experts, top-k routing
 * with capacity factor c and per-expert capacity C = ceil((B*k/E)*c)
 * ("Expert Parallelism", theinfinity.ai, capacity paragraph, read per
 * expert); experts spread contiguously over n_ranks ranks, E/n_ranks each
 * ("Expert Parallelism and the All-to-All Bottleneck", section "The
 * All-to-All Communication Pattern"). */
typedef struct {
  int64_t B;          /* tokens, 0 .. 2^25 with B*k < 2^31 (0: empty batch)  */
  int32_t d;          /* hidden size, multiple of 8                          */
  int32_t E;          /* experts, 1..1024                                    */
  int32_t k;          /* experts per token, 1..min(E, 16)                    */
  double c;           /* capacity factor (> 0 when C < 0)                    */
  int32_t C;          /* < 0: computed as ceil((B*k/E)*c); >= 0: used as is */
  int32_t n_ranks;    /* D >= 1, E % D == 0; rank r owns [r*E/D, (r+1)*E/D) */
  int32_t e_begin;    /* experts whose FFN runs on this GPU: [e_begin, e_end) */
  int32_t e_end;
  int32_t f;          /* expert FFN inner size, multiple of 8                */
  int32_t act;        /* moe_act_t                                           */
  int32_t x_dtype;    /* moe_dtype_t of x and y                              */
  float tau;          /* softmax temperature (> 0), 1 by default             */
  int32_t add_residual; /* 1: y = x + combine; 0: y = combine              */
  /* DEVICE [E] uint8 or NULL.  A nonzero entry marks the expert unavailable
   * ("Expert Parallelism", inferensys.com glossary, "Risk and Threat
   * Considerations": an expert can become unavailable): its capacity is 0,
   * so every assignment to it is dropped exactly like overflow (keep = 0,
   * dest = -1, expert_count = 0).  NULL: every expert has capacity C.
   * Read by moe_dispatch and moe_forward; owned by the caller. */
  const uint8_t* expert_unavailable;
  /* moe_overflow_t: what happens to an assignment past its expert's
   * capacity ("Expert Parallelism", narrativegoldmine.com, "Components and
   * Architecture": overflow tokens are dropped or redirected to a secondary
   * expert).  MOE_OVERFLOW_DROP (0): dropped.  MOE_OVERFLOW_NEXT (1, read
   * by moe_forward only; moe_dispatch returns MOE_ERR_UNSUPPORTED): one
   * fallback round -- the m-th dropped choice of a token goes to its
   * (k + m)-th ranked expert (the router ranks min(2k, E) experts, so
   * min(2k, E) <= 16) and claims the capacity left after the first round, in
   * the original claim order q = j*B + t; what does not fit is dropped.
   * moe_forward's outputs then describe where each assignment ended:
   * topk_idx / topk_w the final expert and its probability, pos the slot
   * (-1 when dropped), expert_load the first-round n_e, expert_count the
   * rows kept in both rounds. */
  int32_t overflow;
} moe_problem_t;

/* ---- host-only helpers (no GPU work) ---------------------------------- */

/* ceil((B*k/E)*c) in IEEE double, in that order; 0 when B == 0; -1 on bad
 * arguments ("Expert Parallelism", theinfinity.ai, capacity paragraph). */
int32_t moe_capacity(int64_t B, int32_t k, int32_t E, double c);

/* The capacity the problem uses (C if C >= 0, else moe_capacity), or -1. */
int32_t moe_problem_capacity(const moe_problem_t* p);

/* min(B*k, E*C): rows the packed buffer must hold; -1 on a bad problem. */
int64_t moe_max_kept(const moe_problem_t* p);

/* Checks every field; MOE_OK or the error code a call would return. */
moe_status_t moe_validate(const moe_problem_t* p);

/* Workspace bytes `op` needs for problem p (0 if none; SIZE_MAX if p is
 * invalid).  The workspace is scratch owned by the caller; its contents on
 * entry do not matter. */
size_t moe_workspace_bytes(const moe_problem_t* p, moe_op_t op);

/* Static description of a status code. */
const char* moe_status_str(moe_status_t s);

/* ---- the path --------------------------------------------------------- */

/* Router logits ("Expert Parallelism", narrativegoldmine.com, "Formal
 * Algorithm", gate computation; "Components and Architecture": a learned
 * linear map with an optional bias on the logits).
 *   x      [B][d]  float32 (x_dtype F32) or bf16 (BF16)
 *   Wg     [d][E]  float32
 *   bias   [E]     float32, or NULL for none
 *   logits [B][E]  float32, out
 * fp32 x: the vector ALUs.  bf16 x: the matrix cores, with every fp32 weight
 * split exactly into three bf16 parts (hi + mid + lo), so each product is
 * exact and the sum is accumulated in fp32. */
moe_status_t moe_gate(const moe_problem_t* p, const void* x, const float* Wg,
                      const float* bias, float* logits, hipStream_t stream);

/* Softmax over E and top-k ("Formal Algorithm": p_t = softmax(g_t / tau),
 * e(t) = argmax p_t, w_t = p_{t,e(t)}; "Components and Architecture": the
 * top-k experts are selected).  Experts are ranked by (logit descending,
 * index ascending): the exact-probability order with ties to the lower
 * index.  topk_w holds the raw (not renormalised) probabilities; choice j = 0
 * is the strongest.
 *   logits   [B][E] float32, in
 *   topk_idx [B][k] int32, out
 *   topk_w   [B][k] float32, out */
moe_status_t moe_route(const moe_problem_t* p, const float* logits,
                       int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* Capacity-limited slot assignment and pack ("Expert Parallelism",
 * theinfinity.ai, capacity paragraph: tokens past C are dropped, overflow
 * max(0, n_e - C); "Expert Parallelism and the All-to-All Bottleneck", "The
 * Mechanism of Expert Parallelism": rows repacked per destination expert).
 * Assignment (t, j) claims its expert's next slot in the order q = j*B + t;
 * pos is its slot, keep = pos < C.  Kept rows are packed compactly,
 * expert-major (so rank-major), in claim order.
 *   x             [B][d]   f32 or bf16 (f32 is rounded to nearest-even bf16)
 *   topk_idx      [B][k]   int32 in [0, E) (others count as dropped)
 *   pos           [B][k]   int32 out (slot; -1 for an out-of-range index)
 *   keep          [B][k]   uint8 out
 *   dest          [B][k]   int32 out: packed row, or -1 when dropped
 *   expert_load   [E]      int32 out n_e (assignments routed), may be NULL
 *   expert_count  [E]      int32 out min(n_e, C)
 *   expert_offset [E+1]    int32 out exclusive prefix sum of expert_count
 *   rank_offset   [D+1]    int32 out expert_offset[r*E/D]
 *   pack_src      [Kmax]   int32 out token of each packed row
 *   packed        [Kmax][d] bf16 out
 *   ws / ws_bytes          workspace, >= moe_workspace_bytes(p, MOE_OP_DISPATCH)
 * Deterministic: no result depends on the order of atomic operations. */
moe_status_t moe_dispatch(const moe_problem_t* p, const void* x,
                          const int32_t* topk_idx, int32_t* pos, uint8_t* keep,
                          int32_t* dest, int32_t* expert_load,
                          int32_t* expert_count, int32_t* expert_offset,
                          int32_t* rank_offset, int32_t* pack_src,
                          moe_bf16_t* packed, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Size of the device-resident table moe_dispatch_noalloc works in. */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* moe_dispatch with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc.  Same arguments, results and errors as
 * moe_dispatch, except that the slot kernels' scratch (a per-tile expert
 * count table, moe_workspace_bytes(p, MOE_OP_DISPATCH) bytes) lives in a
 * fixed device array of MOE_DISPATCH_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; nothing is
 * allocated or freed by the call.  Problems whose table exceeds that size
 * return MOE_ERR_UNSUPPORTED before any launch (use moe_dispatch); a
 * failure looking up the array's device address returns MOE_ERR_HIP.  All
 * calls on one GPU share the array: calls that may overlap on one GPU (on
 * unordered streams) race and must not be issued; calls ordered on one
 * stream are fine (nothing in the array needs to start at zero). */
moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const void* x,
                                  const int32_t* topk_idx, int32_t* pos, uint8_t* keep,
                                  int32_t* dest, int32_t* expert_load, int32_t* expert_count,
                                  int32_t* expert_offset, int32_t* rank_offset,
                                  int32_t* pack_src, moe_bf16_t* packed, hipStream_t stream);

/* Bytes of the blocked expert-weight copy for problem p (SIZE_MAX if p is
 * invalid). */
size_t moe_weights_bytes(const moe_problem_t* p);

/* Rearranges the local experts' weights into the blocked layout the expert
 * GEMM streams: per expert, per output tile (256 output columns of W1 or W2,
 * or 128 columns of W1 plus the same 128 columns of W3 for SwiGLU) and per
 * 64-wide K slice, one contiguous 32 KB block whose columns and 16-byte K
 * chunks are in the order the GEMM's matrix-core fragments take them;
 * padding past f or d is zero.  A one-time format conversion (weights are
 * parameters), not part of the layer; the caller does it when the weights
 * are loaded and owns the copy ("Expert Parallelism", narrativegoldmine.com,
 * "Components and Architecture", Expert GEMM: each expert is a standard
 * MLP, x . W1 then x . W2).
 *   W1, W3  [n_local][d][f] bf16, [in, out] (W3 only for SwiGLU, else NULL)
 *   W2      [n_local][f][d] bf16, [in, out]
 *   wpacked moe_weights_bytes(p) bytes, 16-byte aligned, out
 * The library cannot see tensor shapes: a matrix in the transposed layout
 * has the same size and is not detected here (the Python binding checks
 * full shapes). */
moe_status_t moe_pack_weights(const moe_problem_t* p, const moe_bf16_t* W1,
                              const moe_bf16_t* W3, const moe_bf16_t* W2,
                              void* wpacked, size_t wpacked_bytes,
                              hipStream_t stream);

/* Grouped expert MLP ("Expert Parallelism", narrativegoldmine.com,
 * "Components and Architecture", Expert GEMM; "Formal Algorithm", expert
 * computation on the received tokens).  For every expert e in
 * [e_begin, e_end) and its packed rows [expert_offset[e], expert_offset[e+1]):
 * ret = W2 . act(W1 . x), with bf16 operands, fp32 accumulation and the
 * hidden activation stored as bf16 in the workspace.  Rows of other experts
 * come back unchanged (the missing collective is the identity): with
 * ret == packed nothing is copied, otherwise they are copied to ret.
 *   packed        [Kmax][d] bf16 in
 *   expert_offset [E+1]     int32 in (as written by moe_dispatch)
 *   wpacked       the local experts' weights as written by moe_pack_weights
 *   ret           [Kmax][d] bf16 out; may alias packed
 *   ws / ws_bytes workspace, >= moe_workspace_bytes(p, MOE_OP_FFN) */
moe_status_t moe_expert_ffn(const moe_problem_t* p, const moe_bf16_t* packed,
                            const int32_t* expert_offset, const void* wpacked,
                            moe_bf16_t* ret, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Gate-weighted combine back into token order ("Components and
 * Architecture", expert combine; "Formal Algorithm", residual addition):
 * y[t] = sum_{j<k, dest[t,j]>=0} topk_w[t,j] * ret[dest[t,j]]  (+ x[t]),
 * accumulated in fp32 in j order.  A token whose choices were all dropped
 * gets 0 (or x[t] with the residual).
 *   ret        [Kmax][d] bf16
 *   dest       [B][k] int32 (as written by moe_dispatch)
 *   topk_w     [B][k] float32
 *   x_residual [B][d] x_dtype, required iff add_residual, else ignored
 *   y          [B][d] x_dtype out */
moe_status_t moe_combine(const moe_problem_t* p, const moe_bf16_t* ret,
                         const int32_t* dest, const float* topk_w,
                         const void* x_residual, void* y, hipStream_t stream);

/* Inverse of the pack: out[t][j] = ret[dest[t][j]], zeros where dropped
 * ("The Mechanism of Expert Parallelism": rows return to the original token
 * order).  A checking aid; out is [B][k][d] bf16. */
moe_status_t moe_unpack(const moe_problem_t* p, const moe_bf16_t* ret,
                        const int32_t* dest, moe_bf16_t* out,
                        hipStream_t stream);

/* Routing-health signals of one batch ("Expert Parallelism", inferensys.com
 * glossary, "Practitioner Guidance": expert utilisation and routing entropy
 * as health signals; narrativegoldmine.com, "Components and Architecture",
 * auxiliary load-balancing loss, Switch form: sum over experts of the token
 * share f_e times the mean router probability P_e;
 * theinfinity.ai, figure text: each expert's bar is the share of its
 * capacity in use).  With p_t = softmax(logits_t / tau), n_e = expert_load,
 * kept_e = expert_count and C the problem's capacity:
 *   prob_mean   [E] float   P_e = (1/B) sum_t p_te
 *   token_frac  [E] float   f_e = n_e / B (sums to k)
 *   utilization [E] float   kept_e / C (0 when C = 0)
 *   dropped     [E] int32   n_e - kept_e
 *   summary     [5] double  aux loss sum_e f_e P_e (the caller applies the
 *                           coefficient), routing entropy (mean over tokens
 *                           of -sum_e p_te ln p_te, nats), load entropy
 *                           (-sum_e a_e ln a_e, a_e = n_e / (B k), nats),
 *                           dropped total, kept total
 * Any field may be NULL (not written).  With B = 0 the floats are 0. */
typedef struct {
  float* prob_mean;
  float* token_frac;
  float* utilization;
  int32_t* dropped;
  double* summary;
} moe_routing_stats_t;

/* Routing-health signals ("Expert Parallelism", inferensys.com glossary,
 * Practitioner Guidance: utilization and routing entropy as health signals;
 * "Expert Parallelism", narrativegoldmine.com, "Components and
 * Architecture": the auxiliary load-balancing loss).
 * Fills *out (device buffers) from the router logits [B][E] float32 and the
 * dispatch counts expert_load / expert_count [E] int32 (as written by
 * moe_dispatch or moe_forward).  Deterministic: fixed-order reductions,
 * per-block fp32 partial sums combined in double.
 *   ws / ws_bytes  workspace, >= moe_workspace_bytes(p, MOE_OP_ROUTING_STATS) */
moe_status_t moe_routing_stats(const moe_problem_t* p, const float* logits,
                               const int32_t* expert_load,
                               const int32_t* expert_count,
                               const moe_routing_stats_t* out, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Number of stage events of moe_forward_out_t. */
#define MOE_STAGE_EVENTS 11

/* Optional outputs of moe_forward; any NULL field lives in the workspace. */
typedef struct {
  float* logits;          /* [B][E]   */
  int32_t* topk_idx;      /* [B][k]   */
  float* topk_w;          /* [B][k]   */
  int32_t* pos;           /* [B][k]   */
  uint8_t* keep;          /* [B][k]   */
  int32_t* dest;          /* [B][k]   */
  int32_t* expert_load;   /* [E]      */
  int32_t* expert_count;  /* [E]      */
  int32_t* expert_offset; /* [E+1]    */
  int32_t* rank_offset;   /* [D+1]    */
  int32_t* pack_src;      /* [Kmax]   */
  moe_bf16_t* packed;     /* [Kmax][d]: holds ret after the call (the expert
                             outputs overwrite the local rows in place) */
  moe_bf16_t* z;          /* optional, moe_saved_z_bytes(p) bytes, 16-byte
                             aligned (else MOE_ERR_INVALID): the local rows'
                             pre-activations X . W1 (and X . W3), bf16, in
                             the first expert GEMM's own column order (to be
                             passed back, not read), stored by that GEMM for
                             moe_backward, which then does not recompute
                             them; NULL: not stored (and not in the
                             workspace either) */
  moe_bf16_t* z_shared;   /* moe_forward_shared only, optional,
                             moe_saved_z_bytes(ps) bytes, 16-byte aligned:
                             the same for the shared expert (all B rows),
                             read by moe_backward_shared; NULL: not stored.
                             Must be NULL for moe_forward (else
                             MOE_ERR_INVALID). */
  /* Optional timing: each non-NULL events[i] is recorded on the call's
   * stream from the dispatch timestamps of the stages' own kernels
   * (hipExtLaunchKernelGGL start / end events; no marker packets):
   *   0 gate start          1 gate end
   *   2 route start         3 route end
   *   4 dispatch end (the pack kernel; 3 -> 4 is the slot kernels + pack;
   *     a marker after the slot kernels when the pack has nothing to write:
   *     bf16 tokens and every expert local, see below)
   *   5 expert FFN start    6 end of its first GEMM
   *   7 start of its second GEMM (after the routed GEMMs: the shared
   *     expert's, when there is one)      8 expert FFN end
   *   9 combine start      10 combine end
   * so 1 -> 2, 4 -> 5, 6 -> 7 and 8 -> 9 are the gaps between launches.  A
   * launch that carries an event is timestamped by the runtime, which
   * leaves a gap of a few microseconds on each side of it; launches without
   * events follow each other with none, so time a stage on its own steps.
   * With B == 0 no kernel runs and every event is recorded as a marker.
   * The caller owns the events (created with timing enabled). */
  hipEvent_t events[MOE_STAGE_EVENTS];
} moe_forward_out_t;

/* The whole layer, enqueued on one stream with no host synchronisation, in
 * the order of "Expert Parallelism" (narrativegoldmine.com), "Formal
 * Algorithm: Expert Parallelism Forward Pass" -- router logits, softmax and
 * top-k, dispatch under the capacity, expert computation, weighted combine
 * (and the residual when add_residual) -- with the two all-to-alls of "Expert
 * Parallelism and the All-to-All Bottleneck", "The Mechanism of Expert
 * Parallelism", replaced by the on-device pack and the identity return:
 * gate, route, dispatch, expert FFN (in place on the packed rows), combine.
 * With bf16 tokens the expert FFN's first GEMM reads the local experts'
 * rows straight from x through pack_src, and the pack writes only the rows
 * bound for other ranks (nothing when every expert is local): the same rows
 * in the same order as moe_dispatch + moe_expert_ffn, without the local
 * copy's round trip through HBM.
 * Errors: as the stage calls (checks before any launch); MOE_ERR_WORKSPACE
 * when ws is smaller than moe_workspace_bytes(p, MOE_OP_FORWARD).
 *   x [B][d] x_dtype; Wg [d][E] f32; bias [E] f32 or NULL;
 *   wpacked as in moe_expert_ffn; y [B][d] x_dtype out;
 *   out may be NULL; ws >= moe_workspace_bytes(p, MOE_OP_FORWARD). */
moe_status_t moe_forward(const moe_problem_t* p, const void* x, const float* Wg,
                         const float* bias, const void* wpacked, void* y,
                         moe_forward_out_t* out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* ---- shared expert --------------------------------------------------- */

/* A shared expert ("Expert Parallelism", narrativegoldmine.com, "Major
 * Variants and Families", shared expert routing: one or more experts
 * process every token in addition to the routed experts, a dense path
 * beside them).  It is described by its own problem ps: the same B and d as
 * the routed layer, E = 1, k = 1, e_begin = 0, e_end = 1, its own f and
 * act, x_dtype BF16 (other x types return MOE_ERR_UNSUPPORTED); its weights
 * are packed with moe_pack_weights(ps, W1s, W3s, W2s, ...).
 *
 * moe_shared_ffn: out[t] = W2s . act(W1s . x[t]) for every token (bf16
 * operands, fp32 accumulation, the hidden activation stored as bf16), on
 * the expert GEMM of moe_expert_ffn with all B rows as one expert.
 *   x       [B][d] bf16
 *   wpacked moe_pack_weights(ps, ...) output
 *   out     [B][d] bf16 out
 *   ws      >= moe_workspace_bytes(ps, MOE_OP_SHARED_FFN), 16-byte aligned */
moe_status_t moe_shared_ffn(const moe_problem_t* ps, const moe_bf16_t* x,
                            const void* wpacked, moe_bf16_t* out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* Shared expert ("Expert Parallelism", narrativegoldmine.com, "Major
 * Variants and Families", shared expert routing).
 * moe_combine plus a shared expert's rows, added with weight 1 after the
 * routed sum (and before the residual):
 * y[t] = sum_j topk_w[t,j] ret[dest[t,j]] + shared_out[t] (+ x[t]).
 *   shared_out [B][d] bf16 (moe_shared_ffn's out); the rest as moe_combine */
moe_status_t moe_combine_shared(const moe_problem_t* p, const moe_bf16_t* ret,
                                const int32_t* dest, const float* topk_w,
                                const moe_bf16_t* shared_out,
                                const void* x_residual, void* y,
                                hipStream_t stream);

/* Workspace of moe_forward_shared (SIZE_MAX if either problem is invalid). */
size_t moe_forward_shared_workspace_bytes(const moe_problem_t* p,
                                          const moe_problem_t* ps);

/* Shared expert ("Expert Parallelism", narrativegoldmine.com, "Major
 * Variants and Families", shared expert routing).
 * moe_forward with a shared expert: the routed layer of p, the shared
 * expert of ps on every token (after the routed expert GEMMs, inside the
 * stage events 5 and 6), and the combine of moe_combine_shared.
 * x_dtype must be BF16 for both problems; ps->B == p->B, ps->d == p->d.
 *   wpacked_shared  moe_pack_weights(ps, ...) output
 *   ws >= moe_forward_shared_workspace_bytes(p, ps), 16-byte aligned;
 *   the other arguments as moe_forward. */
moe_status_t moe_forward_shared(const moe_problem_t* p, const moe_problem_t* ps,
                                const void* x, const float* Wg,
                                const float* bias, const void* wpacked,
                                const void* wpacked_shared, void* y,
                                moe_forward_out_t* out, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* ---- expert-choice routing -------------------------------------------- */

/* Expert-choice routing ("Expert Parallelism", narrativegoldmine.com,
 * "Major Variants and Families", expert choice routing): instead of each
 * token choosing k experts, every expert chooses its top-C tokens of the
 * batch, so every expert processes exactly Ce = min(C, B) tokens and a token
 * may be chosen by any number of experts (including none).  C is the
 * problem's capacity ceil((B*k/E)*c), k read as the average number of
 * experts per token.  The score of (t, e) is the router probability
 * p_te = softmax(logits_t / tau)_e in fp32; among equal scores the lower
 * token wins; expert e's rows are e*Ce .. e*Ce + Ce - 1, in token order; the
 * weight of a chosen pair is p_te.  All experts must be local
 * (e_begin = 0, e_end = E; otherwise MOE_ERR_UNSUPPORTED).  R = E * Ce rows. */

/* R = E * min(C, B), the rows of an expert-choice layout; -1 if invalid. */
int64_t moe_expert_choice_rows(const moe_problem_t* p);

/* probs_t [E][B] float32 out: p_te, transposed (one expert's scores
 * contiguous).  logits [B][E] float32. */
moe_status_t moe_router_probs(const moe_problem_t* p, const float* logits,
                              float* probs_t, hipStream_t stream);

/* Every expert's top-Ce tokens from probs_t [E][B]:
 *   sel_t         [E][B] int32 out: packed row of (t, e), or -1
 *   expert_offset [E+1]  int32 out: e * Ce
 *   pack_src      [R]    int32 out: token of each row
 *   pack_w        [R]    float32 out: p_te of each row
 * Exact (a radix select on the fp32 bit patterns and an ordered pass). */
moe_status_t moe_expert_choice(const moe_problem_t* p, const float* probs_t,
                               int32_t* sel_t, int32_t* expert_offset,
                               int32_t* pack_src, float* pack_w,
                               hipStream_t stream);

/* packed[r] = bf16(x[pack_src[r]]) for the R rows.  x [B][d] x_dtype. */
moe_status_t moe_expert_choice_pack(const moe_problem_t* p, const void* x,
                                    const int32_t* pack_src, moe_bf16_t* packed,
                                    hipStream_t stream);

/* y[t] = sum over the experts e that chose t, in expert order, of
 * p_te * ret[row(t, e)] (+ x[t]), fp32; 0 (or x[t]) for a token no expert
 * chose.  ret [R][d] bf16 (moe_expert_ffn on the expert-choice layout,
 * expert_offset from moe_expert_choice), sel_t and pack_w as written by
 * moe_expert_choice; x_residual as in moe_combine. */
moe_status_t moe_expert_choice_combine(const moe_problem_t* p,
                                       const moe_bf16_t* ret,
                                       const int32_t* sel_t,
                                       const float* pack_w,
                                       const void* x_residual, void* y,
                                       hipStream_t stream);

/* Optional outputs of moe_forward_expert_choice; NULL fields live in the
 * workspace.  packed holds ret after the call (FFN in place).  events:
 * each non-NULL one recorded on the stream -- 0 before the gate, 1 after
 * it, 2 after the router probabilities and the choice (markers), 3 / 4 the
 * expert FFN's first dispatch start and last dispatch end, 5 after the
 * combine (marker); the pack falls in 2 -> 3. */
typedef struct {
  float* logits;          /* [B][E] */
  float* probs_t;         /* [E][B] */
  int32_t* sel_t;         /* [E][B] */
  int32_t* expert_offset; /* [E+1]  */
  int32_t* pack_src;      /* [R]    */
  float* pack_w;          /* [R]    */
  moe_bf16_t* packed;     /* [R][d] */
  hipEvent_t events[6];
} moe_expert_choice_out_t;

/* The layer with expert-choice routing on one stream: gate, router
 * probabilities, every expert's top-Ce tokens, gather pack, expert FFN (the
 * grouped GEMM of moe_expert_ffn, Ce rows per expert), combine.  (Use this
 * entry for the expert FFN of an expert-choice layout: moe_expert_ffn's
 * workspace is sized for the token-choice layout's Kmax rows, and R can be
 * larger.)
 *   ws >= moe_workspace_bytes(p, MOE_OP_FORWARD_EXPERT_CHOICE); the other
 *   arguments as moe_forward (wpacked: moe_pack_weights of all E experts). */
moe_status_t moe_forward_expert_choice(const moe_problem_t* p, const void* x,
                                       const float* Wg, const float* bias,
                                       const void* wpacked, void* y,
                                       moe_expert_choice_out_t* out, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/* ---- backward pass (training) ------------------------------------------ */

/* The layer's gradients for an output gradient dy ("Expert Parallelism",
 * narrativegoldmine.com, "About": the sparsely gated layer is trained by
 * backpropagation with an auxiliary load-balancing loss; "Formal
 * Algorithm", last step: the auxiliary loss joins the training loss).  The
 * loss is L = sum_t <dy_t, y_t> + aux_coef * sum_e f_e P_e (f_e = n_e / B
 * counts, constant; P_e the mean router probability).  The top-k choice and
 * the capacity decision are held fixed: gradient flows through the gate
 * weights w_tj = p_{t, idx_tj} and the expert outputs only, and a dropped
 * assignment gets none.  Rows of other ranks' experts pass their gradient
 * back unchanged (their forward return is the identity).  Supported: the
 * drop policy (MOE_OVERFLOW_NEXT returns MOE_ERR_UNSUPPORTED), with or
 * without the residual, any local expert range, the unavailable mask (it
 * only shows in dest).  Matrix products run on bf16 matrix cores with fp32
 * accumulation: dret, the recomputed pre-activations Z, dZ and H are bf16;
 * the router's fp32 operands are split exactly into bf16 parts.  Every call
 * checks its arguments on the host before any launch. */

/* Combine backward: dret[dest[t,j]] = topk_w[t,j] * dy[t] (bf16) and
 * dw[t,j] = <dy[t], ret[dest[t,j]]> (fp32; 0 for a dropped choice).
 *   dy [B][d] x_dtype; ret [Kmax][d] bf16 (the forward's expert outputs);
 *   dest, topk_w [B][k]; dret [Kmax][d] bf16 out (rows of dropped
 *   assignments are not written); dw [B][k] float out. */
moe_status_t moe_combine_backward(const moe_problem_t* p, const void* dy, const moe_bf16_t* ret,
                                  const int32_t* dest, const float* topk_w, moe_bf16_t* dret,
                                  float* dw, hipStream_t stream);

/* "Expert Parallelism", narrativegoldmine.com, "Formal Algorithm" (the
 * weights w_t = p_{t,e(t)}; the auxiliary loss joins the training loss) and
 * "Components and Architecture" (auxiliary load-balancing loss).
 * Router backward: with p_t = softmax(logits_t / tau) and
 * dp[t,e] = sum_j [topk_idx[t,j] = e] dw[t,j] + aux_coef n_e / B^2,
 * dlogits[t,e] = p[t,e] (dp[t,e] - sum_e' p[t,e'] dp[t,e']) / tau.
 *   logits [B][E]; topk_idx, dw [B][k]; expert_load [E] (n_e; may be NULL
 *   when aux_coef == 0); dlogits [B][E] float out. */
moe_status_t moe_route_backward(const moe_problem_t* p, const float* logits,
                                const int32_t* topk_idx, const float* dw,
                                const int32_t* expert_load, float aux_coef, float* dlogits,
                                hipStream_t stream);

/* Bytes of moe_forward_out_t.z: Kloc rows (the local experts' row
 * capacity) of the first expert GEMM's output width, bf16.  The backward
 * reads it in place of recomputing that GEMM; the values are the same bits
 * (the same kernel, the same order of operations). */
size_t moe_saved_z_bytes(const moe_problem_t* p);

/* Bytes of the blocked backward copy of the local experts' weights. */
size_t moe_weights_bwd_bytes(const moe_problem_t* p);

/* The weights rearranged for the expert backward's matrix products (the
 * transposed roles: dH = dret . W2^T and dX = [dZ1 | dZ3] . [W1 | W3]^T),
 * from the same [in, out] matrices as moe_pack_weights; a format
 * conversion done when the weights change, owned by the caller.
 *   W1, W3 [n_local][d][f]; W2 [n_local][f][d]; wpacked_bwd
 *   moe_weights_bwd_bytes(p) bytes, 16-byte aligned, out. */
moe_status_t moe_pack_weights_bwd(const moe_problem_t* p, const moe_bf16_t* W1,
                                  const moe_bf16_t* W3, const moe_bf16_t* W2,
                                  void* wpacked_bwd, size_t wpacked_bwd_bytes,
                                  hipStream_t stream);

/* "Expert Parallelism", narrativegoldmine.com, "Components and
 * Architecture" (the expert GEMM: a standard MLP per expert) and "About"
 * (training by backpropagation).
 * Expert FFN backward.  For each local expert and its packed rows
 * (X = x[pack_src[r]], bf16): the pre-activations Z = X . W1 (and X . W3)
 * are taken from z when the forward saved them (moe_forward_out_t.z) or
 * recomputed (z NULL), then dH = dret . W2^T, dZ = dH * act'(Z) (SwiGLU:
 * dZ1 = dH Z3 silu'(Z1), dZ3 = dH silu(Z1)), dX = dZ1 . W1^T (+ dZ3 . W3^T),
 * dW2 = H^T . dret, dW1 = X^T . dZ1, dW3 = X^T . dZ3 (H = act(Z), bf16).
 * dret is overwritten in place: its local rows become dX, the gradient of
 * the packed rows (other rows already are: the identity return).
 *   x [B][d] x_dtype; pack_src, expert_offset as written by the forward;
 *   wpacked (moe_pack_weights), wpacked_bwd (moe_pack_weights_bwd);
 *   dret [Kmax][d] bf16 in/out; dW1, dW3 [n_local][d][f], dW2
 *   [n_local][f][d] float out (dW3 NULL unless SwiGLU); an expert with no
 *   rows gets zero gradients.
 *   ws >= moe_workspace_bytes(p, MOE_OP_EXPERT_FFN_BACKWARD), 16-byte aligned */
moe_status_t moe_expert_ffn_backward(const moe_problem_t* p, const void* x,
                                     const int32_t* pack_src, const int32_t* expert_offset,
                                     const void* wpacked, const void* wpacked_bwd,
                                     const moe_bf16_t* z, moe_bf16_t* dret, float* dW1,
                                     float* dW3, float* dW2, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* "Expert Parallelism and the All-to-All Bottleneck", "The Mechanism of
 * Expert Parallelism": the rows travel to their experts and back.
 * Dispatch (pack) backward: dx_acc[t] = sum_j dXp[dest[t,j]] over kept
 * choices, in j order, plus dy[t] when the problem adds the residual.
 *   dxp [Kmax][d] bf16; dest [B][k]; dy [B][d] x_dtype (read only with the
 *   residual); dx_acc [B][d] float out. */
moe_status_t moe_dispatch_backward(const moe_problem_t* p, const moe_bf16_t* dxp,
                                   const int32_t* dest, const void* dy, float* dx_acc,
                                   hipStream_t stream);

/* "Expert Parallelism", narrativegoldmine.com, "Formal Algorithm": the
 * router logits as a linear projection of the token.
 * Gate backward: dx = dlogits . Wg^T (+ dx_acc), dWg = x^T . dlogits,
 * dbias = sum_t dlogits[t] (bias of the logits).
 *   x [B][d] x_dtype; Wg [d][E]; dlogits [B][E]; dx_acc [B][d] float or
 *   NULL; dx [B][d] x_dtype out; dWg [d][E] float out; dbias [E] float out
 *   or NULL.  ws >= moe_workspace_bytes(p, MOE_OP_GATE_BACKWARD). */
moe_status_t moe_gate_backward(const moe_problem_t* p, const void* x, const float* Wg,
                               const float* dlogits, const float* dx_acc, void* dx, float* dWg,
                               float* dbias, void* ws, size_t ws_bytes, hipStream_t stream);

/* What the backward reads from the forward (moe_forward's outputs, with
 * packed holding the expert outputs after the call). */
typedef struct {
  const float* logits;          /* [B][E]   */
  const int32_t* topk_idx;      /* [B][k]   */
  const float* topk_w;          /* [B][k]   */
  const int32_t* dest;          /* [B][k]   */
  const int32_t* expert_load;   /* [E]      */
  const int32_t* expert_offset; /* [E+1]    */
  const int32_t* pack_src;      /* [Kmax]   */
  const moe_bf16_t* ret;        /* [Kmax][d] */
  const moe_bf16_t* z;          /* moe_forward_out_t.z, or NULL: recompute */
  const moe_bf16_t* z_shared;   /* moe_forward_out_t.z_shared (moe_backward_shared
                                   only), or NULL: recompute */
} moe_saved_t;

/* The gradients moe_backward writes; dW3 only for SwiGLU, dbias may be
 * NULL, dlogits / dw NULL -> workspace. */
typedef struct {
  void* dx;       /* [B][d] x_dtype      */
  float* dWg;     /* [d][E]              */
  float* dbias;   /* [E]                 */
  float* dW1;     /* [n_local][d][f]     */
  float* dW3;     /* [n_local][d][f]     */
  float* dW2;     /* [n_local][f][d]     */
  float* dlogits; /* [B][E]              */
  float* dw;      /* [B][k]              */
} moe_grads_t;

/* "Expert Parallelism", narrativegoldmine.com, "About" (the layer trained
 * by backpropagation with an auxiliary load-balancing loss).
 * The whole backward on one stream: combine, route, expert FFN, dispatch
 * and gate backward, in that order (the forward's steps reversed).
 *   ws >= moe_workspace_bytes(p, MOE_OP_BACKWARD), 16-byte aligned. */
moe_status_t moe_backward(const moe_problem_t* p, const void* x, const float* Wg,
                          const void* wpacked, const void* wpacked_bwd, const moe_saved_t* saved,
                          const void* dy, float aux_coef, const moe_grads_t* grads, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Workspace of moe_backward_shared (SIZE_MAX if either problem is invalid). */
size_t moe_backward_shared_workspace_bytes(const moe_problem_t* p,
                                           const moe_problem_t* ps);

/* moe_backward for the layer of moe_forward_shared: the routed backward of
 * p, and the shared expert of ps ("Expert Parallelism", narrativegoldmine.com,
 * "Major Variants and Families", shared expert routing), whose output joins y
 * with weight 1, so that its output gradient is dy itself: its weight
 * gradients, and its input gradient added (in fp32) to the tokens' routed
 * input gradient before the router's part is added.
 *   ps as for moe_forward_shared (same B and d, E = 1, bf16 x);
 *   wpacked_shared, wpacked_shared_bwd: moe_pack_weights(ps, ...) and
 *   moe_pack_weights_bwd(ps, ...); dW1s, dW3s [d][fs] (dW3s only for a
 *   SwiGLU shared expert, else NULL), dW2s [fs][d] float out;
 *   ws >= moe_backward_shared_workspace_bytes(p, ps), 16-byte aligned;
 *   the other arguments as moe_backward. */
moe_status_t moe_backward_shared(const moe_problem_t* p, const moe_problem_t* ps,
                                 const void* x, const float* Wg, const void* wpacked,
                                 const void* wpacked_bwd, const void* wpacked_shared,
                                 const void* wpacked_shared_bwd, const moe_saved_t* saved,
                                 const void* dy, float aux_coef, const moe_grads_t* grads,
                                 float* dW1s, float* dW3s, float* dW2s, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
