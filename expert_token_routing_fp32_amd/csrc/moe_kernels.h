// Internal interface between the C ABI (moe_api.hip) and the gfx950 kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moek {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- bf16 helpers (raw 16-bit patterns, finite values) --------------------
__device__ __forceinline__ float bf16_lo(unsigned int v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int v) { return __uint_as_float(v & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest, ties to even
__device__ __forceinline__ unsigned int f32_to_bf16(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// gfx950's v_cvt_pk_bf16_f32 (same result as f32_to_bf16 on finite values)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2_t));
}
// Raw buffer descriptor (stride 0) over bytes [base, base + bytes): loads
// through it take a 32-bit byte offset and read zeros past the end.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// base and bytes must be wavefront-uniform; they are passed through
// readfirstlane so that the descriptor lives in scalar registers (a
// descriptor the compiler takes for divergent costs a loop per load).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  // word 3: 32-bit data format, the value the gfx9 family takes for raw
  // (stride 0) buffers
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}
__device__ __forceinline__ void unpack8(u32x4 v, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = bf16_lo(v[i]);
    o[2 * i + 1] = bf16_hi(v[i]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return r;
}

// ---- routing of one token ---------------------------------------------------
// The token's E logits row[0..E) are spread over L lanes (li = lane within
// the group), V per lane.  Softmax with temperature (inv_tau), then k rounds
// of arg-max by (logit descending, index ascending); lane li == 0 writes
// idx_t[j] and the raw probability w_t[j].  Lanes past E hold nothing, so
// the butterfly trees combine the same values in the same order for any L.
// Value of lane (li - N) mod 16 of this lane's row of 16 lanes (DPP row
// rotation: a VALU operand modifier, no LDS round trip).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ int row_ror(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x120 + N, 0xF, 0xF, false);
}

// L = 16: a token's lanes are one DPP row, so the reductions rotate within
// the row.  After rotations by 8, 4, 2, 1 every lane holds the same sum, and
// the same one as the xor butterfly gives: at each level the partial sums
// repeat with the period the xor partner and the rotation partner share.
// Each arg-max round is a max over the row, then the least index among the
// lanes holding it (a min over the row).
template <int V>
__device__ __forceinline__ void route_token16(const float* row, int E, int k, float inv_tau,
                                              int li, bool tok, int32_t* idx_t, float* w_t) {
  float v[V];
  bool ok[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = li + u * 16;
    ok[u] = tok && e < E;
    v[u] = ok[u] ? row[e] : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < V; ++u) m = fmaxf(m, v[u]);
  m = fmaxf(m, row_ror<8>(m));
  m = fmaxf(m, row_ror<4>(m));
  m = fmaxf(m, row_ror<2>(m));
  m = fmaxf(m, row_ror<1>(m));
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u)
    if (ok[u]) s += expf((v[u] - m) * inv_tau);
  s += row_ror<8>(s);
  s += row_ror<4>(s);
  s += row_ror<2>(s);
  s += row_ror<1>(s);
  unsigned taken = 0u;
  for (int j = 0; j < k; ++j) {
    // the lane's best untaken logit; u ascends with the index, so a strict
    // comparison keeps the lowest index among equal values (entries past E
    // are -inf and never taken)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < V; ++u) {
      if (!((taken >> u) & 1u) && v[u] > bv) {
        bv = v[u];
        bi = li + u * 16;
      }
    }
    float mv = fmaxf(bv, row_ror<8>(bv));
    mv = fmaxf(mv, row_ror<4>(mv));
    mv = fmaxf(mv, row_ror<2>(mv));
    mv = fmaxf(mv, row_ror<1>(mv));
    int ci = bv == mv ? bi : 0x7fffffff;
    ci = min(ci, row_ror<8>(ci));
    ci = min(ci, row_ror<4>(ci));
    ci = min(ci, row_ror<2>(ci));
    ci = min(ci, row_ror<1>(ci));
    if (ci != 0x7fffffff && (ci & 15) == li) taken |= 1u << (ci >> 4);
    if (li == 0 && tok) {
      idx_t[j] = ci;
      w_t[j] = expf((mv - m) * inv_tau) / s;
    }
  }
}

template <int L, int V>
__device__ __forceinline__ void route_token(const float* row, int E, int k, float inv_tau,
                                            int li, bool tok, int32_t* idx_t, float* w_t) {
  if constexpr (L == 16) {
    route_token16<V>(row, E, k, inv_tau, li, tok, idx_t, w_t);
    return;
  }
  float v[V];
  bool ok[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = li + u * L;
    ok[u] = tok && e < E;
    v[u] = ok[u] ? row[e] : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < V; ++u)
    if (ok[u]) m = fmaxf(m, v[u]);
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, L));
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u)
    if (ok[u]) s += expf((v[u] - m) * inv_tau);
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, L);
  unsigned taken = 0u;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int e = li + u * L;
      if (ok[u] && !((taken >> u) & 1u) && (v[u] > bv || (v[u] == bv && e < bi))) {
        bv = v[u];
        bi = e;
      }
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, L);
      const int oi = __shfl_xor(bi, off, L);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi != 0x7fffffff && bi % L == li) taken |= 1u << (bi / L);
    if (li == 0 && tok) {
      idx_t[j] = bi;
      w_t[j] = expf((bv - m) * inv_tau) / s;
    }
  }
}

// ---- launchers --------------------------------------------------------------
// wsplit: device scratch of gate_copy_bytes(...) for a copy of the router
// weights in the gate lanes' order (bf16 x only: the split copy of bf16
// parts, or the blocked fp32 copy, whichever gate_use_split /
// gate_use_block picks), or null to load Wg directly; all give
// bit-identical logits.
// Events e0 / e1 (optional, on these launchers and the FFN's): recorded from
// the start of the first kernel dispatch and the end of the last
// (hipExtLaunchKernelGGL), so timing them adds no marker packets.
hipError_t launch_gate(const void* x, bool x_bf16, const float* Wg, const float* bias,
                       float* logits, int64_t B, int d, int E, void* wsplit, hipStream_t s,
                       hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
size_t gate_split_bytes(int d, int E);
size_t gate_block_bytes(int d, int E);
bool gate_use_split(bool x_bf16, int64_t B, int d, int E);
bool gate_use_block(bool x_bf16, int64_t B, int d, int E);
// bytes of the weight copy the forward uses at this shape (0: none)
size_t gate_copy_bytes(bool x_bf16, int64_t B, int d, int E);
// host-only: exclusive end of the bytes the gate launch reads from the
// weight copy the forward would use at (B, d, E), bf16 x (a self-check of
// the launch plan)
int64_t gate_split_read_end(int64_t B, int d, int E);

hipError_t launch_route(const float* logits, int64_t B, int E, int k, float tau,
                        int32_t* idx, float* w, hipStream_t s, hipEvent_t e0 = nullptr,
                        hipEvent_t e1 = nullptr);

// slot assignment: tile geometry shared by the three kernels
struct SlotPlan {
  int64_t BK;      // B*k assignments
  int tile;        // assignments per tile (multiple of 256)
  int n_tiles;
};
SlotPlan slot_plan(int64_t B, int k);
size_t slot_ws_bytes(int64_t B, int k, int E);

// unavail: optional [E] device mask; a nonzero entry gives that expert
// capacity 0 (every assignment to it is dropped).  cap_in: optional [E]
// device capacities used instead of C and the mask.
hipError_t launch_slots(const int32_t* idx, int64_t B, int k, int E, int C,
                        const uint8_t* unavail, int D,
                        int32_t* pos, uint8_t* keep, int32_t* dest, int32_t* expert_load,
                        int32_t* expert_count, int32_t* expert_offset, int32_t* rank_offset,
                        int32_t* pack_src, int32_t* ws_hist, hipStream_t s,
                        const int32_t* cap_in = nullptr);

// Overflow redirected to the next-best expert (one fallback round).
//   split: idx [B][k] = ranked [B][K2] columns 0..k-1
//   fallback: the m-th dropped choice of a token -> its rank k + m (fb = -1
//     past K2), rk = that rank; rem[e] = capacity - kept in round 1
//   merge_offsets (one block): count = count1 + count2, offsets, rank offsets
//   merge: final expert / weight / slot / keep / dest / pack_src per
//     assignment from both rounds
hipError_t launch_split_ranked(const int32_t* ranked, int64_t B, int K2, int k, int32_t* idx,
                               hipStream_t s);
hipError_t launch_fallback(const int32_t* ranked, const uint8_t* keep1, const int32_t* count1,
                           int64_t B, int K2, int k, int E, int C, const uint8_t* unavail,
                           int32_t* fb, int32_t* rk, int32_t* rem, hipStream_t s);
hipError_t launch_merge_offsets(const int32_t* count1, const int32_t* count2, int E, int D,
                                int32_t* count, int32_t* expert_offset, int32_t* rank_offset,
                                hipStream_t s);
hipError_t launch_merge(const float* ranked_w, int64_t B, int K2, int k, const uint8_t* keep1,
                        const int32_t* pos1, const int32_t* fb, const int32_t* rk,
                        const uint8_t* keep2, const int32_t* pos2, const int32_t* count1,
                        const int32_t* expert_offset, int32_t* idx, float* w, int32_t* pos,
                        uint8_t* keep, int32_t* dest, int32_t* pack_src, hipStream_t s);

// expert-choice routing (choice.hip): router probabilities transposed
// [E][B]; every expert's top-Ce tokens (sel_t [E][B]: packed row or -1;
// rows e*Ce.. in token order, pack_src / pack_w per row; expert_offset
// e*Ce); the gather pack; the combine over the experts that chose a token
hipError_t launch_router_probs(const float* logits, int64_t B, int E, float tau, float* probs_t,
                               hipStream_t s);
hipError_t launch_expert_choice(const float* probs_t, int64_t B, int E, int Ce, int32_t* sel_t,
                                int32_t* expert_offset, int32_t* pack_src, float* pack_w,
                                hipStream_t s);
hipError_t launch_ec_pack(const void* x, bool x_bf16, const int32_t* pack_src, int64_t rows,
                          int d, uint16_t* packed, hipStream_t s);
hipError_t launch_ec_combine(const uint16_t* ret, const int32_t* sel_t, const float* pack_w,
                             const void* x_res, bool x_bf16, void* y, int64_t B, int E, int d,
                             hipStream_t s);

// routing-health signals (health.hip): workspace bytes and the two launches
size_t stats_ws_bytes(int64_t B, int E);
hipError_t launch_routing_stats(const float* logits, int64_t B, int E, int k, int C, float tau,
                                const int32_t* load, const int32_t* count, float* prob_mean,
                                float* token_frac, float* utilization, int32_t* dropped,
                                double* summary, void* ws, hipStream_t s);

// skip_eo (optional): packed rows [skip_eo[skip_b], skip_eo[skip_e]) are
// not written (the forward's first GEMM gathers those rows from x itself)
hipError_t launch_pack(const void* x, bool x_bf16, const int32_t* dest, int64_t B, int k,
                       int d, uint16_t* packed, hipStream_t s, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr, const int32_t* skip_eo = nullptr, int skip_b = 0,
                       int skip_e = 0);

// shared (optional): a shared expert's output rows [B][d] bf16, added with
// weight 1
hipError_t launch_combine(const uint16_t* ret, const int32_t* dest, const float* w,
                          const void* x_res, bool x_bf16, void* y, int64_t B, int k, int d,
                          int64_t kmax, hipStream_t s, const uint16_t* shared = nullptr,
                          hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// The shared expert: one expert over every token's row of x (bf16) -- the
// grouped GEMM with expert_offset = {0, B} (written into eo, 2 int32 of
// device scratch), hidden activations in H [B][f].
hipError_t launch_shared_ffn(const uint16_t* x, int64_t B, int d, int f, bool swiglu,
                             const void* wp, uint16_t* H, int32_t* eo, uint16_t* out,
                             hipStream_t s, hipEvent_t ev_stop = nullptr,
                             uint16_t* zsave = nullptr);

hipError_t launch_unpack(const uint16_t* ret, const int32_t* dest, int64_t B, int k, int d,
                         int64_t kmax, uint16_t* out, hipStream_t s);

// rows of [0, expert_offset[E]) outside [expert_offset[e_begin], expert_offset[e_end])
hipError_t launch_copy_remote(const uint16_t* src, uint16_t* dst, const int32_t* expert_offset,
                              int E, int e_begin, int e_end, int64_t kmax, int d,
                              hipStream_t s);

// grouped expert MLP: H = act(X W1^T [, X W3^T]) then Out = H W2^T, with the
// weights in the blocked layout written by launch_pack_weights
size_t packed_weights_bytes(int n_local, int d, int f, bool swiglu);
hipError_t launch_pack_weights(const uint16_t* W1, const uint16_t* W3, const uint16_t* W2,
                               int n_local, int d, int f, bool swiglu, void* wp, hipStream_t s);
// rows_hint: expected rows per local expert (chooses the tile schedule only)
// ev_start / ev_stop (optional): taken by the first launch's start and the
// last launch's end, ev_mid_end / ev_mid_start by the first launch's end and
// the second's start (HIP fills them from the dispatches' own timestamps,
// no marker packets); recorded as plain markers if nothing is launched.
// gidx (optional): the first GEMM reads its rows from gx ([gx_rows][d]
// bf16, 2 gx_rows d < 2^32) through the index -- packed row r is gx row
// gidx[r] -- instead of from packed.
hipError_t launch_expert_ffn(const uint16_t* packed, const int32_t* expert_offset, int e_begin,
                             int n_local, int rows_max, int rows_hint, int d, int f, bool swiglu,
                             const void* wp, uint16_t* H, uint16_t* ret, hipStream_t s,
                             hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                             hipEvent_t ev_mid_end = nullptr, hipEvent_t ev_mid_start = nullptr,
                             const uint16_t* gx = nullptr, const int32_t* gidx = nullptr,
                             int64_t gx_rows = 0, uint16_t* zsave = nullptr);

// ---- backward pass (backward.hip, wgrad.hip, expert_gemm.hip) -------------
hipError_t launch_combine_bwd(const void* dy, bool x_bf16, const uint16_t* ret,
                              const int32_t* dest, const float* w, int64_t B, int k, int d,
                              int64_t kmax, uint16_t* dret, float* dw, hipStream_t s);
// load: expert_load [E] (read when aux_coef != 0)
hipError_t launch_route_bwd(const float* logits, const int32_t* idx, const float* dw,
                            const int32_t* load, float aux_coef, int64_t B, int E, int k,
                            float tau, float* dl, hipStream_t s);
hipError_t launch_gather_rows(const void* x, bool x_bf16, const int32_t* pack_src,
                              const int32_t* eo, int e_begin, int e_end, int64_t B, int d,
                              int64_t rows_max, uint16_t* out, hipStream_t s);
// rows of one RB8 segment: the row capacity rounded up to 32
int64_t rb8_rows(int64_t rows);
// mode 0 copy, 1 GELU of Z, 2 SwiGLU of the interleaved Z1/Z3 columns
// rel: src rows are local (row 0 = expert_offset[e_begin]); else absolute
hipError_t launch_relayout_rb8(int mode, const uint16_t* src, int64_t src_ld, const int32_t* eo,
                               int e_begin, int rel, int n_seg, int64_t rows_cap, int W,
                               int src_w, int one_col, uint16_t* out, hipStream_t s,
                               const int32_t* ridx = nullptr, int64_t src_rows = 0);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
// shared expert backward: pack_src[t] = t, expert_offset {0, B}, dret = dy
// (bf16 [B][d]); and acc += v (fp32 += bf16, n a multiple of 8)
hipError_t launch_shared_bwd_prep(int32_t* pack_src, int32_t* eo, const uint16_t* dy,
                                  uint16_t* dret, int64_t B, int d, hipStream_t s);
hipError_t launch_add_bf16(float* acc, const uint16_t* v, int64_t n, hipStream_t s);
// out0[m][n] (m < M0) / out1[n] (m == M0) = sum over g of part[g][m][n], in g
// order; part is [G][M0 + 1][N]
hipError_t launch_sum_parts(const float* part, int G, int M0, int N, float* out0, float* out1,
                            hipStream_t s);
hipError_t launch_split_rows(const float* src, int64_t rows, int cols, int Wp, uint16_t* o0,
                             uint16_t* o1, uint16_t* o2, hipStream_t s);
// RB8 of an fp32 matrix split into bf16 parts: element (r, c) = src[r ld + c]
// (trans: src[c ld + r]) for r < rows, c < cols; rows padded to 32 with zeros
hipError_t launch_split_rb8(const float* src, int64_t rows, int cols, int64_t ld, bool trans,
                            int Wp, int one_col, uint16_t* o0, uint16_t* o1, uint16_t* o2,
                            hipStream_t s);
hipError_t launch_unpack_sum(const uint16_t* dxp, const int32_t* dest, const void* dy,
                             bool x_bf16, bool residual, int64_t B, int k, int d, int64_t kmax,
                             float* dx_acc, hipStream_t s);

// Grouped K-fragment GEMM (wgrad.hip): C_g = sum over segments of A B^T with
// both operands in the RB8 layout (a_w / b_w columns).  Groups: K from
// expert_offset (eo, e_begin) or K.
struct KGemm {
  const uint16_t* A[6];
  const uint16_t* B[6];
  int nseg;
  int a_w, b_w;
  int64_t a_es, b_es;        // per-group element offsets
  int64_t a_bytes, b_bytes;  // bytes of each segment's operand (reads past: zeros)
  const int32_t* eo;
  int e_begin;
  int K;
  int Ktot;  // > 0 (eo null): split-K, group g takes rows g K .. min((g+1) K, Ktot)
  int groups, M, N;
  int mode;  // 0: fp32 into C0 (m < M0, n < N0) or C1 at (m - r1, n - col1);
             // 1: acc + add stored to xo (bf16 or fp32), rows M0, cols N0, stride ldc0
  float* C0;
  int64_t ldc0, c0_es;
  int M0, N0;
  float* C1;
  int64_t ldc1, c1_es;
  int r1, col1, M1, N1;
  const float* add;
  int64_t ld_add;
  void* xo;
  int x_bf16;
};
hipError_t launch_kgemm(const KGemm& q, hipStream_t s);

// Expert FFN backward pieces on the forward's grouped GEMM:
//   recompute:  Z = X_loc W1 (no activation; SwiGLU: W1 and W3 products in
//               the GEMM1 tile order, zw = expert_ffn_zw columns)
//   dact:       dZ = dact(dret W2^T, Z) ([dZ1 | dZ3] for SwiGLU), local rows
//   dgrad:      dXp = dZ [W1 | W3]^T, written over the local rows of dret
// wpb: the blocked backward weights (launch_pack_weights_bwd).
int expert_ffn_zw(int f, bool swiglu);
size_t packed_weights_bwd_bytes(int n_local, int d, int f, bool swiglu);
hipError_t launch_pack_weights_bwd(const uint16_t* W1, const uint16_t* W3, const uint16_t* W2,
                                   int n_local, int d, int f, bool swiglu, void* wpb,
                                   hipStream_t s);
hipError_t launch_ffn_recompute(const uint16_t* xloc, const int32_t* expert_offset, int e_begin,
                                int n_local, int rows_max, int rows_hint, int d, int f,
                                bool swiglu, const void* wp, uint16_t* Z, hipStream_t s);
hipError_t launch_ffn_dact(const uint16_t* dret, const int32_t* expert_offset, int e_begin,
                           int n_local, int rows_max, int rows_hint, int d, int f, bool swiglu,
                           const void* wpb, const uint16_t* Z, uint16_t* dZ, hipStream_t s);
hipError_t launch_ffn_dgrad(const uint16_t* dZ, const int32_t* expert_offset, int e_begin,
                            int n_local, int rows_max, int rows_hint, int d, int f, bool swiglu,
                            const void* wpb, uint16_t* dxp, hipStream_t s);

}  // namespace moek
