// C ABI of the MoE layer forward: host-side checks, capacity, workspace
// layout and the launch order of the kernels.  Declared in include/moe.h.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "moe.h"
#include "moe_check.h"
#include "moe_kernels.h"

namespace {

constexpr int32_t kMaxE = 1024;
constexpr int32_t kMaxK = 16;
constexpr int32_t kMaxDim = 1 << 16;
// tokens: the router launch has up to 64 lanes per token in one grid
// dimension, which holds fewer than 2^32 work-items
constexpr int64_t kMaxB = (int64_t)1 << 25;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool a4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int32_t capacity_of(const moe_problem_t* p) {
  if (p->C >= 0) return p->C;
  return moe_capacity(p->B, p->k, p->E, p->c);
}

// rows one expert can hold: min(C, B) (a token picks an expert at most once)
int64_t rows_per_expert(const moe_problem_t* p) {
  const int64_t C = capacity_of(p);
  return C < p->B ? C : p->B;
}

// expected rows per expert with even routing, B k / E, at most the row cap
int rows_hint(const moe_problem_t* p) {
  const int64_t even = ((int64_t)p->B * p->k + p->E - 1) / p->E;
  const int64_t cap = rows_per_expert(p);
  return (int)(even < cap ? even : cap);
}

int64_t kmax_of(const moe_problem_t* p) {
  const int64_t bk = p->B * p->k;
  const int64_t ec = (int64_t)p->E * rows_per_expert(p);
  return bk < ec ? bk : ec;
}

int64_t kloc_of(const moe_problem_t* p) {
  const int64_t bk = p->B * p->k;
  const int64_t ec = (int64_t)(p->e_end - p->e_begin) * rows_per_expert(p);
  return bk < ec ? bk : ec;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

size_t ffn_ws(const moe_problem_t* p) { return align_up((size_t)kloc_of(p) * p->f * 2); }
// rows of an expert-choice layout: E * min(C, B)
int64_t ec_rows(const moe_problem_t* p) {
  const int64_t C = capacity_of(p);
  return (int64_t)p->E * (C < p->B ? C : p->B);
}

struct EcBufs {
  float* logits;
  float* probs_t;
  int32_t* sel_t;
  int32_t* eo;
  int32_t* pack_src;
  float* pack_w;
  uint16_t* packed;
  uint16_t* H;
  void* wsplit;
};

// workspace of moe_forward_expert_choice: fields the caller did not supply,
// H [R][f], the router's split weight copy when the gate uses one
size_t carve_ec(const moe_problem_t* p, const moe_expert_choice_out_t* o, void* ws, EcBufs* b);

// scratch of a shared expert (moe_shared_ffn): expert_offset {0, B} in one
// aligned slot, then H [B][f] bf16
size_t shared_ws(const moe_problem_t* ps) {
  return align_up(2 * sizeof(int32_t)) + align_up((size_t)ps->B * ps->f * 2);
}
size_t dispatch_ws(const moe_problem_t* p) {
  return align_up(moek::slot_ws_bytes(p->B, p->k, p->E));
}

// Workspace carving for moe_forward: fields the caller did not supply.
struct Carve {
  size_t off = 0;
  char* base = nullptr;
  template <typename T>
  T* take(T* given, size_t bytes) {
    if (given) return given;
    T* r = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(bytes);
    return r;
  }
};

struct FwdBufs {
  float* logits;
  int32_t* idx;
  float* w;
  int32_t *pos, *dest;
  uint8_t* keep;
  int32_t *load, *count, *eo, *ro, *pack_src;
  uint16_t* packed;
  int32_t* hist;
  uint16_t* H;
  void* wsplit;  // split copy of the router weights, or null
  // overflow redirected (MOE_OVERFLOW_NEXT): ranked choices and both rounds
  int32_t* ranked;
  float* ranked_w;
  int32_t *pos1, *count1, *fb, *rk, *rem, *pos2, *load2, *count2, *eo2, *ro2, *dest2, *ps2;
  uint8_t *keep1, *keep2;
};

size_t carve_forward(const moe_problem_t* p, const moe_forward_out_t* o, void* ws, FwdBufs* b) {
  moe_forward_out_t none;
  std::memset(&none, 0, sizeof(none));
  if (!o) o = &none;
  Carve c;
  c.base = static_cast<char*>(ws);
  const size_t BE = (size_t)p->B * p->E, BKn = (size_t)p->B * p->k;
  const size_t km = (size_t)kmax_of(p);
  FwdBufs t;
  t.logits = c.take(o->logits, BE * 4);
  t.idx = c.take(o->topk_idx, BKn * 4);
  t.w = c.take(o->topk_w, BKn * 4);
  t.pos = c.take(o->pos, BKn * 4);
  t.keep = c.take(o->keep, BKn);
  t.dest = c.take(o->dest, BKn * 4);
  t.load = c.take(o->expert_load, (size_t)p->E * 4);
  t.count = c.take(o->expert_count, (size_t)p->E * 4);
  t.eo = c.take(o->expert_offset, (size_t)(p->E + 1) * 4);
  t.ro = c.take(o->rank_offset, (size_t)(p->n_ranks + 1) * 4);
  t.pack_src = c.take(o->pack_src, km * 4);
  t.packed = c.take(reinterpret_cast<uint16_t*>(o->packed), km * p->d * 2);
  t.hist = c.take<int32_t>(nullptr, dispatch_ws(p));
  t.H = c.take<uint16_t>(nullptr, ffn_ws(p));
  t.wsplit = moek::gate_copy_bytes(p->x_dtype == MOE_BF16, p->B, p->d, p->E) > 0
                 ? c.take<char>(nullptr, moek::gate_copy_bytes(p->x_dtype == MOE_BF16, p->B,
                                                               p->d, p->E))
                 : nullptr;
  if (p->overflow == MOE_OVERFLOW_NEXT) {
    const size_t K2 = (size_t)(2 * p->k < p->E ? 2 * p->k : p->E);
    t.ranked = c.take<int32_t>(nullptr, (size_t)p->B * K2 * 4);
    t.ranked_w = c.take<float>(nullptr, (size_t)p->B * K2 * 4);
    t.pos1 = c.take<int32_t>(nullptr, BKn * 4);
    t.keep1 = c.take<uint8_t>(nullptr, BKn);
    t.count1 = c.take<int32_t>(nullptr, (size_t)p->E * 4);
    t.fb = c.take<int32_t>(nullptr, BKn * 4);
    t.rk = c.take<int32_t>(nullptr, BKn * 4);
    t.rem = c.take<int32_t>(nullptr, (size_t)p->E * 4);
    t.pos2 = c.take<int32_t>(nullptr, BKn * 4);
    t.keep2 = c.take<uint8_t>(nullptr, BKn);
    t.load2 = c.take<int32_t>(nullptr, (size_t)p->E * 4);
    t.count2 = c.take<int32_t>(nullptr, (size_t)p->E * 4);
    t.eo2 = c.take<int32_t>(nullptr, (size_t)(p->E + 1) * 4);
    t.ro2 = c.take<int32_t>(nullptr, (size_t)(p->n_ranks + 1) * 4);
    t.dest2 = c.take<int32_t>(nullptr, BKn * 4);
    t.ps2 = c.take<int32_t>(nullptr, km * 4);
  }
  if (b) *b = t;
  return c.off;
}

size_t carve_ec(const moe_problem_t* p, const moe_expert_choice_out_t* o, void* ws, EcBufs* b) {
  moe_expert_choice_out_t none;
  std::memset(&none, 0, sizeof(none));
  if (!o) o = &none;
  Carve c;
  c.base = static_cast<char*>(ws);
  const size_t BE = (size_t)p->B * p->E, R = (size_t)ec_rows(p);
  EcBufs t;
  t.logits = c.take(o->logits, BE * 4);
  t.probs_t = c.take(o->probs_t, BE * 4);
  t.sel_t = c.take(o->sel_t, BE * 4);
  t.eo = c.take(o->expert_offset, (size_t)(p->E + 1) * 4);
  t.pack_src = c.take(o->pack_src, R * 4);
  t.pack_w = c.take(o->pack_w, R * 4);
  t.packed = c.take(reinterpret_cast<uint16_t*>(o->packed), R * p->d * 2);
  t.H = c.take<uint16_t>(nullptr, R * p->f * 2);
  t.wsplit = moek::gate_copy_bytes(p->x_dtype == MOE_BF16, p->B, p->d, p->E) > 0
                 ? c.take<char>(nullptr, moek::gate_copy_bytes(p->x_dtype == MOE_BF16, p->B,
                                                               p->d, p->E))
                 : nullptr;
  if (b) *b = t;
  return c.off;
}

// ---- backward workspaces -------------------------------------------------
struct FfnBwdBufs {
  uint16_t *xloc, *Z, *dZ, *X8, *H8, *dret8, *dZ8;
};
// expert FFN backward: the local rows' inputs, recomputed pre-activations,
// dZ, and the RB8 operands of the weight-gradient GEMMs
size_t carve_ffn_bwd(const moe_problem_t* p, void* ws, FfnBwdBufs* b) {
  Carve c;
  c.base = static_cast<char*>(ws);
  const bool sw = p->act == MOE_SWIGLU;
  const size_t kl = (size_t)kloc_of(p);
  const size_t nl = (size_t)(p->e_end - p->e_begin);
  const size_t r8 = (size_t)moek::rb8_rows(rows_per_expert(p));
  const size_t zw = (size_t)moek::expert_ffn_zw(p->f, sw);
  const size_t zwd = sw ? 2 * (size_t)p->f : (size_t)p->f;
  FfnBwdBufs t;
  t.xloc = c.take<uint16_t>(nullptr, kl * p->d * 2);
  t.Z = c.take<uint16_t>(nullptr, kl * zw * 2);
  t.dZ = c.take<uint16_t>(nullptr, kl * zwd * 2);
  t.X8 = c.take<uint16_t>(nullptr, nl * r8 * p->d * 2);
  t.H8 = c.take<uint16_t>(nullptr, nl * r8 * p->f * 2);
  t.dret8 = c.take<uint16_t>(nullptr, nl * r8 * p->d * 2);
  t.dZ8 = c.take<uint16_t>(nullptr, nl * r8 * zwd * 2);
  if (b) *b = t;
  return c.off;
}

struct GateBwdBufs {
  uint16_t *dlt[2], *wgt[2], *x8[3], *dl8[3];
  float* part;
};
int pad32(int v) { return (v + 31) / 32 * 32; }
// split-K of the token contraction of dWg: enough workgroups to fill the
// CUs, at least 1024 tokens per split
struct GateSplit {
  int G, Ks;
};
GateSplit gate_split(const moe_problem_t* p) {
  const int64_t Br = moek::rb8_rows(p->B);
  if (Br == 0) return GateSplit{1, 32};
  // as many groups as one round of workgroups over the 256 CUs holds (the
  // weight-gradient GEMM's tiles are 256 x 256; a second round for a few
  // tiles would double the time)
  const int64_t tiles = (int64_t)((p->d + 1 + 255) / 256) * ((p->E + 255) / 256);
  int64_t G = 256 / tiles;
  const int64_t gmax = (Br + 1023) / 1024;
  if (G > gmax) G = gmax;
  if (G < 1) G = 1;
  if (G > 64) G = 64;
  // each group's slice of x in RB8 stays under 1 GB (32-bit offsets)
  const int64_t gmin = (Br * (int64_t)(p->d + 8) * 2 + (1LL << 30) - 1) >> 30;
  if (G < gmin) G = gmin;
  int64_t Ks = (Br + G - 1) / G;
  Ks = (Ks + 31) / 32 * 32;
  G = (Br + Ks - 1) / Ks;
  GateSplit s;
  s.G = (int)G;
  s.Ks = (int)Ks;
  return s;
}
// gate backward: the split router operands (row-major for dx, RB8 over the
// tokens for dWg and the bias) and x in RB8 with a ones column
size_t carve_gate_bwd(const moe_problem_t* p, void* ws, GateBwdBufs* b) {
  Carve c;
  c.base = static_cast<char*>(ws);
  const size_t B = (size_t)p->B, Ep = (size_t)pad32(p->E), d = (size_t)p->d;
  const size_t Br = (size_t)moek::rb8_rows(p->B);
  const int nx = p->x_dtype == MOE_BF16 ? 1 : 3;
  GateBwdBufs t{};
  // dl and Wg in RB8 over the experts (the contraction of dx = dl Wg^T)
  for (int i = 0; i < 2; ++i) t.dlt[i] = c.take<uint16_t>(nullptr, B * Ep * 2);
  for (int i = 0; i < 2; ++i) t.wgt[i] = c.take<uint16_t>(nullptr, d * Ep * 2);
  for (int i = 0; i < nx; ++i) t.x8[i] = c.take<uint16_t>(nullptr, Br * (d + 8) * 2);
  for (int i = 0; i < 3; ++i) t.dl8[i] = c.take<uint16_t>(nullptr, Br * Ep * 2);
  const GateSplit gs = gate_split(p);
  t.part = c.take<float>(nullptr, (size_t)gs.G * (d + 1) * p->E * 4);
  if (b) *b = t;
  return c.off;
}

struct BwdBufs {
  uint16_t* dret;
  float *dw, *dl, *dx_acc;
  void *ffn_ws, *gate_ws;
  size_t ffn_bytes, gate_bytes;
};
size_t carve_bwd(const moe_problem_t* p, const moe_grads_t* g, void* ws, BwdBufs* b) {
  Carve c;
  c.base = static_cast<char*>(ws);
  const size_t BK = (size_t)p->B * p->k, BE = (size_t)p->B * p->E;
  BwdBufs t;
  t.dret = c.take<uint16_t>(nullptr, (size_t)kmax_of(p) * p->d * 2);
  t.dw = c.take(g ? g->dw : nullptr, BK * 4);
  t.dl = c.take(g ? g->dlogits : nullptr, BE * 4);
  t.dx_acc = c.take<float>(nullptr, (size_t)p->B * p->d * 4);
  t.ffn_bytes = carve_ffn_bwd(p, nullptr, nullptr);
  t.ffn_ws = c.take<char>(nullptr, t.ffn_bytes);
  t.gate_bytes = carve_gate_bwd(p, nullptr, nullptr);
  t.gate_ws = c.take<char>(nullptr, t.gate_bytes);
  if (b) *b = t;
  return c.off;
}

}  // namespace

extern "C" {

int32_t moe_capacity(int64_t B, int32_t k, int32_t E, double c) {
  if (B < 0 || k < 1 || E < 1 || !(c > 0.0) || !std::isfinite(c)) return -1;
  if (B == 0) return 0;
  const double v = std::ceil(((double)(B * k) / (double)E) * c);
  if (!(v <= 2147483647.0)) return -1;
  return (int32_t)v;
}

int32_t moe_problem_capacity(const moe_problem_t* p) {
  if (moe_validate(p) != MOE_OK) return -1;
  return capacity_of(p);
}

int64_t moe_max_kept(const moe_problem_t* p) {
  if (moe_validate(p) != MOE_OK) return -1;
  return kmax_of(p);
}

moe_status_t moe_validate(const moe_problem_t* p) {
  if (!p) return MOE_ERR_INVALID;
  if (p->B < 0 || p->d < 8 || p->d % 8 || p->E < 1 || p->k < 1 || p->k > p->E)
    return MOE_ERR_INVALID;
  if (p->C < 0 && !(p->c > 0.0 && std::isfinite(p->c))) return MOE_ERR_INVALID;
  if (p->n_ranks < 1 || p->E % p->n_ranks) return MOE_ERR_INVALID;
  if (p->e_begin < 0 || p->e_end > p->E || p->e_begin > p->e_end) return MOE_ERR_INVALID;
  if (p->f < 8 || p->f % 8) return MOE_ERR_INVALID;
  if (p->act != MOE_GELU && p->act != MOE_SWIGLU) return MOE_ERR_INVALID;
  if (p->x_dtype != MOE_F32 && p->x_dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (!(p->tau > 0.0f) || !std::isfinite(p->tau)) return MOE_ERR_INVALID;
  if (p->add_residual != 0 && p->add_residual != 1) return MOE_ERR_INVALID;
  if (p->overflow != MOE_OVERFLOW_DROP && p->overflow != MOE_OVERFLOW_NEXT)
    return MOE_ERR_INVALID;
  if (p->overflow == MOE_OVERFLOW_NEXT && (2 * p->k < p->E ? 2 * p->k : p->E) > kMaxK)
    return MOE_ERR_UNSUPPORTED;
  if (p->E > kMaxE || p->k > kMaxK || p->d > kMaxDim || p->f > kMaxDim)
    return MOE_ERR_UNSUPPORTED;
  if (p->B > kMaxB || p->B > (int64_t)INT32_MAX / p->k) return MOE_ERR_UNSUPPORTED;
  if (p->C < 0 && moe_capacity(p->B, p->k, p->E, p->c) < 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_problem_t* p, moe_op_t op) {
  if (moe_validate(p) != MOE_OK) return SIZE_MAX;
  switch (op) {
    case MOE_OP_DISPATCH:
      return dispatch_ws(p);
    case MOE_OP_FFN:
      return ffn_ws(p);
    case MOE_OP_FORWARD:
      return carve_forward(p, nullptr, nullptr, nullptr);
    case MOE_OP_ROUTING_STATS:
      return moek::stats_ws_bytes(p->B, p->E);
    case MOE_OP_SHARED_FFN:
      return shared_ws(p);
    case MOE_OP_FORWARD_EXPERT_CHOICE:
      return carve_ec(p, nullptr, nullptr, nullptr);
    case MOE_OP_EXPERT_FFN_BACKWARD:
      return carve_ffn_bwd(p, nullptr, nullptr);
    case MOE_OP_GATE_BACKWARD:
      return carve_gate_bwd(p, nullptr, nullptr);
    case MOE_OP_BACKWARD:
      return carve_bwd(p, nullptr, nullptr, nullptr);
  }
  return SIZE_MAX;
}

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK:
      return "ok";
    case MOE_ERR_INVALID:
      return "invalid argument";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported size";
    case MOE_ERR_WORKSPACE:
      return "workspace too small";
    case MOE_ERR_HIP:
      return "HIP runtime error";
  }
  return "unknown status";
}

moe_status_t moe_gate(const moe_problem_t* p, const void* x, const float* Wg, const float* bias,
                      float* logits, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!x || !Wg || !logits)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(x) || !a4(Wg) || !a4(logits) || (bias && !a4(bias))))
    return MOE_ERR_INVALID;
  return hip_status(moek::launch_gate(x, p->x_dtype == MOE_BF16, Wg, bias, logits, p->B, p->d,
                                      p->E, nullptr, stream));
}

moe_status_t moe_routing_stats(const moe_problem_t* p, const float* logits,
                               const int32_t* expert_load, const int32_t* expert_count,
                               const moe_routing_stats_t* out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!out || !expert_load || !expert_count) return MOE_ERR_INVALID;
  if (p->B > 0 && (!logits || !a4(logits))) return MOE_ERR_INVALID;
  if (!a4(expert_load) || !a4(expert_count) || !a4(out->prob_mean) || !a4(out->token_frac) ||
      !a4(out->utilization) || !a4(out->dropped) ||
      (reinterpret_cast<uintptr_t>(out->summary) & 7u) != 0)
    return MOE_ERR_INVALID;
  const size_t need = moek::stats_ws_bytes(p->B, p->E);
  if (need > 0 && (!ws || ws_bytes < need || !a4(ws))) return MOE_ERR_WORKSPACE;
  return hip_status(moek::launch_routing_stats(
      logits, p->B, p->E, p->k, capacity_of(p), p->tau, expert_load, expert_count,
      out->prob_mean, out->token_frac, out->utilization, out->dropped, out->summary, ws, stream));
}

moe_status_t moe_route(const moe_problem_t* p, const float* logits, int32_t* topk_idx,
                       float* topk_w, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!logits || !topk_idx || !topk_w)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a4(logits) || !a4(topk_idx) || !a4(topk_w))) return MOE_ERR_INVALID;
  return hip_status(moek::launch_route(logits, p->B, p->E, p->k, p->tau, topk_idx, topk_w, stream));
}

moe_status_t moe_dispatch(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                          int32_t* pos, uint8_t* keep, int32_t* dest, int32_t* expert_load,
                          int32_t* expert_count, int32_t* expert_offset, int32_t* rank_offset,
                          int32_t* pack_src, moe_bf16_t* packed, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->overflow != MOE_OVERFLOW_DROP) return MOE_ERR_UNSUPPORTED;  // needs ranked choices
  if (!expert_count || !expert_offset || !rank_offset) return MOE_ERR_INVALID;
  if (p->B > 0 && (!x || !topk_idx || !pos || !keep || !dest || !pack_src || !packed))
    return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(x) || !a16(packed))) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < dispatch_ws(p)) return MOE_ERR_WORKSPACE;
  const int C = capacity_of(p);
  hipError_t e = moek::launch_slots(topk_idx, p->B, p->k, p->E, C, p->expert_unavailable,
                                    p->n_ranks, pos, keep, dest,
                                    expert_load, expert_count, expert_offset, rank_offset,
                                    pack_src, static_cast<int32_t*>(ws), stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(
      moek::launch_pack(x, p->x_dtype == MOE_BF16, dest, p->B, p->k, p->d, packed, stream));
}

size_t moe_weights_bytes(const moe_problem_t* p) {
  if (moe_validate(p) != MOE_OK) return SIZE_MAX;
  return moek::packed_weights_bytes(p->e_end - p->e_begin, p->d, p->f, p->act == MOE_SWIGLU);
}

moe_status_t moe_pack_weights(const moe_problem_t* p, const moe_bf16_t* W1, const moe_bf16_t* W3,
                              const moe_bf16_t* W2, void* wpacked, size_t wpacked_bytes,
                              hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool swiglu = p->act == MOE_SWIGLU;
  const int n_local = p->e_end - p->e_begin;
  if (n_local == 0) return MOE_OK;
  if (!W1 || !W2 || (swiglu && !W3) || !wpacked) return MOE_ERR_INVALID;
  if (!a16(W1) || !a16(W2) || (swiglu && !a16(W3)) || !a16(wpacked)) return MOE_ERR_INVALID;
  if (wpacked_bytes < moek::packed_weights_bytes(n_local, p->d, p->f, swiglu))
    return MOE_ERR_WORKSPACE;
  return hip_status(moek::launch_pack_weights(W1, swiglu ? W3 : nullptr, W2, n_local, p->d, p->f,
                                              swiglu, wpacked, stream));
}

moe_status_t moe_expert_ffn(const moe_problem_t* p, const moe_bf16_t* packed,
                            const int32_t* expert_offset, const void* wpacked, moe_bf16_t* ret,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool swiglu = p->act == MOE_SWIGLU;
  const int n_local = p->e_end - p->e_begin;
  if (!expert_offset || (p->B > 0 && (!packed || !ret))) return MOE_ERR_INVALID;
  if (n_local > 0 && !wpacked) return MOE_ERR_INVALID;
  if ((packed && !a16(packed)) || (ret && !a16(ret)) || (wpacked && !a16(wpacked)))
    return MOE_ERR_INVALID;
  const size_t need = ffn_ws(p);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (p->B == 0) return MOE_OK;
  if (ret != packed) {
    hipError_t e = moek::launch_copy_remote(packed, ret, expert_offset, p->E, p->e_begin,
                                            p->e_end, kmax_of(p), p->d, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(moek::launch_expert_ffn(packed, expert_offset, p->e_begin, n_local,
                                            (int)rows_per_expert(p), rows_hint(p), p->d, p->f,
                                            swiglu, wpacked,
                                            static_cast<uint16_t*>(ws), ret, stream));
}

moe_status_t moe_combine(const moe_problem_t* p, const moe_bf16_t* ret, const int32_t* dest,
                         const float* topk_w, const void* x_residual, void* y,
                         hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!ret || !dest || !topk_w || !y)) return MOE_ERR_INVALID;
  if (p->B > 0 && p->add_residual && !x_residual) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(ret) || !a16(y) || (p->add_residual && !a16(x_residual))))
    return MOE_ERR_INVALID;
  return hip_status(moek::launch_combine(ret, dest, topk_w, p->add_residual ? x_residual : nullptr,
                                         p->x_dtype == MOE_BF16, y, p->B, p->k, p->d,
                                         kmax_of(p), stream));
}

moe_status_t moe_unpack(const moe_problem_t* p, const moe_bf16_t* ret, const int32_t* dest,
                        moe_bf16_t* out, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!ret || !dest || !out)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(ret) || !a16(out))) return MOE_ERR_INVALID;
  return hip_status(moek::launch_unpack(ret, dest, p->B, p->k, p->d, kmax_of(p), out, stream));
}

}  // extern "C"

namespace {

// The shared expert of moe_forward_shared: its problem, packed weights and
// scratch (expert_offset {0, B}, hidden activations, output rows).
struct SharedRun {
  const moe_problem_t* ps;
  const void* wp;
  int32_t* eo;
  uint16_t* H;
  uint16_t* S;
};

moe_status_t check_shared(const moe_problem_t* ps) {
  moe_status_t st = moe_validate(ps);
  if (st != MOE_OK) return st;
  if (ps->E != 1 || ps->k != 1 || ps->e_begin != 0 || ps->e_end != 1) return MOE_ERR_INVALID;
  if (ps->x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The layer on one stream (moe_forward; with sh, moe_forward_shared).  ws
// holds the routed layer's buffers (carve_forward) only.
moe_status_t forward_chain(const moe_problem_t* p, const void* x, const float* Wg,
                           const float* bias, const void* wpacked, void* y,
                           moe_forward_out_t* out, void* ws, size_t ws_bytes, hipStream_t stream,
                           const SharedRun* sh) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool swiglu = p->act == MOE_SWIGLU;
  const int n_local = p->e_end - p->e_begin;
  if (p->B > 0 && (!x || !Wg || !y)) return MOE_ERR_INVALID;
  if (n_local > 0 && !wpacked) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(x) || !a16(y) || !a4(Wg) || (bias && !a4(bias)))) return MOE_ERR_INVALID;
  if (wpacked && !a16(wpacked)) return MOE_ERR_INVALID;
  if (out && out->packed && !a16(out->packed)) return MOE_ERR_INVALID;
  if (out && out->z && !a16(out->z)) return MOE_ERR_INVALID;
  if (out && out->z_shared && (!sh || !a16(out->z_shared))) return MOE_ERR_INVALID;
  const size_t need = carve_forward(p, out, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  FwdBufs b;
  carve_forward(p, out, ws, &b);
  const bool xb = p->x_dtype == MOE_BF16;
  const int C = capacity_of(p);
  hipError_t e = hipSuccess;
  // stage events: dispatch timestamps of the stages' own kernels (no marker
  // packets); with no tokens there are no kernels and every event is a marker
  hipEvent_t ev[MOE_STAGE_EVENTS] = {};
  if (out)
    for (int i = 0; i < MOE_STAGE_EVENTS; ++i) ev[i] = out->events[i];
  if (p->B == 0) {
    for (int i = 0; i < MOE_STAGE_EVENTS && e == hipSuccess; ++i)
      if (ev[i]) e = hipEventRecord(ev[i], stream);
    for (int i = 0; i < MOE_STAGE_EVENTS; ++i) ev[i] = nullptr;
  }
  if (e == hipSuccess)
    e = moek::launch_gate(x, xb, Wg, bias, b.logits, p->B, p->d, p->E, b.wsplit, stream, ev[0],
                          ev[1]);
  const bool redirect = p->overflow == MOE_OVERFLOW_NEXT;
  const int K2 = 2 * p->k < p->E ? 2 * p->k : p->E;
  if (e == hipSuccess) {
    if (redirect)
      e = moek::launch_route(b.logits, p->B, p->E, K2, p->tau, b.ranked, b.ranked_w, stream,
                             ev[2], ev[3]);
    else
      e = moek::launch_route(b.logits, p->B, p->E, p->k, p->tau, b.idx, b.w, stream, ev[2],
                             ev[3]);
  }
  if (!redirect) {
    if (e == hipSuccess)
      e = moek::launch_slots(b.idx, p->B, p->k, p->E, C, p->expert_unavailable, p->n_ranks,
                             b.pos, b.keep, b.dest, b.load, b.count, b.eo, b.ro, b.pack_src,
                             b.hist, stream);
  } else {
    // round 1 on the top-k choices, the fallbacks of the dropped ones, round
    // 2 on the capacity left, then the merged layout (dest / pack_src of the
    // two rounds' own layouts are scratch)
    if (e == hipSuccess) e = moek::launch_split_ranked(b.ranked, p->B, K2, p->k, b.idx, stream);
    if (e == hipSuccess)
      e = moek::launch_slots(b.idx, p->B, p->k, p->E, C, p->expert_unavailable, p->n_ranks,
                             b.pos1, b.keep1, b.dest2, b.load, b.count1, b.eo2, b.ro2, b.ps2,
                             b.hist, stream);
    if (e == hipSuccess)
      e = moek::launch_fallback(b.ranked, b.keep1, b.count1, p->B, K2, p->k, p->E, C,
                                p->expert_unavailable, b.fb, b.rk, b.rem, stream);
    if (e == hipSuccess)
      e = moek::launch_slots(b.fb, p->B, p->k, p->E, C, nullptr, p->n_ranks, b.pos2, b.keep2,
                             b.dest2, b.load2, b.count2, b.eo2, b.ro2, b.ps2, b.hist, stream,
                             b.rem);
    if (e == hipSuccess)
      e = moek::launch_merge_offsets(b.count1, b.count2, p->E, p->n_ranks, b.count, b.eo, b.ro,
                                     stream);
    if (e == hipSuccess)
      e = moek::launch_merge(b.ranked_w, p->B, K2, p->k, b.keep1, b.pos1, b.fb, b.rk, b.keep2,
                             b.pos2, b.count1, b.eo, b.idx, b.w, b.pos, b.keep, b.dest,
                             b.pack_src, stream);
  }
  // bf16 tokens: the first GEMM gathers the local experts' rows from x
  // through pack_src, so the pack writes only the rows bound for the other
  // ranks (nothing at all when every expert is local); the local rows of
  // packed receive the expert outputs as before
  const bool gather =
      xb && n_local > 0 && (int64_t)p->B * p->d * 2 < ((int64_t)1 << 32);
  if (e == hipSuccess) {
    if (gather && p->e_begin == 0 && p->e_end == p->E) {
      if (ev[4]) e = hipEventRecord(ev[4], stream);
    } else {
      e = moek::launch_pack(x, xb, b.dest, p->B, p->k, p->d, b.packed, stream, nullptr, ev[4],
                            gather ? b.eo : nullptr, p->e_begin, p->e_end);
    }
  }
  // with a shared expert its GEMMs follow the routed ones inside the FFN pair
  if (p->B > 0) {
    if (e == hipSuccess)
      e = moek::launch_expert_ffn(b.packed, b.eo, p->e_begin, n_local, (int)rows_per_expert(p),
                                  rows_hint(p), p->d, p->f, swiglu, wpacked, b.H, b.packed,
                                  stream, ev[5], sh ? nullptr : ev[8], ev[6], ev[7],
                                  gather ? static_cast<const uint16_t*>(x) : nullptr,
                                  gather ? b.pack_src : nullptr, p->B, out ? out->z : nullptr);
    if (e == hipSuccess && sh)
      e = moek::launch_shared_ffn(static_cast<const uint16_t*>(x), p->B, p->d, sh->ps->f,
                                  sh->ps->act == MOE_SWIGLU, sh->wp, sh->H, sh->eo, sh->S, stream,
                                  ev[8], out ? out->z_shared : nullptr);
  }
  if (e == hipSuccess)
    e = moek::launch_combine(b.packed, b.dest, b.w, p->add_residual ? x : nullptr, xb, y, p->B,
                             p->k, p->d, kmax_of(p), stream, sh ? sh->S : nullptr, ev[9], ev[10]);
  return hip_status(e);
}

}  // namespace

extern "C" {

moe_status_t moe_forward(const moe_problem_t* p, const void* x, const float* Wg, const float* bias,
                         const void* wpacked, void* y, moe_forward_out_t* out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  return forward_chain(p, x, Wg, bias, wpacked, y, out, ws, ws_bytes, stream, nullptr);
}

moe_status_t moe_shared_ffn(const moe_problem_t* ps, const moe_bf16_t* x, const void* wpacked,
                            moe_bf16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_shared(ps);
  if (st != MOE_OK) return st;
  if (ps->B == 0) return MOE_OK;
  if (!x || !wpacked || !out || !a16(x) || !a16(wpacked) || !a16(out)) return MOE_ERR_INVALID;
  if (!ws || ws_bytes < shared_ws(ps) || !a16(ws)) return MOE_ERR_WORKSPACE;
  int32_t* eo = static_cast<int32_t*>(ws);
  uint16_t* H = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + align_up(8));
  return hip_status(moek::launch_shared_ffn(x, ps->B, ps->d, ps->f, ps->act == MOE_SWIGLU,
                                            wpacked, H, eo, out, stream));
}

moe_status_t moe_combine_shared(const moe_problem_t* p, const moe_bf16_t* ret,
                                const int32_t* dest, const float* topk_w,
                                const moe_bf16_t* shared_out, const void* x_residual, void* y,
                                hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!ret || !dest || !topk_w || !y || !shared_out)) return MOE_ERR_INVALID;
  if (p->B > 0 && p->add_residual && !x_residual) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(ret) || !a16(y) || !a16(shared_out) ||
                   (p->add_residual && !a16(x_residual))))
    return MOE_ERR_INVALID;
  return hip_status(moek::launch_combine(ret, dest, topk_w, p->add_residual ? x_residual : nullptr,
                                         p->x_dtype == MOE_BF16, y, p->B, p->k, p->d,
                                         kmax_of(p), stream, shared_out));
}

size_t moe_forward_shared_workspace_bytes(const moe_problem_t* p, const moe_problem_t* ps) {
  if (moe_validate(p) != MOE_OK || check_shared(ps) != MOE_OK) return SIZE_MAX;
  return carve_forward(p, nullptr, nullptr, nullptr) + shared_ws(ps) +
         align_up((size_t)p->B * p->d * 2);
}

moe_status_t moe_forward_shared(const moe_problem_t* p, const moe_problem_t* ps, const void* x,
                                const float* Wg, const float* bias, const void* wpacked,
                                const void* wpacked_shared, void* y, moe_forward_out_t* out,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  st = check_shared(ps);
  if (st != MOE_OK) return st;
  if (ps->B != p->B || ps->d != p->d) return MOE_ERR_INVALID;
  if (p->x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (p->B > 0 && (!wpacked_shared || !a16(wpacked_shared))) return MOE_ERR_INVALID;
  const size_t nf = carve_forward(p, out, nullptr, nullptr);
  const size_t need = nf + shared_ws(ps) + align_up((size_t)p->B * p->d * 2);
  if (p->B > 0 && (!ws || ws_bytes < need || !a16(ws))) return MOE_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  SharedRun sh;
  sh.ps = ps;
  sh.wp = wpacked_shared;
  sh.eo = p->B > 0 ? reinterpret_cast<int32_t*>(base + nf) : nullptr;
  sh.H = p->B > 0 ? reinterpret_cast<uint16_t*>(base + nf + align_up(8)) : nullptr;
  sh.S = p->B > 0 ? reinterpret_cast<uint16_t*>(base + nf + shared_ws(ps)) : nullptr;
  return forward_chain(p, x, Wg, bias, wpacked, y, out, ws, nf, stream, &sh);
}

int64_t moe_expert_choice_rows(const moe_problem_t* p) {
  if (moe_validate(p) != MOE_OK) return -1;
  return ec_rows(p);
}

static moe_status_t check_ec(const moe_problem_t* p) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->e_begin != 0 || p->e_end != p->E) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t moe_router_probs(const moe_problem_t* p, const float* logits, float* probs_t,
                              hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!logits || !probs_t || !a4(logits) || !a4(probs_t))) return MOE_ERR_INVALID;
  return hip_status(moek::launch_router_probs(logits, p->B, p->E, p->tau, probs_t, stream));
}

moe_status_t moe_expert_choice(const moe_problem_t* p, const float* probs_t, int32_t* sel_t,
                               int32_t* expert_offset, int32_t* pack_src, float* pack_w,
                               hipStream_t stream) {
  moe_status_t st = check_ec(p);
  if (st != MOE_OK) return st;
  if (!expert_offset || !a4(expert_offset)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!probs_t || !sel_t || !a4(probs_t) || !a4(sel_t))) return MOE_ERR_INVALID;
  if (ec_rows(p) > 0 && (!pack_src || !pack_w || !a4(pack_src) || !a4(pack_w)))
    return MOE_ERR_INVALID;
  const int64_t C = capacity_of(p);
  const int Ce = (int)(C < p->B ? C : p->B);
  return hip_status(moek::launch_expert_choice(probs_t, p->B, p->E, Ce, sel_t, expert_offset,
                                               pack_src, pack_w, stream));
}

moe_status_t moe_expert_choice_pack(const moe_problem_t* p, const void* x,
                                    const int32_t* pack_src, moe_bf16_t* packed,
                                    hipStream_t stream) {
  moe_status_t st = check_ec(p);
  if (st != MOE_OK) return st;
  const int64_t R = ec_rows(p);
  if (R > 0 && (!x || !pack_src || !packed || !a16(x) || !a16(packed))) return MOE_ERR_INVALID;
  return hip_status(
      moek::launch_ec_pack(x, p->x_dtype == MOE_BF16, pack_src, R, p->d, packed, stream));
}

moe_status_t moe_expert_choice_combine(const moe_problem_t* p, const moe_bf16_t* ret,
                                       const int32_t* sel_t, const float* pack_w,
                                       const void* x_residual, void* y, hipStream_t stream) {
  moe_status_t st = check_ec(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!sel_t || !y || !a16(y))) return MOE_ERR_INVALID;
  if (p->B > 0 && ec_rows(p) > 0 && (!ret || !pack_w || !a16(ret))) return MOE_ERR_INVALID;
  if (p->B > 0 && p->add_residual && (!x_residual || !a16(x_residual))) return MOE_ERR_INVALID;
  return hip_status(moek::launch_ec_combine(ret, sel_t, pack_w,
                                            p->add_residual ? x_residual : nullptr,
                                            p->x_dtype == MOE_BF16, y, p->B, p->E, p->d, stream));
}

moe_status_t moe_forward_expert_choice(const moe_problem_t* p, const void* x, const float* Wg,
                                       const float* bias, const void* wpacked, void* y,
                                       moe_expert_choice_out_t* out, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  moe_status_t st = check_ec(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!x || !Wg || !y || !wpacked)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(x) || !a16(y) || !a4(Wg) || (bias && !a4(bias)) || !a16(wpacked)))
    return MOE_ERR_INVALID;
  if (out && out->packed && !a16(out->packed)) return MOE_ERR_INVALID;
  const size_t need = carve_ec(p, out, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  EcBufs b;
  carve_ec(p, out, ws, &b);
  const bool xb = p->x_dtype == MOE_BF16;
  const int64_t C = capacity_of(p);
  const int Ce = (int)(C < p->B ? C : p->B);
  const int64_t R = ec_rows(p);
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (e == hipSuccess && out && out->events[i]) e = hipEventRecord(out->events[i], stream);
  };
  mark(0);
  if (e == hipSuccess)
    e = moek::launch_gate(x, xb, Wg, bias, b.logits, p->B, p->d, p->E, b.wsplit, stream);
  mark(1);
  if (e == hipSuccess)
    e = moek::launch_router_probs(b.logits, p->B, p->E, p->tau, b.probs_t, stream);
  if (e == hipSuccess)
    e = moek::launch_expert_choice(b.probs_t, p->B, p->E, Ce, b.sel_t, b.eo, b.pack_src,
                                   b.pack_w, stream);
  mark(2);
  if (e == hipSuccess) e = moek::launch_ec_pack(x, xb, b.pack_src, R, p->d, b.packed, stream);
  if (R > 0) {
    if (e == hipSuccess)
      e = moek::launch_expert_ffn(b.packed, b.eo, 0, p->E, Ce, Ce, p->d, p->f,
                                  p->act == MOE_SWIGLU, wpacked, b.H, b.packed, stream,
                                  out ? out->events[3] : nullptr, out ? out->events[4] : nullptr);
  } else {
    mark(3);
    mark(4);
  }
  if (e == hipSuccess)
    e = moek::launch_ec_combine(b.packed, b.sel_t, b.pack_w, p->add_residual ? x : nullptr, xb,
                                y, p->B, p->E, p->d, stream);
  mark(5);
  return hip_status(e);
}

}  // extern "C"

extern "C" int32_t moe_check_gate_split_reach(int64_t B, int32_t d, int32_t E, int64_t* read_end,
                                              int64_t* copy_bytes) {
  if (B < 1 || d < 8 || d % 8 || E < 1 || E > kMaxE || !read_end || !copy_bytes) return -1;
  *read_end = moek::gate_split_read_end(B, d, E);
  *copy_bytes = (int64_t)(moek::gate_use_split(true, B, d, E) ? moek::gate_split_bytes(d, E)
                                                               : moek::gate_block_bytes(d, E));
  return moek::gate_use_split(true, B, d, E) ? 1 : moek::gate_use_block(true, B, d, E) ? 2 : 0;
}

// ---------------------------------------------------------------------------
// backward pass
namespace {

moe_status_t check_bwd(const moe_problem_t* p) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->overflow != MOE_OVERFLOW_DROP) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// the expert FFN backward on carved scratch (shared by the stage call and
// the chain)
hipError_t ffn_backward(const moe_problem_t* p, const void* x, const int32_t* pack_src,
                        const int32_t* eo, const void* wp, const void* wpb, const uint16_t* zsaved,
                        uint16_t* dret, float* dW1, float* dW3, float* dW2, void* ws,
                        hipStream_t s) {
  const int nl = p->e_end - p->e_begin;
  if (nl <= 0 || p->B == 0) return hipSuccess;
  FfnBwdBufs b;
  carve_ffn_bwd(p, ws, &b);
  const bool sw = p->act == MOE_SWIGLU, xb = p->x_dtype == MOE_BF16;
  const int d = p->d, f = p->f, zw = moek::expert_ffn_zw(f, sw), zwd = sw ? 2 * f : f;
  const int rpe = (int)rows_per_expert(p), rh = rows_hint(p);
  const int64_t kl = kloc_of(p);
  // The local rows X = x[pack_src[r]]: gathered for the recompute, or, with
  // the pre-activations saved and bf16 tokens, read through pack_src by the
  // RB8 re-layout with no gathered copy.
  const bool direct = zsaved && xb;
  hipError_t e = hipSuccess;
  if (!direct)
    e = moek::launch_gather_rows(x, xb, pack_src, eo, p->e_begin, p->e_end, p->B, d, kl, b.xloc,
                                 s);
  // Z = X W1 (, X W3): the forward's first GEMM without its activation,
  // unless the forward saved it (the same kernel and order: the same bits)
  const uint16_t* Z = zsaved ? zsaved : b.Z;
  if (e == hipSuccess && !zsaved)
    e = moek::launch_ffn_recompute(b.xloc, eo, p->e_begin, nl, rpe, rh, d, f, sw, wp, b.Z, s);
  // RB8 operands of the weight gradients: X, H = act(Z), dret (local rows)
  if (e == hipSuccess)
    e = direct ? moek::launch_relayout_rb8(0, static_cast<const uint16_t*>(x), d, eo, p->e_begin,
                                           1, nl, rpe, d, d, -1, b.X8, s, pack_src, p->B)
               : moek::launch_relayout_rb8(0, b.xloc, d, eo, p->e_begin, 1, nl, rpe, d, d, -1,
                                           b.X8, s);
  if (e == hipSuccess)
    e = moek::launch_relayout_rb8(sw ? 2 : 1, Z, zw, eo, p->e_begin, 1, nl, rpe, f, zw, -1,
                                  b.H8, s);
  // dret is indexed by the absolute packed row
  if (e == hipSuccess)
    e = moek::launch_relayout_rb8(0, dret, d, eo, p->e_begin, 0, nl, rpe, d, d, -1, b.dret8, s);
  // dZ = dact(dret W2^T, Z), then dZ in RB8
  if (e == hipSuccess)
    e = moek::launch_ffn_dact(dret, eo, p->e_begin, nl, rpe, rh, d, f, sw, wpb, Z, b.dZ, s);
  if (e == hipSuccess)
    e = moek::launch_relayout_rb8(0, b.dZ, zwd, eo, p->e_begin, 1, nl, rpe, zwd, zwd, -1, b.dZ8,
                                  s);
  // dX = dZ [W1 | W3]^T over dret's local rows
  if (e == hipSuccess)
    e = moek::launch_ffn_dgrad(b.dZ, eo, p->e_begin, nl, rpe, rh, d, f, sw, wpb, dret, s);
  const int64_t r8 = moek::rb8_rows(rpe);
  // dW2 = H^T dret: C[m < f][n < d]
  if (e == hipSuccess) {
    moek::KGemm q{};
    q.A[0] = b.H8;
    q.B[0] = b.dret8;
    q.nseg = 1;
    q.a_w = f;
    q.b_w = d;
    q.a_es = r8 * f;
    q.b_es = r8 * d;
    q.a_bytes = 2 * r8 * f * nl;
    q.b_bytes = 2 * r8 * d * nl;
    q.eo = eo;
    q.e_begin = p->e_begin;
    q.groups = nl;
    q.M = f;
    q.N = d;
    q.C0 = dW2;
    q.ldc0 = d;
    q.c0_es = (int64_t)f * d;
    q.M0 = f;
    q.N0 = d;
    e = moek::launch_kgemm(q, s);
  }
  // [dW1 | dW3] = X^T [dZ1 | dZ3]: C[m < d][n < zwd], columns past f to dW3
  if (e == hipSuccess) {
    moek::KGemm q{};
    q.A[0] = b.X8;
    q.B[0] = b.dZ8;
    q.nseg = 1;
    q.a_w = d;
    q.b_w = zwd;
    q.a_es = r8 * d;
    q.b_es = r8 * zwd;
    q.a_bytes = 2 * r8 * d * nl;
    q.b_bytes = 2 * r8 * zwd * nl;
    q.eo = eo;
    q.e_begin = p->e_begin;
    q.groups = nl;
    q.M = d;
    q.N = zwd;
    q.C0 = dW1;
    q.ldc0 = f;
    q.c0_es = (int64_t)d * f;
    q.M0 = d;
    q.N0 = f;
    if (sw) {
      q.C1 = dW3;
      q.ldc1 = f;
      q.c1_es = (int64_t)d * f;
      q.r1 = 0;
      q.col1 = f;
      q.M1 = d;
      q.N1 = f;
    }
    e = moek::launch_kgemm(q, s);
  }
  return e;
}

hipError_t gate_backward(const moe_problem_t* p, const void* x, const float* Wg,
                         const float* dl, const float* dx_acc, void* dx, float* dWg, float* dbias,
                         void* ws, hipStream_t s) {
  if (p->B == 0) return hipSuccess;
  GateBwdBufs b;
  carve_gate_bwd(p, ws, &b);
  const bool xb = p->x_dtype == MOE_BF16;
  const int d = p->d, E = p->E, Ep = pad32(E);
  const int64_t B = p->B;
  // dx = dl Wg^T + dx_acc, contracting over the experts: dl and Wg in RB8
  // over e (parts hi, mid; three products (hi, hi) + (hi, mid) + (mid, hi))
  hipError_t e = moek::launch_split_rb8(dl, E, (int)B, E, true, (int)B, -1, b.dlt[0], b.dlt[1],
                                        nullptr, s);
  if (e == hipSuccess)
    e = moek::launch_split_rb8(Wg, E, d, E, true, d, -1, b.wgt[0], b.wgt[1], nullptr, s);
  if (e == hipSuccess) {
    moek::KGemm q{};
    const uint16_t* As[3] = {b.dlt[0], b.dlt[0], b.dlt[1]};
    const uint16_t* Bs[3] = {b.wgt[0], b.wgt[1], b.wgt[0]};
    for (int i = 0; i < 3; ++i) {
      q.A[i] = As[i];
      q.B[i] = Bs[i];
    }
    q.nseg = 3;
    q.a_w = (int)B;
    q.b_w = d;
    q.a_bytes = (int64_t)Ep * B * 2;
    q.b_bytes = (int64_t)Ep * d * 2;
    q.K = Ep;
    q.groups = 1;
    q.M = (int)B;
    q.N = d;
    q.mode = 1;
    q.M0 = (int)B;
    q.N0 = d;
    q.ldc0 = d;
    q.add = dx_acc;
    q.ld_add = d;
    q.xo = dx;
    q.x_bf16 = xb ? 1 : 0;
    e = moek::launch_kgemm(q, s);
  }
  // [dWg ; dbias] = [x | 1]^T dl over the tokens
  if (e == hipSuccess) {
    if (xb)
      e = moek::launch_relayout_rb8(0, static_cast<const uint16_t*>(x), d, nullptr, 0, 0, 1, B,
                                    d + 8, d, d, b.x8[0], s);
    else
      e = moek::launch_split_rb8(static_cast<const float*>(x), B, d, d, false, d + 8, d, b.x8[0],
                                 b.x8[1], b.x8[2], s);
  }
  if (e == hipSuccess)
    e = moek::launch_split_rb8(dl, B, E, E, false, Ep, -1, b.dl8[0], b.dl8[1], b.dl8[2], s);
  if (e == hipSuccess) {
    moek::KGemm q{};
    if (xb) {
      for (int i = 0; i < 3; ++i) {
        q.A[i] = b.x8[0];
        q.B[i] = b.dl8[i];
      }
      q.nseg = 3;
    } else {
      const int ai[6] = {0, 0, 1, 0, 2, 1}, bi[6] = {0, 1, 0, 2, 0, 1};
      for (int i = 0; i < 6; ++i) {
        q.A[i] = b.x8[ai[i]];
        q.B[i] = b.dl8[bi[i]];
      }
      q.nseg = 6;
    }
    // split-K over the tokens: group g sums tokens g Ks .. (g + 1) Ks into
    // its own [d + 1][E] partial; the partials are then added in g order
    const GateSplit gs = gate_split(p);
    const int64_t Br = moek::rb8_rows(B);
    q.a_w = d + 8;
    q.b_w = Ep;
    q.a_es = (int64_t)gs.Ks * (d + 8);
    q.b_es = (int64_t)gs.Ks * Ep;
    q.a_bytes = Br * (d + 8) * 2;
    q.b_bytes = Br * Ep * 2;
    q.K = gs.Ks;
    q.Ktot = (int)Br;
    q.groups = gs.G;
    q.M = d + 1;
    q.N = E;
    q.C0 = b.part;
    q.ldc0 = E;
    q.c0_es = (int64_t)(d + 1) * E;
    q.M0 = d + 1;
    q.N0 = E;
    e = moek::launch_kgemm(q, s);
    if (e == hipSuccess) e = moek::launch_sum_parts(b.part, gs.G, d, E, dWg, dbias, s);
  }
  return e;
}

}  // namespace

extern "C" {

moe_status_t moe_combine_backward(const moe_problem_t* p, const void* dy, const moe_bf16_t* ret,
                                  const int32_t* dest, const float* topk_w, moe_bf16_t* dret,
                                  float* dw, hipStream_t stream) {
  moe_status_t st = check_bwd(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!dy || !ret || !dest || !topk_w || !dret || !dw)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(dy) || !a16(ret) || !a16(dret) || !a4(dest) || !a4(topk_w) || !a4(dw)))
    return MOE_ERR_INVALID;
  return hip_status(moek::launch_combine_bwd(dy, p->x_dtype == MOE_BF16, ret, dest, topk_w, p->B,
                                             p->k, p->d, kmax_of(p), dret, dw, stream));
}

moe_status_t moe_route_backward(const moe_problem_t* p, const float* logits,
                                const int32_t* topk_idx, const float* dw,
                                const int32_t* expert_load, float aux_coef, float* dlogits,
                                hipStream_t stream) {
  moe_status_t st = check_bwd(p);
  if (st != MOE_OK) return st;
  if (!std::isfinite(aux_coef)) return MOE_ERR_INVALID;
  if (aux_coef != 0.0f && (!expert_load || !a4(expert_load))) return MOE_ERR_INVALID;
  if (p->B > 0 && (!logits || !topk_idx || !dw || !dlogits)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a4(logits) || !a4(topk_idx) || !a4(dw) || !a4(dlogits)))
    return MOE_ERR_INVALID;
  return hip_status(moek::launch_route_bwd(logits, topk_idx, dw, expert_load, aux_coef, p->B,
                                           p->E, p->k, p->tau, dlogits, stream));
}

size_t moe_saved_z_bytes(const moe_problem_t* p) {
  if (moe_validate(p) != MOE_OK) return SIZE_MAX;
  return (size_t)kloc_of(p) * (size_t)moek::expert_ffn_zw(p->f, p->act == MOE_SWIGLU) * 2;
}

size_t moe_weights_bwd_bytes(const moe_problem_t* p) {
  if (moe_validate(p) != MOE_OK) return SIZE_MAX;
  return moek::packed_weights_bwd_bytes(p->e_end - p->e_begin, p->d, p->f,
                                        p->act == MOE_SWIGLU);
}

moe_status_t moe_pack_weights_bwd(const moe_problem_t* p, const moe_bf16_t* W1,
                                  const moe_bf16_t* W3, const moe_bf16_t* W2, void* wpb,
                                  size_t wpb_bytes, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool sw = p->act == MOE_SWIGLU;
  const int nl = p->e_end - p->e_begin;
  if (nl == 0) return MOE_OK;
  if (!W1 || !W2 || (sw && !W3) || !wpb) return MOE_ERR_INVALID;
  if (!a16(W1) || !a16(W2) || (sw && !a16(W3)) || !a16(wpb)) return MOE_ERR_INVALID;
  if (wpb_bytes < moek::packed_weights_bwd_bytes(nl, p->d, p->f, sw)) return MOE_ERR_WORKSPACE;
  return hip_status(
      moek::launch_pack_weights_bwd(W1, sw ? W3 : nullptr, W2, nl, p->d, p->f, sw, wpb, stream));
}

moe_status_t moe_expert_ffn_backward(const moe_problem_t* p, const void* x,
                                     const int32_t* pack_src, const int32_t* expert_offset,
                                     const void* wpacked, const void* wpacked_bwd,
                                     const moe_bf16_t* z, moe_bf16_t* dret, float* dW1,
                                     float* dW3, float* dW2, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  moe_status_t st = check_bwd(p);
  if (st != MOE_OK) return st;
  const bool sw = p->act == MOE_SWIGLU;
  const int nl = p->e_end - p->e_begin;
  if (nl == 0) return MOE_OK;
  if (!expert_offset || !a4(expert_offset)) return MOE_ERR_INVALID;
  if (!wpacked || !wpacked_bwd || !dW1 || !dW2 || (sw && !dW3)) return MOE_ERR_INVALID;
  if (!a16(wpacked) || !a16(wpacked_bwd) || !a4(dW1) || !a4(dW2) || (sw && !a4(dW3)))
    return MOE_ERR_INVALID;
  if (p->B > 0 && (!x || !pack_src || !dret || !a16(x) || !a16(dret) || !a4(pack_src)))
    return MOE_ERR_INVALID;
  if (z && !a16(z)) return MOE_ERR_INVALID;
  const size_t need = carve_ffn_bwd(p, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need || !a16(ws))) return MOE_ERR_WORKSPACE;
  if (p->B == 0) {
    // no rows: every weight gradient is zero
    const int64_t n = (int64_t)nl * p->d * p->f;
    hipError_t e = moek::launch_fill_zero(dW1, n, stream);
    if (e == hipSuccess) e = moek::launch_fill_zero(dW2, n, stream);
    if (e == hipSuccess && sw) e = moek::launch_fill_zero(dW3, n, stream);
    return hip_status(e);
  }
  return hip_status(ffn_backward(p, x, pack_src, expert_offset, wpacked, wpacked_bwd, z, dret,
                                 dW1, sw ? dW3 : nullptr, dW2, ws, stream));
}

moe_status_t moe_dispatch_backward(const moe_problem_t* p, const moe_bf16_t* dxp,
                                   const int32_t* dest, const void* dy, float* dx_acc,
                                   hipStream_t stream) {
  moe_status_t st = check_bwd(p);
  if (st != MOE_OK) return st;
  if (p->B > 0 && (!dxp || !dest || !dx_acc || (p->add_residual && !dy))) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(dxp) || !a4(dest) || !a16(dx_acc) || (p->add_residual && !a16(dy))))
    return MOE_ERR_INVALID;
  return hip_status(moek::launch_unpack_sum(dxp, dest, dy, p->x_dtype == MOE_BF16,
                                            p->add_residual != 0, p->B, p->k, p->d, kmax_of(p),
                                            dx_acc, stream));
}

moe_status_t moe_gate_backward(const moe_problem_t* p, const void* x, const float* Wg,
                               const float* dlogits, const float* dx_acc, void* dx, float* dWg,
                               float* dbias, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_bwd(p);
  if (st != MOE_OK) return st;
  if (!dWg || !a4(dWg) || (dbias && !a4(dbias))) return MOE_ERR_INVALID;
  if (p->B > 0 && (!x || !Wg || !dlogits || !dx)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(x) || !a4(Wg) || !a4(dlogits) || !a4(dx) || (dx_acc && !a4(dx_acc))))
    return MOE_ERR_INVALID;
  const size_t need = carve_gate_bwd(p, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need || !a16(ws))) return MOE_ERR_WORKSPACE;
  if (p->B == 0) {
    hipError_t e = moek::launch_fill_zero(dWg, (int64_t)p->d * p->E, stream);
    if (e == hipSuccess && dbias) e = moek::launch_fill_zero(dbias, p->E, stream);
    return hip_status(e);
  }
  return hip_status(gate_backward(p, x, Wg, dlogits, dx_acc, dx, dWg, dbias, ws, stream));
}

}  // extern "C"

namespace {

// The shared expert of moe_backward_shared: its problem, packed weights,
// weight gradients, and its part of the workspace (after the routed one).
struct SharedBwd {
  const moe_problem_t* ps;
  const void *wp, *wpb;
  float *dW1, *dW3, *dW2;
};
// shared expert part of the backward workspace: its rows' indices (the
// tokens), expert_offset {0, B}, its output gradient (bf16 dy, overwritten
// by its input gradient), the expert FFN backward's scratch
struct SharedBwdBufs {
  int32_t *pack_src, *eo;
  uint16_t* dret;
  void* ffn_ws;
};
size_t carve_shared_bwd(const moe_problem_t* ps, void* ws, SharedBwdBufs* b) {
  Carve c;
  c.base = static_cast<char*>(ws);
  SharedBwdBufs t;
  t.pack_src = c.take<int32_t>(nullptr, (size_t)ps->B * 4);
  t.eo = c.take<int32_t>(nullptr, 2 * 4);
  t.dret = c.take<uint16_t>(nullptr, (size_t)ps->B * ps->d * 2);
  t.ffn_ws = c.take<char>(nullptr, carve_ffn_bwd(ps, nullptr, nullptr));
  if (b) *b = t;
  return c.off;
}

moe_status_t backward_chain(const moe_problem_t* p, const void* x, const float* Wg,
                            const void* wpacked, const void* wpacked_bwd, const moe_saved_t* sv,
                            const void* dy, float aux_coef, const moe_grads_t* g, void* ws,
                            size_t ws_bytes, hipStream_t stream, const SharedBwd* sh) {
  moe_status_t st = check_bwd(p);
  if (st != MOE_OK) return st;
  if (!sv || !g) return MOE_ERR_INVALID;
  if (!std::isfinite(aux_coef)) return MOE_ERR_INVALID;
  const bool sw = p->act == MOE_SWIGLU;
  const int nl = p->e_end - p->e_begin;
  if (!g->dWg || (nl > 0 && (!g->dW1 || !g->dW2 || (sw && !g->dW3)))) return MOE_ERR_INVALID;
  if (nl > 0 && (!wpacked || !wpacked_bwd || !a16(wpacked) || !a16(wpacked_bwd)))
    return MOE_ERR_INVALID;
  if (!sv->expert_offset || (aux_coef != 0.0f && !sv->expert_load)) return MOE_ERR_INVALID;
  if (p->B > 0 && (!x || !Wg || !dy || !g->dx || !sv->logits || !sv->topk_idx || !sv->topk_w ||
                   !sv->dest || !sv->pack_src || !sv->ret))
    return MOE_ERR_INVALID;
  if (p->B > 0 && (!a16(x) || !a16(dy) || !a16(sv->ret) || !a4(g->dx)))
    return MOE_ERR_INVALID;
  if (sv->z && !a16(sv->z)) return MOE_ERR_INVALID;
  if (sv->z_shared && (!sh || !a16(sv->z_shared))) return MOE_ERR_INVALID;
  if ((g->dw && !a4(g->dw)) || (g->dlogits && !a4(g->dlogits))) return MOE_ERR_INVALID;
  const bool ssw = sh && sh->ps->act == MOE_SWIGLU;
  if (sh) {
    st = check_shared(sh->ps);
    if (st != MOE_OK) return st;
    if (sh->ps->B != p->B || sh->ps->d != p->d) return MOE_ERR_INVALID;
    if (p->x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (!sh->wp || !sh->wpb || !a16(sh->wp) || !a16(sh->wpb)) return MOE_ERR_INVALID;
    if (!sh->dW1 || !sh->dW2 || (ssw && !sh->dW3) || !a4(sh->dW1) || !a4(sh->dW2) ||
        (ssw && !a4(sh->dW3)))
      return MOE_ERR_INVALID;
  }
  const size_t routed = align_up(carve_bwd(p, g, nullptr, nullptr));
  const size_t need = routed + (sh ? carve_shared_bwd(sh->ps, nullptr, nullptr) : 0);
  if (need > 0 && (!ws || ws_bytes < need || !a16(ws))) return MOE_ERR_WORKSPACE;
  BwdBufs b;
  carve_bwd(p, g, ws, &b);
  const bool xb = p->x_dtype == MOE_BF16;
  hipError_t e = hipSuccess;
  if (p->B == 0) {
    if (nl > 0) {
      const int64_t n = (int64_t)nl * p->d * p->f;
      e = moek::launch_fill_zero(g->dW1, n, stream);
      if (e == hipSuccess) e = moek::launch_fill_zero(g->dW2, n, stream);
      if (e == hipSuccess && sw) e = moek::launch_fill_zero(g->dW3, n, stream);
    }
    if (sh) {
      const int64_t n = (int64_t)p->d * sh->ps->f;
      if (e == hipSuccess) e = moek::launch_fill_zero(sh->dW1, n, stream);
      if (e == hipSuccess) e = moek::launch_fill_zero(sh->dW2, n, stream);
      if (e == hipSuccess && ssw) e = moek::launch_fill_zero(sh->dW3, n, stream);
    }
    if (e == hipSuccess) e = moek::launch_fill_zero(g->dWg, (int64_t)p->d * p->E, stream);
    if (e == hipSuccess && g->dbias) e = moek::launch_fill_zero(g->dbias, p->E, stream);
    return hip_status(e);
  }
  e = moek::launch_combine_bwd(dy, xb, sv->ret, sv->dest, sv->topk_w, p->B, p->k, p->d,
                               kmax_of(p), b.dret, b.dw, stream);
  if (e == hipSuccess)
    e = moek::launch_route_bwd(sv->logits, sv->topk_idx, b.dw, sv->expert_load, aux_coef, p->B,
                               p->E, p->k, p->tau, b.dl, stream);
  if (e == hipSuccess && nl > 0)
    e = ffn_backward(p, x, sv->pack_src, sv->expert_offset, wpacked, wpacked_bwd, sv->z, b.dret,
                     g->dW1, sw ? g->dW3 : nullptr, g->dW2, b.ffn_ws, stream);
  if (e == hipSuccess)
    e = moek::launch_unpack_sum(b.dret, sv->dest, dy, xb, p->add_residual != 0, p->B, p->k, p->d,
                                kmax_of(p), b.dx_acc, stream);
  if (sh) {
    // the shared expert's output entered y with weight 1: its output
    // gradient is dy; its input gradient joins the routed one before the
    // router's
    SharedBwdBufs s;
    carve_shared_bwd(sh->ps, static_cast<char*>(ws) + routed, &s);
    if (e == hipSuccess)
      e = moek::launch_shared_bwd_prep(s.pack_src, s.eo, static_cast<const uint16_t*>(dy), s.dret,
                                       p->B, p->d, stream);
    if (e == hipSuccess)
      e = ffn_backward(sh->ps, x, s.pack_src, s.eo, sh->wp, sh->wpb, sv->z_shared, s.dret,
                       sh->dW1, ssw ? sh->dW3 : nullptr, sh->dW2, s.ffn_ws, stream);
    if (e == hipSuccess) e = moek::launch_add_bf16(b.dx_acc, s.dret, p->B * p->d, stream);
  }
  if (e == hipSuccess)
    e = gate_backward(p, x, Wg, b.dl, b.dx_acc, g->dx, g->dWg, g->dbias, b.gate_ws, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

moe_status_t moe_backward(const moe_problem_t* p, const void* x, const float* Wg,
                          const void* wpacked, const void* wpacked_bwd, const moe_saved_t* sv,
                          const void* dy, float aux_coef, const moe_grads_t* g, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return backward_chain(p, x, Wg, wpacked, wpacked_bwd, sv, dy, aux_coef, g, ws, ws_bytes,
                        stream, nullptr);
}

size_t moe_backward_shared_workspace_bytes(const moe_problem_t* p, const moe_problem_t* ps) {
  if (check_bwd(p) != MOE_OK || check_shared(ps) != MOE_OK) return SIZE_MAX;
  return align_up(carve_bwd(p, nullptr, nullptr, nullptr)) + carve_shared_bwd(ps, nullptr, nullptr);
}

moe_status_t moe_backward_shared(const moe_problem_t* p, const moe_problem_t* ps, const void* x,
                                 const float* Wg, const void* wpacked, const void* wpacked_bwd,
                                 const void* wpacked_shared, const void* wpacked_shared_bwd,
                                 const moe_saved_t* saved, const void* dy, float aux_coef,
                                 const moe_grads_t* grads, float* dW1s, float* dW3s, float* dW2s,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ps) return MOE_ERR_INVALID;
  const SharedBwd sh{ps, wpacked_shared, wpacked_shared_bwd, dW1s, dW3s, dW2s};
  return backward_chain(p, x, Wg, wpacked, wpacked_bwd, saved, dy, aux_coef, grads, ws, ws_bytes,
                        stream, &sh);
}

}  // extern "C"
