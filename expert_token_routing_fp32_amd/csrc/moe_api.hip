// C ABI of the MoE layer forward: host-side checks, capacity, workspace
// layout and the launch order of the kernels.  Declared in include/moe.h.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "moe.h"
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
  t.wsplit = moek::gate_use_split(p->x_dtype == MOE_BF16, p->B, p->d, p->E)
                 ? c.take<char>(nullptr, moek::gate_split_bytes(p->d, p->E))
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
  t.wsplit = moek::gate_use_split(p->x_dtype == MOE_BF16, p->B, p->d, p->E)
                 ? c.take<char>(nullptr, moek::gate_split_bytes(p->d, p->E))
                 : nullptr;
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
  if (e == hipSuccess)
    e = moek::launch_pack(x, xb, b.dest, p->B, p->k, p->d, b.packed, stream, nullptr, ev[4]);
  // with a shared expert its GEMMs follow the routed ones inside the FFN pair
  if (p->B > 0) {
    if (e == hipSuccess)
      e = moek::launch_expert_ffn(b.packed, b.eo, p->e_begin, n_local, (int)rows_per_expert(p),
                                  rows_hint(p), p->d, p->f, swiglu, wpacked, b.H, b.packed,
                                  stream, ev[5], sh ? nullptr : ev[6]);
    if (e == hipSuccess && sh)
      e = moek::launch_shared_ffn(static_cast<const uint16_t*>(x), p->B, p->d, sh->ps->f,
                                  sh->ps->act == MOE_SWIGLU, sh->wp, sh->H, sh->eo, sh->S, stream,
                                  ev[6]);
  }
  if (e == hipSuccess)
    e = moek::launch_combine(b.packed, b.dest, b.w, p->add_residual ? x : nullptr, xb, y, p->B,
                             p->k, p->d, kmax_of(p), stream, sh ? sh->S : nullptr, ev[7], ev[8]);
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
