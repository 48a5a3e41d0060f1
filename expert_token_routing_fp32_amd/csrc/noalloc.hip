// moe_dispatch without a workspace argument, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops or
// harnesses that forbid hipMalloc).  The slot kernels' per-tile count table
// lives in a fixed, device-resident array instead of a caller workspace.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, from the first use until the
// process ends.  In host code the variable's name is only a host-side
// handle, so the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever passed to kernels.
//
// Nothing in the table needs to start at zero: the histogram kernel writes
// every (tile, expert) count, and clears the multi-block scan's completion
// counter, before the scan or rank kernels read them.  All
// calls on one GPU share the table, so calls that overlap on one GPU (on
// different streams, unordered) race and must not be issued.
#include <mutex>

#include <hip/hip_runtime.h>

#include "moe.h"
#include "moe_kernels.h"

namespace {

constexpr size_t kScratchBytes = MOE_DISPATCH_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first
// call on the device (the current one); null on a HIP error.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const void* x,
                                             const int32_t* topk_idx, int32_t* pos,
                                             uint8_t* keep, int32_t* dest, int32_t* expert_load,
                                             int32_t* expert_count, int32_t* expert_offset,
                                             int32_t* rank_offset, int32_t* pack_src,
                                             moe_bf16_t* packed, hipStream_t stream) {
  moe_status_t st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->overflow != MOE_OVERFLOW_DROP) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_workspace_bytes(p, MOE_OP_DISPATCH);
  if (need > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* ws = scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  return moe_dispatch(p, x, topk_idx, pos, keep, dest, expert_load, expert_count, expert_offset,
                      rank_offset, pack_src, packed, ws, kScratchBytes, stream);
}
