// Gate-weighted combine back into token order, its unpack helper, and the
// identity return of rows whose experts run elsewhere.
//
// "Expert Parallelism" (narrativegoldmine.com), "Components and
// Architecture", expert combine: a token's k expert outputs are weighted by
// their gating probabilities and summed before the residual addition;
// "Formal Algorithm", expert combine and residual addition.  "Expert
// Parallelism and the All-to-All Bottleneck", "The Mechanism of Expert
// Parallelism": the gathered rows return to (tokens, hidden) in the original
// token order.  On one GPU the return all-to-all is the identity, so the
// combine reads the packed rows in place (a gather by dest; no atomics, fixed
// j order, fp32 accumulation).
//
// All three kernels are row copies/gathers bound by HBM: one thread moves a
// 16-byte chunk (8 bf16), consecutive threads walk a row.
#include "launch.h"
#include "moe_kernels.h"

namespace moek {
namespace {

unsigned grid_for(int64_t work, int threads) {
  int64_t g = (work + threads - 1) / threads;
  if (g > (1 << 20)) g = 1 << 20;
  if (g < 1) g = 1;
  return (unsigned)g;
}

// One wavefront per token row, one lane per 16-byte chunk: block (4 tokens)
// x (64 chunks), grid (ceil(B / 4), ceil(d / 512)).  The token index is
// wavefront-uniform, so dest and the weights come through scalar loads; the
// expert rows are read once, non-temporally.  SH: a shared expert's output
// row (bf16, "Major Variants and Families", shared expert routing) is added
// with weight 1 after the routed sum, before the residual.
template <bool XBF16, bool RES, bool SH>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint16_t* __restrict__ ret, const int32_t* __restrict__ dest,
    const float* __restrict__ w, const void* __restrict__ xres,
    const uint16_t* __restrict__ shared, void* __restrict__ y, int64_t B, int k, int d,
    int64_t kmax) {
  const int cpr = d / 8;
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t ntb = (B + 3) / 4;
  for (int64_t tb = blockIdx.y; tb < ntb; tb += gridDim.y) {
    const int64_t t = tb * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= B || c >= cpr) continue;
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = dest[t * k + j];
      if (r >= 0 && r < kmax) {
        const float wj = w[t * k + j];
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)(ret + (int64_t)r * d + c * 8));
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fmaf(wj, f[u], acc[u]);
      }
    }
    if (SH) {
      float sv[8];
      unpack8(__builtin_nontemporal_load((const u32x4*)(shared + t * d + c * 8)), sv);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += sv[u];
    }
    if (RES) {
      float xr[8];
      if (XBF16) {
        unpack8(*(const u32x4*)((const uint16_t*)xres + t * d + c * 8), xr);
      } else {
        const float* xf = (const float*)xres + t * d + c * 8;
        const f32x4 a = *(const f32x4*)xf;
        const f32x4 b = *(const f32x4*)(xf + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) { xr[u] = a[u]; xr[u + 4] = b[u]; }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += xr[u];
    }
    // y is stored non-temporally: nothing in the layer reads it again, and
    // normal stores let it displace the expert rows still to be read (EP
    // share: combine 760 -> 711 us; the drop-heavy shape 14.5 -> 13.4 us;
    // the others unchanged)
    if (XBF16) {
      __builtin_nontemporal_store(pack8(acc), (u32x4*)((uint16_t*)y + t * d + c * 8));
    } else {
      float* yf = (float*)y + t * d + c * 8;
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)yf);
      __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, (f32x4*)(yf + 4));
    }
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint16_t* __restrict__ ret,
                                                     const int32_t* __restrict__ dest, int64_t B,
                                                     int k, int d, int64_t kmax,
                                                     uint16_t* __restrict__ out) {
  const int cpr = d / 8;
  const int64_t total = B * k * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t tj = i / cpr;
    const int c = (int)(i - tj * cpr);
    const int r = dest[tj];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= 0 && r < kmax) v = *(const u32x4*)(ret + (int64_t)r * d + c * 8);
    *(u32x4*)(out + tj * d + c * 8) = v;
  }
}

__global__ __launch_bounds__(256) void copy_remote_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst,
                                                          const int32_t* __restrict__ eo, int E,
                                                          int e_begin, int e_end, int64_t kmax,
                                                          int d) {
  const int64_t K = eo[E];
  const int64_t lo = eo[e_begin], hi = eo[e_end];
  const int cpr = d / 8;
  const int64_t total = (K < kmax ? K : kmax) * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cpr;
    if (r >= lo && r < hi) continue;
    const int c = (int)(i - r * cpr);
    *(u32x4*)(dst + r * d + c * 8) = *(const u32x4*)(src + r * d + c * 8);
  }
}

}  // namespace

template <bool XBF16, bool RES>
void launch_combine_t(dim3 g, const uint16_t* ret, const int32_t* dest, const float* w,
                      const void* x_res, const uint16_t* shared, void* y, int64_t B, int k, int d,
                      int64_t kmax, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (shared)
    launch_timed((combine_kernel<XBF16, RES, true>), g, dim3(256), 0, s, e0, e1, ret,
                 dest, w, x_res, shared, y, B, k, d, kmax);
  else
    launch_timed((combine_kernel<XBF16, RES, false>), g, dim3(256), 0, s, e0, e1, ret,
                 dest, w, x_res, shared, y, B, k, d, kmax);
}

hipError_t launch_combine(const uint16_t* ret, const int32_t* dest, const float* w,
                          const void* x_res, bool x_bf16, void* y, int64_t B, int k, int d,
                          int64_t kmax, hipStream_t s, const uint16_t* shared, hipEvent_t e0,
                          hipEvent_t e1) {
  if (B == 0) return hipSuccess;
  // x: 512-column piece of the rows (fastest in dispatch order, so
  // consecutive workgroups cover consecutive pieces of the same rows);
  // y: groups of 4 rows, at most 65535 (the kernel loops over the rest)
  const int64_t ntb = (B + 3) / 4;
  const dim3 g((unsigned)((d / 8 + 63) / 64), (unsigned)(ntb < 65535 ? ntb : 65535));
  if (x_bf16) {
    if (x_res)
      launch_combine_t<true, true>(g, ret, dest, w, x_res, shared, y, B, k, d, kmax, s, e0, e1);
    else
      launch_combine_t<true, false>(g, ret, dest, w, x_res, shared, y, B, k, d, kmax, s, e0, e1);
  } else {
    if (x_res)
      launch_combine_t<false, true>(g, ret, dest, w, x_res, shared, y, B, k, d, kmax, s, e0, e1);
    else
      launch_combine_t<false, false>(g, ret, dest, w, x_res, shared, y, B, k, d, kmax, s, e0, e1);
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const uint16_t* ret, const int32_t* dest, int64_t B, int k, int d,
                         int64_t kmax, uint16_t* out, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const unsigned g = grid_for(B * k * (d / 8), 256);
  hipLaunchKernelGGL(unpack_kernel, dim3(g), dim3(256), 0, s, ret, dest, B, k, d, kmax, out);
  return hipGetLastError();
}

hipError_t launch_copy_remote(const uint16_t* src, uint16_t* dst, const int32_t* expert_offset,
                              int E, int e_begin, int e_end, int64_t kmax, int d, hipStream_t s) {
  if (kmax <= 0) return hipSuccess;
  const unsigned g = grid_for(kmax * (d / 8), 256);
  hipLaunchKernelGGL(copy_remote_kernel, dim3(g), dim3(256), 0, s, src, dst, expert_offset, E,
                     e_begin, e_end, kmax, d);
  return hipGetLastError();
}

}  // namespace moek
