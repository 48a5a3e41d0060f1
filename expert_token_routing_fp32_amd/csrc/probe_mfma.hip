// Matrix-core ceiling probe (measurement only; not part of the forward path).
//
// Runs the expert GEMM's inner-loop instruction mix -- one wavefront per
// SIMD, v_mfma_f32_32x32x16_bf16 into 16 accumulator blocks, every A
// fragment re-read from LDS after the two MFMAs that use it -- with no
// global memory traffic, so the time it takes is set by the matrix cores
// and the clock alone.  With random bf16 operands (random signs and
// mantissas) the part draws more power than with near-constant operands,
// and the sustained clock, hence the reachable fraction of the datasheet
// peak, drops; both cases are offered so that a GEMM's utilisation can be
// read against what the chip sustains under the same kind of data.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probe.h"

namespace {

typedef unsigned int p_u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 p_bf16x8 __attribute__((ext_vector_type(8)));
typedef float p_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLds = 160 * 1024;

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(float* __restrict__ out, int iters,
                                                            int random_data) {
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  const int lane = threadIdx.x & 63;
  // operands: 32 KB of A fragments and 2 KB of B fragments in LDS
  for (int i = threadIdx.x; i < (34 * 1024) / 4; i += 256) {
    uint32_t h = (uint32_t)(i + 7919 * blockIdx.x) * 2654435761u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    // random data: two bf16 numbers with random sign and mantissa and
    // magnitude in [0.5, 1); otherwise small values repeating every 8 words
    reinterpret_cast<uint32_t*>(smem)[i] =
        random_data ? ((h & 0x807F807Fu) | 0x3F003F00u) : __float_as_uint(0.001f * (i & 7));
  }
  __syncthreads();
  p_f32x16 acc[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][i][r] = 0.f;
  p_u32x4 fa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fa[i] = *(const p_u32x4*)(smem + 4096 * i + 16 * lane);
  const p_u32x4 b0 = *(const p_u32x4*)(smem + 32768 + 16 * lane);
  const p_u32x4 b1 = *(const p_u32x4*)(smem + 33792 + 16 * lane);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const p_bf16x8 a = __builtin_bit_cast(p_bf16x8, fa[i]);
        acc[0][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(p_bf16x8, b0),
                                                            acc[0][i], 0, 0, 0);
        acc[1][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(p_bf16x8, b1),
                                                            acc[1][i], 0, 0, 0);
        fa[i] = *(const p_u32x4*)(smem + 4096 * i + 1024 * ((s + 1) & 3) + 16 * lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // one value per thread keeps every accumulator live
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[c][i][r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace

extern "C" int moe_probe_mfma(float* out, int grid, int iters, int random_data,
                              hipStream_t stream) {
  if (!out || grid <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(256), 0, stream, out, iters,
                     random_data);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" double moe_probe_mfma_flop(int grid, int iters) {
  // per wavefront and iteration: 64 MFMAs of 32 x 32 x 16 multiply-adds
  return (double)grid * 4.0 * (double)iters * 64.0 * (2.0 * 32 * 32 * 16);
}

// ---- HBM streaming probes ----------------------------------------------------
namespace {

__global__ __launch_bounds__(256) void hbm_probe_kernel(int mode, const p_u32x4* __restrict__ src,
                                                        p_u32x4* __restrict__ dst, int64_t n,
                                                        unsigned* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (mode == 0) {
    unsigned acc = 0u;
    for (; i < n; i += stride) {
      const p_u32x4 v = __builtin_nontemporal_load(src + i);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
  } else if (mode == 1) {
    const p_u32x4 v = {(unsigned)i, 1u, 2u, 3u};
    for (; i < n; i += stride) __builtin_nontemporal_store(v, dst + i);
  } else {
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  }
}

}  // namespace

extern "C" int moe_probe_hbm(int mode, const void* src, void* dst, size_t bytes, unsigned* out,
                             int grid, hipStream_t stream) {
  if (mode < 0 || mode > 2 || bytes == 0 || bytes % 16 || grid < 1) return 1;
  if ((mode != 1 && !src) || (mode != 0 && !dst) || (mode == 0 && !out)) return 1;
  hipLaunchKernelGGL(hbm_probe_kernel, dim3(grid), dim3(256), 0, stream, mode,
                     static_cast<const p_u32x4*>(src), static_cast<p_u32x4*>(dst),
                     (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
