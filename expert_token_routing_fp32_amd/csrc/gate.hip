// Router logits g = x . Wg (+ b) in fp32 on the vector ALUs.
//
// "Expert Parallelism" (narrativegoldmine.com), "Formal Algorithm": the
// router logit vector g_t comes from the routing linear projection;
// "Components and Architecture": a learned linear map, with a bias term on
// the routing logits in the aux-loss-free variant.
//
// The router is an fp32 layer, so this contraction stays off the bf16 matrix
// cores.  A block owns BT tokens x BE experts; its four waves split each
// 128-wide slice of d four ways (split-K inside the block), every lane keeps
// a TM x 4 register tile, and each wave sums its 32 products per slice into a
// fresh partial before adding it to the running total (blocked accumulation
// keeps the fp32 error near sqrt(32) + sqrt(d/32) roundings, not sqrt(d)).
// The four wave totals are added in a fixed order, so results do not depend
// on scheduling.
#include "moe_kernels.h"

namespace moek {
namespace {

constexpr int kGateThreads = 256;
constexpr int kGateBK = 32;                 // d values per wave per slice
constexpr int kGateKC = 4 * kGateBK;        // d values per block per slice

template <int BE, int TM, bool XBF16>
__global__ __launch_bounds__(kGateThreads) void gate_kernel(
    const void* __restrict__ xv, const float* __restrict__ Wg, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t B, int d, int E) {
  constexpr int TN = 4;
  constexpr int LE = BE / TN;     // lanes along experts
  constexpr int LT = kWave / LE;  // lanes along tokens
  constexpr int BT = LT * TM;     // tokens per block
  __shared__ float xs[kGateKC][BT];
  __shared__ float ws[kGateKC][BE];
  __shared__ float red[4][BT][BE];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int le = lane % LE, lt = lane / LE;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int e0 = blockIdx.y * BE;
  const bool vecw = (E % 4) == 0;

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  for (int kc = 0; kc < d; kc += kGateKC) {
    // stage x[t0 .. t0+BT) x [kc .. kc+KC) as fp32, k-major
    for (int i = tid; i < BT * (kGateKC / 8); i += kGateThreads) {
      const int r = i / (kGateKC / 8), c8 = i % (kGateKC / 8);
      const int64_t t = t0 + r;
      const int kk = kc + c8 * 8;
      float v[8];
      if (t < B && kk < d) {
        if (XBF16) {
          const u32x4 q = *(const u32x4*)((const uint16_t*)xv + t * d + kk);
          unpack8(q, v);
        } else {
          const f32x4 a = *(const f32x4*)((const float*)xv + t * d + kk);
          const f32x4 b = *(const f32x4*)((const float*)xv + t * d + kk + 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) { v[u] = a[u]; v[u + 4] = b[u]; }
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) xs[c8 * 8 + u][r] = v[u];
    }
    // stage Wg[kc .. kc+KC) x [e0 .. e0+BE)
    if (vecw) {
      for (int i = tid; i < kGateKC * (BE / 4); i += kGateThreads) {
        const int r = i / (BE / 4), c4 = (i % (BE / 4)) * 4;
        const int kk = kc + r, e = e0 + c4;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (kk < d && e < E) v = *(const f32x4*)(Wg + (int64_t)kk * E + e);
        *(f32x4*)&ws[r][c4] = v;
      }
    } else {
      for (int i = tid; i < kGateKC * BE; i += kGateThreads) {
        const int r = i / BE, c = i % BE;
        const int kk = kc + r, e = e0 + c;
        ws[r][c] = (kk < d && e < E) ? Wg[(int64_t)kk * E + e] : 0.f;
      }
    }
    __syncthreads();

    float part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) part[i][j] = 0.f;
    const int kb = wave * kGateBK;
#pragma unroll 8
    for (int kk = 0; kk < kGateBK; ++kk) {
      float xr[TM];
      if constexpr (TM == 4) {
        const f32x4 q = *(const f32x4*)&xs[kb + kk][lt * TM];
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[i] = q[i];
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) xr[i] = xs[kb + kk][lt * TM + i];
      }
      const f32x4 wr = *(const f32x4*)&ws[kb + kk][le * TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) part[i][j] = fmaf(xr[i], wr[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) red[wave][lt * TM + i][le * TN + j] = acc[i][j];
  __syncthreads();
  for (int o = tid; o < BT * BE; o += kGateThreads) {
    const int r = o / BE, c = o % BE;
    const int64_t t = t0 + r;
    const int e = e0 + c;
    if (t < B && e < E) {
      float s = red[0][r][c];
      s += red[1][r][c];
      s += red[2][r][c];
      s += red[3][r][c];
      if (bias) s += bias[e];
      logits[t * E + e] = s;
    }
  }
}

template <int BE, int TM>
hipError_t launch_gate_t(const void* x, bool x_bf16, const float* Wg, const float* bias,
                         float* logits, int64_t B, int d, int E, hipStream_t s) {
  constexpr int BT = (kWave / (BE / 4)) * TM;
  dim3 grid((unsigned)((B + BT - 1) / BT), (unsigned)((E + BE - 1) / BE));
  if (x_bf16)
    hipLaunchKernelGGL((gate_kernel<BE, TM, true>), grid, dim3(kGateThreads), 0, s, x, Wg, bias,
                       logits, B, d, E);
  else
    hipLaunchKernelGGL((gate_kernel<BE, TM, false>), grid, dim3(kGateThreads), 0, s, x, Wg, bias,
                       logits, B, d, E);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const void* x, bool x_bf16, const float* Wg, const float* bias,
                       float* logits, int64_t B, int d, int E, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (E > 32) return launch_gate_t<64, 4>(x, x_bf16, Wg, bias, logits, B, d, E, s);
  if (E > 16) return launch_gate_t<32, 4>(x, x_bf16, Wg, bias, logits, B, d, E, s);
  if (E > 8) return launch_gate_t<16, 2>(x, x_bf16, Wg, bias, logits, B, d, E, s);
  return launch_gate_t<8, 1>(x, x_bf16, Wg, bias, logits, B, d, E, s);
}

}  // namespace moek
