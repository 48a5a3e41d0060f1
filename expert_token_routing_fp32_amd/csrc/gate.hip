// Router logits g = x . Wg (+ b), fp32.
//
// "Expert Parallelism" (narrativegoldmine.com), "Formal Algorithm": the
// router logit vector g_t comes from the routing linear projection;
// "Components and Architecture": a learned linear map, with a bias term on
// the routing logits in the aux-loss-free variant.
//
// bf16 activations: matrix cores, with fp32 semantics kept exactly.  Every
// fp32 router weight w is split into three bf16 numbers w = hi + mid + lo
// with no rounding at all (hi = w truncated to bf16, mid = the next 8
// significant bits of the remainder, lo = the last 8), so each product x*w
// is the sum of three products of bf16 numbers, each exact in fp32.  The
// three bf16 MFMAs per step therefore accumulate exactly the terms an fp32
// FMA loop would, in fp32 (in another order), at 3/16 of the cost of fp32
// matrix instructions.  x is bf16 already and is used as is.
//
//   wave     = 32 MI tokens x 32 experts x a K range (v_mfma_f32_32x32x16_bf16)
//   block    = EB expert blocks x KS K ranges; the KS partial sums are added
//              in a fixed order through LDS, so results do not depend on
//              scheduling
//   operands = straight from global memory into registers (x rows: 16 bytes
//              per lane; weights: the lane's expert column, 8 k values per
//              step), one group of steps prefetched ahead; the EB waves of a
//              block read the same x rows, which the caches serve
//
// fp32 activations: the vector ALUs (a block owns BT tokens x BE experts;
// four waves split each 128-wide slice of d; blocked accumulation keeps the
// fp32 error near sqrt(32) + sqrt(d/32) roundings; the four wave totals are
// added in a fixed order).
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

typedef __bf16 g_bf16x8 __attribute__((ext_vector_type(8)));
typedef float g_f32x16 __attribute__((ext_vector_type(16)));

// Exact three-way split of 8 fp32 weights into bf16 octets (lane layout of
// an MFMA B operand: 8 consecutive k of one column).
__device__ __forceinline__ void split3(const float* v, u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned int u0 = __float_as_uint(v[2 * j]), u1 = __float_as_uint(v[2 * j + 1]);
    const unsigned int h0 = u0 & 0xFFFF0000u, h1 = u1 & 0xFFFF0000u;
    const float r0 = v[2 * j] - __uint_as_float(h0), r1 = v[2 * j + 1] - __uint_as_float(h1);
    const unsigned int m0 = __float_as_uint(r0) & 0xFFFF0000u, m1 = __float_as_uint(r1) & 0xFFFF0000u;
    // r - m has at most 8 significant bits: exactly a bf16 number
    const unsigned int q0 = __float_as_uint(r0 - __uint_as_float(m0));
    const unsigned int q1 = __float_as_uint(r1 - __uint_as_float(m1));
    hi[j] = (h0 >> 16) | h1;
    mid[j] = (m0 >> 16) | m1;
    lo[j] = (q0 >> 16) | (q1 & 0xFFFF0000u);
  }
}

template <int MI, int G, int EB, int KS>
__global__ __launch_bounds__(64 * EB * KS) void gate_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ Wg, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t B, int d, int E) {
  extern __shared__ float red[];  // [EB][KS-1][MI*16][64]
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int eb = w % EB, kq = w / EB;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * (32 * MI);
  const int e0 = (blockIdx.y * EB + eb) * 32;
  const int kspan = (d + 16 * KS - 1) / (16 * KS) * 16;
  const int kb = kq * kspan;
  const int ke = kb + kspan < d ? kb + kspan : d;
  const int nsteps = ke > kb ? (ke - kb + 15) / 16 : 0;

  // rows / column past the edge read a valid neighbour; their results are
  // never stored
  const uint16_t* xr[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t t = t0 + 32 * i + l32;
    xr[i] = x + (t < B ? t : B - 1) * d + 8 * h;
  }
  const float* wc = Wg + (e0 + l32 < E ? e0 + l32 : E - 1);

  g_f32x16 acc[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  u32x4 xa[2][G][MI];
  float wv[2][G][8];
  // step s covers k = kb + 16 s .. +15; this lane's half is k + 8 h .. +7,
  // which lies wholly inside or outside [kb, ke) (d is a multiple of 8)
#define GATE_LOAD(BUF, S0)                                                        \
  _Pragma("unroll") for (int g_ = 0; g_ < G; ++g_) {                              \
    const int k_ = kb + 16 * ((S0) + g_) + 8 * h;                                  \
    const bool ok_ = k_ < ke;                                                      \
    /* outside: the row's first chunk (xr already points 8 h into the row) */     \
    const int kc_ = ok_ ? k_ - 8 * h : -8 * h;                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < MI; ++i_)                              \
      xa[BUF][g_][i_] = *(const u32x4*)(xr[i_] + kc_);                             \
    const float* wp_ = wc + (int64_t)(ok_ ? k_ : 0) * E;                           \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) {                             \
      const float v_ = wp_[(int64_t)j_ * E];                                       \
      wv[BUF][g_][j_] = ok_ ? v_ : 0.f;                                            \
    }                                                                              \
  }
#define GATE_COMPUTE(BUF)                                                         \
  _Pragma("unroll") for (int g_ = 0; g_ < G; ++g_) {                              \
    u32x4 hi_, mid_, lo_;                                                          \
    split3(wv[BUF][g_], hi_, mid_, lo_);                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < MI; ++i_) {                            \
      const g_bf16x8 a_ = __builtin_bit_cast(g_bf16x8, xa[BUF][g_][i_]);           \
      acc[i_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                          \
          a_, __builtin_bit_cast(g_bf16x8, lo_), acc[i_], 0, 0, 0);                \
      acc[i_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                          \
          a_, __builtin_bit_cast(g_bf16x8, mid_), acc[i_], 0, 0, 0);               \
      acc[i_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                          \
          a_, __builtin_bit_cast(g_bf16x8, hi_), acc[i_], 0, 0, 0);                \
    }                                                                              \
  }

  if (nsteps > 0) {
    GATE_LOAD(0, 0)
    for (int s0 = 0; s0 < nsteps; s0 += 2 * G) {
      GATE_LOAD(1, s0 + G)
      GATE_COMPUTE(0)
      if (s0 + 2 * G < nsteps) {
        GATE_LOAD(0, s0 + 2 * G)
      }
      GATE_COMPUTE(1)
    }
  }
#undef GATE_LOAD
#undef GATE_COMPUTE

  // acc[i][r] is token t0 + 32 i + 8 (r / 4) + 4 h + r % 4, expert e0 + l32
  if (KS > 1) {
    if (kq > 0) {
      float* dst = red + ((eb * (KS - 1) + kq - 1) * MI * 16) * 64 + lane;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(i * 16 + r) * 64] = acc[i][r];
    }
    __syncthreads();
    if (kq > 0) return;
#pragma unroll
    for (int q = 1; q < KS; ++q) {
      const float* src = red + ((eb * (KS - 1) + q - 1) * MI * 16) * 64 + lane;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] += src[(i * 16 + r) * 64];
    }
  }
  const int e = e0 + l32;
  if (e >= E) return;
  const float be = bias ? bias[e] : 0.f;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
      if (t < B) logits[t * E + e] = acc[i][r] + be;
    }
}

template <int MI, int EB, int KS>
hipError_t launch_gate_mfma_t(const uint16_t* x, const float* Wg, const float* bias, float* logits,
                              int64_t B, int d, int E, hipStream_t s) {
  constexpr int G = MI == 4 ? 2 : 4;
  const int neb = (E + 31) / 32;
  dim3 grid((unsigned)((B + 32 * MI - 1) / (32 * MI)), (unsigned)((neb + EB - 1) / EB));
  const size_t lds = (size_t)EB * (KS - 1) * MI * 16 * 64 * sizeof(float);
  hipLaunchKernelGGL((gate_mfma_kernel<MI, G, EB, KS>), grid, dim3(64 * EB * KS), lds, s, x, Wg,
                     bias, logits, B, d, E);
  return hipGetLastError();
}

template <int EB, int KS>
hipError_t launch_gate_mfma_mi(int mi, const uint16_t* x, const float* Wg, const float* bias,
                               float* logits, int64_t B, int d, int E, hipStream_t s) {
  if (mi == 4) return launch_gate_mfma_t<4, EB, KS>(x, Wg, bias, logits, B, d, E, s);
  if (mi == 2) return launch_gate_mfma_t<2, EB, KS>(x, Wg, bias, logits, B, d, E, s);
  return launch_gate_mfma_t<1, EB, KS>(x, Wg, bias, logits, B, d, E, s);
}

// Block shape: up to 8 waves; EB expert blocks (up to 256 experts share the
// x rows), the rest of the 8 waves split K while each wave keeps >= 64 k;
// token tiles (at most 8 / KS row blocks) shrink until there are >= 128
// blocks.
hipError_t launch_gate_mfma(const uint16_t* x, const float* Wg, const float* bias, float* logits,
                            int64_t B, int d, int E, hipStream_t s) {
  const int neb = (E + 31) / 32;
  const int eb = neb >= 8 ? 8 : neb >= 4 ? 4 : neb >= 2 ? 2 : 1;
  int ks = 8 / eb;
  while (ks > 1 && d / ks < 64) ks /= 2;
  const int64_t gy = (neb + eb - 1) / eb;
  int mi = ks >= 8 ? 1 : ks >= 4 ? 2 : 4;  // keeps the K-split partials in registers
  while (mi > 1 && ((B + 32 * mi - 1) / (32 * mi)) * gy < 128) mi /= 2;
  switch (eb * 16 + ks) {
    case 8 * 16 + 1: return launch_gate_mfma_mi<8, 1>(mi, x, Wg, bias, logits, B, d, E, s);
    case 4 * 16 + 2: return launch_gate_mfma_mi<4, 2>(mi, x, Wg, bias, logits, B, d, E, s);
    case 4 * 16 + 1: return launch_gate_mfma_mi<4, 1>(mi, x, Wg, bias, logits, B, d, E, s);
    case 2 * 16 + 4: return launch_gate_mfma_mi<2, 4>(mi, x, Wg, bias, logits, B, d, E, s);
    case 2 * 16 + 2: return launch_gate_mfma_mi<2, 2>(mi, x, Wg, bias, logits, B, d, E, s);
    case 2 * 16 + 1: return launch_gate_mfma_mi<2, 1>(mi, x, Wg, bias, logits, B, d, E, s);
    case 1 * 16 + 8: return launch_gate_mfma_mi<1, 8>(mi, x, Wg, bias, logits, B, d, E, s);
    case 1 * 16 + 4: return launch_gate_mfma_mi<1, 4>(mi, x, Wg, bias, logits, B, d, E, s);
    case 1 * 16 + 2: return launch_gate_mfma_mi<1, 2>(mi, x, Wg, bias, logits, B, d, E, s);
    default: return launch_gate_mfma_mi<1, 1>(mi, x, Wg, bias, logits, B, d, E, s);
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
  if (x_bf16) return launch_gate_mfma(static_cast<const uint16_t*>(x), Wg, bias, logits, B, d, E, s);
  if (E > 32) return launch_gate_t<64, 4>(x, x_bf16, Wg, bias, logits, B, d, E, s);
  if (E > 16) return launch_gate_t<32, 4>(x, x_bf16, Wg, bias, logits, B, d, E, s);
  if (E > 8) return launch_gate_t<16, 2>(x, x_bf16, Wg, bias, logits, B, d, E, s);
  return launch_gate_t<8, 1>(x, x_bf16, Wg, bias, logits, B, d, E, s);
}

}  // namespace moek
