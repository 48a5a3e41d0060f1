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
//   operands = x rows staged in LDS by DMA, shared by the EB waves of a K
//              range; weights straight from global memory into registers
//              (the lane's expert column, 8 k per step), split there; or,
//              in moe_forward, from a copy of the weights made at the start
//              of the call: their bf16 parts in the lanes' order (the split
//              copy), or the fp32 values in the lanes' order (the blocked
//              copy: two 16-byte loads per step instead of eight 4-byte
//              ones)
//
// fp32 activations: the vector ALUs (a block owns BT tokens x BE experts;
// four waves split each 128-wide slice of d; blocked accumulation keeps the
// fp32 error near sqrt(32) + sqrt(d/32) roundings; the four wave totals are
// added in a fixed order).
#include "launch.h"
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

// Router weights split once per call into the layout the gate's MFMAs read:
// for expert block eb (32 experts), K step ks (16 k) and part p (0: lo,
// 1: mid, 2: hi), 64 lanes x 16 bytes; lane l holds the 8 bf16 parts of
// k = 16 ks + 8 (l / 32) .. +7 of expert 32 eb + l % 32 (zeros past d or E).
// One thread per (eb, ks, lane).
__global__ __launch_bounds__(256) void gate_split_kernel(const float* __restrict__ Wg, int d,
                                                         int E, int neb, int nks,
                                                         u32x4* __restrict__ out) {
  const int64_t n = (int64_t)neb * nks * 64;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int lane = (int)(i & 63);
    const int64_t bk = i >> 6;  // eb * nks + ks
    const int ks = (int)(bk % nks), eb = (int)(bk / nks);
    const int e = 32 * eb + (lane & 31);
    const int k0 = 16 * ks + 8 * (lane >> 5);
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (e < E && k0 + q < d) ? Wg[(int64_t)(k0 + q) * E + e] : 0.f;
    u32x4 hi, mid, lo;
    split3(v, hi, mid, lo);
    out[(bk * 3 + 0) * 64 + lane] = lo;
    out[(bk * 3 + 1) * 64 + lane] = mid;
    out[(bk * 3 + 2) * 64 + lane] = hi;
  }
}

// Blocked fp32 copy of the router weights, in the order the gate's lanes
// load them: for expert block eb (32 experts) and K step ks (16 k), 64 lanes
// x 32 bytes as two 1 KB halves -- half hf of lane l holds k = 16 ks +
// 8 (l / 32) + 4 hf .. +3 of expert 32 eb + l % 32 (zeros past d or E).
// One thread per (eb, ks, lane).
__global__ __launch_bounds__(256) void gate_block_kernel(const float* __restrict__ Wg, int d,
                                                         int E, int neb, int nks,
                                                         f32x4* __restrict__ out) {
  const int64_t n = (int64_t)neb * nks * 64;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int lane = (int)(i & 63);
    const int64_t bk = i >> 6;  // eb * nks + ks
    const int ks = (int)(bk % nks), eb = (int)(bk / nks);
    const int e = 32 * eb + (lane & 31);
    const int k0 = 16 * ks + 8 * (lane >> 5);
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (e < E && k0 + q < d) ? Wg[(int64_t)(k0 + q) * E + e] : 0.f;
    out[(bk * 2 + 0) * 64 + lane] = f32x4{v[0], v[1], v[2], v[3]};
    out[(bk * 2 + 1) * 64 + lane] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// The token rows are staged once per block in LDS, shared by the EB waves
// of one K range.  Stages of 64 k; a 3-slot ring filled by DMA
// (buffer_load_dwordx4 ... lds, rows bank-swizzled) two stages ahead; the
// lane's weight column (8 k per MFMA step) prefetched two stages ahead in
// registers and split there, or its three bf16 parts loaded as they are
// from the split copy (gate_split_kernel: 3 16-byte loads per step instead
// of 8 4-byte loads and the split), or its 8 fp32 values loaded from the
// blocked copy (gate_block_kernel: 2 16-byte loads) and split there.
enum GateW { kWDirect = 0, kWSplit = 1, kWBlock = 2 };
typedef __attribute__((address_space(3))) void g_lds_void_t;

template <int N>
__device__ __forceinline__ void g_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// 16 bytes per lane from byte offset off of the buffer [base, base + bytes)
// into LDS at lds + 16 * lane (buffer_load_dwordx4 ... lds).  The descriptor
// is built here, not in the kernel body: a kernel with a local of the
// descriptor type gets no host-side launch stub.
// lds: a 32-bit LDS offset (a generic pointer would cost a null check per load)
__device__ __forceinline__ void g_dma16(const void* base, uint32_t bytes, uint32_t off, uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), (g_lds_void_t*)(uintptr_t)lds, 16, off,
                                           0, 0, 0);
}
__device__ __forceinline__ int g_swz(int r, int ch) { return r * 128 + ((ch ^ ((r >> 1) & 7)) << 4); }

// The MFMA steps of one 64-k stage: sa = the stage's rows in LDS (this K
// range's slot), the lane's weights for the stage as the copy's 16-byte
// parts (wq) or as fp32 values (wv).
template <int MI, int WM, int NP>
__device__ __forceinline__ void gl_mul(g_f32x16 (&acc)[MI], const char* sa, const u32x4 (&wq)[4][NP],
                                       const float (&wv)[4][8], int l32, int h) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 hi, mid, lo;
    if constexpr (WM == kWSplit) {
      lo = wq[j][0];
      mid = wq[j][1];
      hi = wq[j][2];
    } else if constexpr (WM == kWBlock) {
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[q] = __uint_as_float(wq[j][0][q]);
        f[4 + q] = __uint_as_float(wq[j][NP - 1][q]);
      }
      split3(f, hi, mid, lo);
    } else {
      split3(wv[j], hi, mid, lo);
    }
    // the three products of a row block accumulate into one register set,
    // so the parts go round the row blocks (lo of every block, then mid,
    // then hi): consecutive matrix instructions are independent whenever
    // MI > 1, and each accumulator still adds lo, mid, hi in that order
    g_bf16x8 a[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[i] = __builtin_bit_cast(g_bf16x8, *(const u32x4*)(sa + g_swz(32 * i + l32, 2 * j + h)));
#pragma unroll
    for (int i = 0; i < MI; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], __builtin_bit_cast(g_bf16x8, lo), acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < MI; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], __builtin_bit_cast(g_bf16x8, mid), acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < MI; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], __builtin_bit_cast(g_bf16x8, hi), acc[i], 0, 0, 0);
  }
}

template <int MI, int EB, int KS, int WM>
__global__ __launch_bounds__(64 * EB * KS) void gate_lds_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ Wg, const u32x4* __restrict__ Wsp,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t B, int d, int E) {
  extern __shared__ __attribute__((aligned(16))) char gsm[];
  const uint32_t gsm_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)gsm;
  constexpr int SLOT = 32 * MI * 128;  // one stage (64 k) of the block's rows
  constexpr int NSL = 3;
  constexpr int ND = 4 * MI / EB;      // DMA instructions per wave per stage
  static_assert(ND >= 1 && ND * EB == 4 * MI, "rows split evenly over the expert waves");
  constexpr bool PS = WM != kWDirect;  // weights from a copy in the lanes' order
  constexpr int NP = WM == kWSplit ? 3 : 2;  // 16-byte loads per lane and MFMA step
  constexpr int LOADS = (PS ? 4 * NP : 32) + ND;  // vector-memory loads per wave per stage
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int eb = w % EB, kq = w / EB;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * (32 * MI);
  const int e0 = (blockIdx.y * EB + eb) * 32;
  const int kspan = (d + 64 * KS - 1) / (64 * KS) * 64;
  const int kb = kq * kspan;
  const int ke = kb + kspan < d ? kb + kspan : d;
  const int nst = kspan / 64;  // the same for every wave (barriers)

  // DMA: instruction q covers rows 8 (eb + EB q) .. +7; lane -> row + lane / 8,
  // LDS chunk lane % 8 holding K chunk (lane % 8) ^ key(row)
  // the block's rows as one buffer (byte offsets are 32-bit)
  const int nrows = B - t0 < 32 * MI ? (int)(B - t0) : 32 * MI;
  const uint16_t* xblk = x + t0 * d;
  const uint32_t xbytes = 2u * (uint32_t)nrows * (uint32_t)d;
  uint32_t xrow[ND];
  int dcol[ND], dofs[ND];
#pragma unroll
  for (int q = 0; q < ND; ++q) {
    const int row = 8 * (eb + EB * q) + (lane >> 3);
    const int r = row < nrows ? row : nrows - 1;  // past B: any valid row, never stored
    xrow[q] = 2u * (uint32_t)r * (uint32_t)d;
    dcol[q] = 8 * ((lane & 7) ^ ((row >> 1) & 7));
    dofs[q] = kq * SLOT + 8 * (eb + EB * q) * 128;
  }
  // weight loads go through buffer descriptors over the wavefront's own K
  // range, so K steps past it read zeros: no select on a loaded value (which
  // would make the compiler wait for the load there and undo the prefetch)
  const int ec = e0 + l32 < E ? e0 + l32 : E - 1;  // past E: any valid column, never stored

  g_f32x16 acc[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float wv[PS ? 1 : NSL][4][8];
  u32x4 wq[PS ? NSL : 1][4][NP];
  // PS: this wavefront's expert block in the copy, and its first K step.
  // The copy holds neb = ceil(E / 32) blocks; a wavefront whose block lies
  // past them (the last row of the grid when EB does not divide neb) reads
  // the last block instead -- in bounds, and its results are never stored
  // (e >= E below).
  // Likewise a K range that starts past d (more K ranges than d needs)
  // reads no step of its own: its base is clamped to the block's last step.
  const int nks = (d + 15) / 16;
  const int neb = (E + 31) / 32;
  const int ebs = (int)blockIdx.y * EB + eb < neb ? (int)blockIdx.y * EB + eb : neb - 1;
  const int kb16 = kb / 16 < nks ? kb / 16 : nks - 1;
  // PS: the copy's K steps kb / 16 .. ceil(ke / 16) of this expert block
  const int nvalid = ke > kb ? (ke - kb + 15) / 16 : 0;
  const rsrc_t wrs =
      PS ? make_rsrc(Wsp + ((int64_t)ebs * nks + kb16) * NP * 64, (uint32_t)nvalid * NP * 1024u)
         : make_rsrc(Wg + (int64_t)kb * E, 4u * (uint32_t)(ke > kb ? ke - kb : 0) * (uint32_t)E);

  // stage s (clamped to the last one): weights, then rows.  K chunks past
  // the end of the row read the row's last chunk; their weights are zero.
#define GL_ISSUE(S, B_)                                                              \
  {                                                                                  \
    const int sc_ = (S) < nst ? (S) : nst - 1;                                       \
    if constexpr (PS) {                                                              \
      /* steps past the wave's K range lie past the descriptor: zeros */             \
      _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_)                               \
        _Pragma("unroll") for (int p_ = 0; p_ < NP; ++p_)                            \
          wq[B_][j_][p_] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128( \
              wrs, (uint32_t)(((4 * sc_ + j_) * NP + p_) * 64 + lane) * 16u, 0, 0));  \
    } else {                                                                         \
      /* rows k >= ke lie past the descriptor: zeros */                              \
      _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_) {                             \
        const uint32_t r_ = (uint32_t)(64 * sc_ + 16 * j_ + 8 * h);                  \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_)                             \
          wv[B_][j_][i_] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(     \
              wrs, ((r_ + i_) * (uint32_t)E + (uint32_t)ec) * 4u, 0, 0));            \
      }                                                                              \
    }                                                                                \
    const int kx_ = kb + 64 * sc_;                                                   \
    const uint32_t sl_ = gsm_lds + ((S) % NSL) * KS * SLOT;                          \
    _Pragma("unroll") for (int q_ = 0; q_ < ND; ++q_) {                              \
      const int kk_ = kx_ + dcol[q_];                                                \
      g_dma16(xblk, xbytes, xrow[q_] + 2u * (kk_ < d ? kk_ : d - 8), sl_ + dofs[q_]); \
    }                                                                                \
  }
  // one stage: wait for stage s (at most one stage's loads left in flight),
  // barrier, issue stage s + 2 into the slot stage s - 1 used, multiply
#define GL_STAGE(S, U)                                                               \
  {                                                                                  \
    g_wait_vmcnt<LOADS>();                                                           \
    __builtin_amdgcn_s_barrier();                                                    \
    GL_ISSUE((S) + 2, ((U) + 2) % NSL)                                               \
    __builtin_amdgcn_sched_barrier(0);                                               \
    gl_mul<MI, WM, NP>(acc, gsm + ((S) % NSL) * KS * SLOT + kq * SLOT, wq[(U) % NSL_Q], \
                       wv[(U) % NSL_V], l32, h);                                     \
  }
  constexpr int NSL_Q = PS ? NSL : 1, NSL_V = PS ? 1 : NSL;
  GL_ISSUE(0, 0)
  GL_ISSUE(1, 1)
  // whole groups of NSL stages, then the remainder: no condition inside the
  // unrolled group, so the compiler can see which loads each step waits for
  // (with one, its own waits fall back to nearly every load in flight)
  const int nfull = nst - nst % NSL;
  for (int s0 = 0; s0 < nfull; s0 += NSL) {
#pragma unroll
    for (int u = 0; u < NSL; ++u) GL_STAGE(s0 + u, u)
  }
  if (nst - nfull > 0) GL_STAGE(nfull, 0)
  if (nst - nfull > 1) GL_STAGE(nfull + 1, 1)
#undef GL_STAGE
#undef GL_ISSUE
  g_wait_vmcnt<0>();
  __syncthreads();

  // acc[i][r] is token t0 + 32 i + 8 (r / 4) + 4 h + r % 4, expert e0 + l32;
  // the K-range partials are added in a fixed order through LDS (the ring's
  // space, now free)
  float* red = reinterpret_cast<float*>(gsm);
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
hipError_t launch_gate_mfma_t(const uint16_t* x, const float* Wg, const u32x4* wsp, int wm,
                              const float* bias, float* logits, int64_t B, int d, int E,
                              hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int neb = (E + 31) / 32;
  dim3 grid((unsigned)((B + 32 * MI - 1) / (32 * MI)), (unsigned)((neb + EB - 1) / EB));
  const size_t lds = (size_t)EB * (KS - 1) * MI * 16 * 64 * sizeof(float);
  const size_t ring = (size_t)3 * KS * 32 * MI * 128;
  const size_t sh = lds > ring ? lds : ring;
  if (wm == kWSplit)
    launch_timed((gate_lds_kernel<MI, EB, KS, kWSplit>), grid, dim3(64 * EB * KS), sh, s, e0, e1,
                 x, Wg, wsp, bias, logits, B, d, E);
  else if (wm == kWBlock)
    launch_timed((gate_lds_kernel<MI, EB, KS, kWBlock>), grid, dim3(64 * EB * KS), sh, s, e0, e1,
                 x, Wg, wsp, bias, logits, B, d, E);
  else
    launch_timed((gate_lds_kernel<MI, EB, KS, kWDirect>), grid, dim3(64 * EB * KS), sh, s, e0,
                 e1, x, Wg, wsp, bias, logits, B, d, E);
  return hipGetLastError();
}

// MI as the launcher picks it: at most 8 / KS row blocks of 32 (the K-split
// partials stay in registers), at least 2 when EB = 8 (4 MI row groups of 8
// shared by the EB waves); only those shapes are compiled.
template <int EB, int KS>
hipError_t launch_gate_mfma_mi(int mi, const uint16_t* x, const float* Wg, const u32x4* wsp,
                               int wm, const float* bias, float* logits, int64_t B, int d, int E,
                               hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int MI_MAX = KS >= 8 ? 1 : KS >= 4 ? 2 : 4;
  constexpr int MI_MIN = EB >= 8 ? 2 : 1;
  if constexpr (MI_MAX >= 4)
    if (mi >= 4) return launch_gate_mfma_t<4, EB, KS>(x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
  if constexpr (MI_MAX >= 2)
    if (mi >= 2 || MI_MIN >= 2)
      return launch_gate_mfma_t<2, EB, KS>(x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
  if constexpr (MI_MIN <= 1)
    return launch_gate_mfma_t<1, EB, KS>(x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
  return hipErrorInvalidValue;
}

// Block shape: up to 8 waves; EB expert blocks (up to 256 experts share the
// x rows), the rest of the 8 waves split K while each wave keeps >= 64 k;
// token tiles (at most 8 / KS row blocks) shrink until there are >= 128
// blocks.  (Token tiles smaller than that would multiply the weight reads,
// which bound these launches.)
struct GatePlan {
  int eb, ks, mi;
  int64_t blocks;
};
// Workgroup shape (bf16 x); split: the router weights come as the split copy.
GatePlan gate_plan(int64_t B, int d, int E, bool split) {
  const int neb = (E + 31) / 32;
  GatePlan g;
  g.eb = neb >= 8 ? 8 : neb >= 4 ? 4 : neb >= 2 ? 2 : 1;
  // Two or three expert blocks and too few token tiles to give every CU a
  // workgroup (at 32 tokens per tile): one expert block per workgroup, so
  // the x rows are read once per expert block but the grid doubles and each
  // wavefront's K range halves (the launch is latency-bound, not bandwidth-
  // bound, at these sizes).
  if (g.eb == 2 && ((B + 31) / 32) * ((neb + 1) / 2) < 256) g.eb = 1;
  g.ks = 8 / g.eb;
  while (g.ks > 1 && d / g.ks < 64) g.ks /= 2;
  const int64_t gy = (neb + g.eb - 1) / g.eb;
  g.mi = g.ks >= 8 ? 1 : g.ks >= 4 ? 2 : 4;  // keeps the K-split partials in registers
  const int mi_min = g.eb >= 8 ? 2 : 1;      // 4 MI row groups of 8 shared by EB waves
  if (g.mi < mi_min) g.mi = mi_min;
  // with the split copy the per-workgroup weight work is cheap enough to
  // give every CU a workgroup
  const int64_t want = split ? 256 : 128;
  while (g.mi > mi_min && ((B + 32 * g.mi - 1) / (32 * g.mi)) * gy < want) g.mi /= 2;
  g.blocks = ((B + 32 * g.mi - 1) / (32 * g.mi)) * gy;
  return g;
}

hipError_t launch_gate_mfma(const uint16_t* x, const float* Wg, const u32x4* wsp, int wm,
                            const float* bias, float* logits, int64_t B, int d, int E,
                            hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const GatePlan g = gate_plan(B, d, E, wm == kWSplit);
  const int eb = g.eb, ks = g.ks, mi = g.mi;
  switch (eb * 16 + ks) {
    case 8 * 16 + 1: return launch_gate_mfma_mi<8, 1>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 4 * 16 + 2: return launch_gate_mfma_mi<4, 2>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 4 * 16 + 1: return launch_gate_mfma_mi<4, 1>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 2 * 16 + 4: return launch_gate_mfma_mi<2, 4>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 2 * 16 + 2: return launch_gate_mfma_mi<2, 2>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 2 * 16 + 1: return launch_gate_mfma_mi<2, 1>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 1 * 16 + 8: return launch_gate_mfma_mi<1, 8>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 1 * 16 + 4: return launch_gate_mfma_mi<1, 4>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    case 1 * 16 + 2: return launch_gate_mfma_mi<1, 2>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
    default: return launch_gate_mfma_mi<1, 1>(mi, x, Wg, wsp, wm, bias, logits, B, d, E, s, e0, e1);
  }
}

template <int BE, int TM>
hipError_t launch_gate_t(const void* x, bool x_bf16, const float* Wg, const float* bias,
                         float* logits, int64_t B, int d, int E, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  constexpr int BT = (kWave / (BE / 4)) * TM;
  dim3 grid((unsigned)((B + BT - 1) / BT), (unsigned)((E + BE - 1) / BE));
  if (x_bf16)
    launch_timed((gate_kernel<BE, TM, true>), grid, dim3(kGateThreads), 0, s, e0, e1,
                 x, Wg, bias, logits, B, d, E);
  else
    launch_timed((gate_kernel<BE, TM, false>), grid, dim3(kGateThreads), 0, s, e0, e1,
                 x, Wg, bias, logits, B, d, E);
  return hipGetLastError();
}

}  // namespace

size_t gate_split_bytes(int d, int E) {
  return (size_t)((E + 31) / 32) * ((d + 15) / 16) * 3 * 1024;
}
size_t gate_block_bytes(int d, int E) {
  return (size_t)((E + 31) / 32) * ((d + 15) / 16) * 2 * 1024;
}

// Exclusive end (bytes) of what gate_lds_kernel reads from the weight copy
// the forward would use at (B, d, E) (split: 3 parts per step, blocked: 2),
// walking the launch the plan gives: every workgroup row, wavefront expert
// block and K range, every stage and MFMA step, with the kernel's own index
// arithmetic.
int64_t gate_split_read_end(int64_t B, int d, int E) {
  const bool split = gate_use_split(true, B, d, E);
  const int np = split ? 3 : 2;
  const GatePlan g = gate_plan(B, d, E, split);
  const int neb = (E + 31) / 32, nks = (d + 15) / 16;
  const int64_t gy = (neb + g.eb - 1) / g.eb;
  const int kspan = (d + 64 * g.ks - 1) / (64 * g.ks) * 64;
  const int nst = kspan / 64;
  int64_t end = 0;
  for (int64_t by = 0; by < gy; ++by)
    for (int eb = 0; eb < g.eb; ++eb)
      for (int kq = 0; kq < g.ks; ++kq) {
        const int kb = kq * kspan, ke = kb + kspan < d ? kb + kspan : d;
        const int ebs = by * g.eb + eb < neb ? (int)(by * g.eb + eb) : neb - 1;
        const int kb16 = kb / 16 < nks ? kb / 16 : nks - 1;
        const int64_t base = ((int64_t)ebs * nks + kb16) * np * 64;
        for (int sc = 0; sc < nst; ++sc)
          for (int j = 0; j < 4; ++j) {
            const bool ok = kb + 64 * sc + 16 * j < ke;
            const int64_t st = ok ? (int64_t)(4 * sc + j) * np * 64 : 0;
            const int64_t last = base + st + (np - 1) * 64 + 63;  // last part, lane 63
            if (16 * (last + 1) > end) end = 16 * (last + 1);
          }
      }
  return end;
}

bool gate_use_split(bool x_bf16, int64_t B, int d, int E) {
  // The split copy costs a launch and 1.5x the weight bytes per workgroup;
  // it pays where it lets the grid fill the CUs (smaller token tiles, the
  // weight split no longer repeated by every workgroup): 16384 tokens x 128
  // experts, 128 -> 256 workgroups, gate 55 -> 45 us.  Where the grid is
  // full already it does not (EP share: 374 -> 398 us), nor for small
  // problems (4096 tokens x 64 experts).
  if (!x_bf16 || B * E < ((int64_t)1 << 20)) return false;
  return gate_plan(B, d, E, false).blocks < 256 && gate_plan(B, d, E, true).blocks > 128;
}

// The blocked fp32 copy: the same bytes per workgroup as reading Wg itself,
// in two 16-byte loads per MFMA step instead of eight 4-byte ones.  Worth its
// launch on large gates (EP share: 256 workgroups that each read all of
// Wg); small ones keep the direct loads.
bool gate_use_block(bool x_bf16, int64_t B, int d, int E) {
  return x_bf16 && !gate_use_split(x_bf16, B, d, E) && B * E >= ((int64_t)1 << 22) && d >= 64;
}

size_t gate_copy_bytes(bool x_bf16, int64_t B, int d, int E) {
  if (gate_use_split(x_bf16, B, d, E)) return gate_split_bytes(d, E);
  if (gate_use_block(x_bf16, B, d, E)) return gate_block_bytes(d, E);
  return 0;
}

hipError_t launch_gate(const void* x, bool x_bf16, const float* Wg, const float* bias,
                       float* logits, int64_t B, int d, int E, void* wsplit, hipStream_t s,
                       hipEvent_t e0, hipEvent_t e1) {
  if (B == 0) return hipSuccess;
  int wm = kWDirect;
  if (x_bf16 && wsplit) {
    const int neb = (E + 31) / 32, nks = (d + 15) / 16;
    const int64_t n = (int64_t)neb * nks * 64;
    const int64_t g = (n + 255) / 256;
    const dim3 grid((unsigned)(g < 65536 ? g : 65536));
    // the start event goes with the first of the two launches
    if (gate_use_split(x_bf16, B, d, E)) {
      wm = kWSplit;
      launch_timed(gate_split_kernel, grid, dim3(256), 0, s, e0, nullptr, Wg, d, E, neb, nks,
                   static_cast<u32x4*>(wsplit));
    } else {
      wm = kWBlock;
      launch_timed(gate_block_kernel, grid, dim3(256), 0, s, e0, nullptr, Wg, d, E, neb, nks,
                   static_cast<f32x4*>(wsplit));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e0 = nullptr;
  }
  if (x_bf16)
    return launch_gate_mfma(static_cast<const uint16_t*>(x), Wg, static_cast<const u32x4*>(wsplit),
                            wm, bias, logits, B, d, E, s, e0, e1);
  if (E > 32) return launch_gate_t<64, 4>(x, x_bf16, Wg, bias, logits, B, d, E, s, e0, e1);
  if (E > 16) return launch_gate_t<32, 4>(x, x_bf16, Wg, bias, logits, B, d, E, s, e0, e1);
  if (E > 8) return launch_gate_t<16, 2>(x, x_bf16, Wg, bias, logits, B, d, E, s, e0, e1);
  return launch_gate_t<8, 1>(x, x_bf16, Wg, bias, logits, B, d, E, s, e0, e1);
}

}  // namespace moek
