// Grouped expert MLP on bf16 matrix cores (gfx950 MFMA 32x32x16).
//
// "Expert Parallelism" (narrativegoldmine.com), "Components and
// Architecture", Expert GEMM: each expert is a standard transformer MLP run on
// the tokens routed to it, with no communication during the compute phase;
// "Formal Algorithm": the work is proportional to received tokens times the
// expert FFN cost.
//
// Two launches per call, each a grouped GEMM over the experts' contiguous
// packed segments (rows [expert_offset[e], expert_offset[e+1])):
//   GEMM1  H   = act(X . W1^T)               (GELU)   or
//          H   = silu(X . W1^T) * (X . W3^T)  (SwiGLU, both products in one tile)
//   GEMM2  Out = H . W2^T
//
// Weight streaming.  With ~100-2000 rows per expert the GEMMs of the smaller
// workloads are bound by reading the weights from HBM once.  Weights are
// therefore kept in a blocked layout (moe_pack_weights, once per model): for
// every expert, 256-row output tile and 64-wide K stage, one contiguous 32 KB
// block holding the 256 rows' 128-byte K slices in exactly the order (and
// bank swizzle) the tile uses in LDS.  A workgroup streams its tile's blocks
// front to back, so every weight byte is read once, as whole 1 KB DMA
// requests, from consecutive addresses.  Tails (N or K not a multiple of
// 256 / 64) are zero in the blocks, so the MFMAs need no masking.
//
// Tile: 256 rows x 256 output columns (128 for SwiGLU), K stages of 64,
// 8 wavefronts = 2 (rows) x 4 (columns).
//  * One tile row usually covers a whole expert segment (C is 160 / 256 in
//    the HBM-bound workloads); only the 32-row blocks that hold rows run
//    MFMAs (the block count is a template parameter chosen per tile).
//  * Operands move global -> LDS by DMA (global_load_lds_dwordx4, no register
//    staging), NST - 1 stages ahead of the MFMAs, with NST as large as the
//    160 KB LDS allows (2..4).
//  * Each wavefront owns 64 output columns and half of the row blocks:
//    accumulators <= 128 registers, so two wavefronts share each SIMD and hide
//    each other's LDS and barrier latency.
//  * Tiles are numbered so that those sharing an expert's activations land
//    on the same XCD (workgroups are dealt round-robin over the 8 XCDs), so
//    the activation rows are read from HBM once per expert.
#include "moe_kernels.h"

namespace moek {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kThreads = 512;
constexpr int BM = 256;                   // rows per tile
constexpr int BK = 64;                    // K per stage
constexpr int kRowBytes = BK * 2;         // one K slice of a row: 128 B
constexpr int kTileRows = 256;            // weight rows per tile
constexpr int kBStage = kTileRows * kRowBytes;  // 32 KB weight block per stage
constexpr int kLdsBytes = 160 * 1024;
constexpr int kXcd = 8;

enum { MODE_GELU = 0, MODE_SWIGLU = 1, MODE_PLAIN = 2 };

struct GemmArgs {
  const uint16_t* A;         // rows of length K
  const int32_t* eo;         // expert_offset [E+1]
  const uint16_t* Wp;        // blocked weights of this GEMM
  uint16_t* Out;             // rows of length Nout
  int a_local, o_local;      // row index relative to expert_offset[e_begin]
  int e_begin;
  int K, Nout;
  int n_tiles_n, m_tiles, nk, total;
  int per_wg;                // consecutive tiles per workgroup
  int remap;                 // one tile per workgroup, same-expert tiles on one XCD
};

// GELU with the exact-erf definition, 0.5 z (1 + erf(z / sqrt 2)).  erf is
// evaluated with Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (absolute error <= 1.5e-7, far below the bf16 rounding of
// the stored activation): erf(x) = 1 - (a1 t + ... + a5 t^5) e^{-x^2},
// t = 1 / (1 + p x) for x >= 0, odd symmetry for x < 0.  A dozen VALU
// operations instead of a general-purpose erff: the epilogue evaluates it
// once per hidden activation.
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __frcp_rn(fmaf(0.3275911f, ax, 1.0f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float y = 1.0f - p * __expf(-ax * ax);
  return copysignf(y, x);
}
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erf_as7126(z * 0.7071067811865475f));
}
__device__ __forceinline__ float silu_f(float z) { return z * __frcp_rn(1.0f + __expf(-z)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4; lds must be wavefront-uniform).
__device__ __forceinline__ void dma16(const void* g, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds, 16, 0, 0);
}

// wait until at most N vector-memory operations of this wavefront are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Byte offset of 16-byte chunk `ch` of row `r` in a tile of 128-byte rows.
// Chunks are XOR-swizzled by row so that the lanes of one MFMA operand read
// (consecutive rows, same chunk) hit distinct banks: LDS has 64 banks of
// 4 bytes, so a 128-byte row covers half of them (even rows the lower half,
// odd rows the upper) and 16 lanes x 16 bytes are served together; XOR-ing
// the chunk with (r / 2) % 8 spreads 16 consecutive rows over all 64 banks.
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz(int r, int ch) {
  return r * kRowBytes + ((ch ^ swz_key(r)) << 4);
}

// LDS ring for a tile of NS row blocks: each stage holds the activation
// slice (rounded up to whole 64-row DMA rounds) and the 32 KB weight block;
// as many stages as fit in 160 KB, at most 4.
template <int NS>
struct Ring {
  static constexpr int A_ROUNDS = (NS + 1) / 2;
  static constexpr int A_BYTES = A_ROUNDS * 64 * kRowBytes;
  static constexpr int STAGE = A_BYTES + kBStage;
  static constexpr int NST = kLdsBytes / STAGE > 4 ? 4 : kLdsBytes / STAGE;
  static constexpr int LOADS = A_ROUNDS + 4;  // DMA instructions per thread per stage
};

// A run of `ntile` consecutive output tiles (columns n0 .. n0+ntile-1) of one
// expert and one 256-row slice with NS active 32-row blocks, as seen by one
// wavefront that multiplies MI of the row blocks starting at block FIRST.
// Every wavefront runs the same loop (same barriers); MI may be 0.
//
// The run is one continuous pipeline over ntile * nk stages: the prefetch
// for the next tile's first stages is in flight while a tile's last stages
// and its epilogue run, so the weight stream does not stop between tiles.
// The epilogue stores straight from the accumulators (no LDS), pairing
// neighbouring columns across lanes into 4-byte stores.
template <int MODE, int NS, int MI>
__device__ __forceinline__ void gemm_run(const GemmArgs& a, char* __restrict__ smem, int el,
                                         int n0, int ntile, int64_t a_row0, int64_t o_row0,
                                         int rows, int first) {
  using R = Ring<NS>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, lg = lane >> 5;
  const int wn = wave & 3;
  const int K = a.K;
  const int nk = a.nk;
  const int nstage = ntile * nk;

  // DMA lane geometry: in round i the block fills rows 64 i + 8 wave + lane/8,
  // LDS chunk lane % 8, which holds K chunk (lane % 8) ^ swz_key(row) (the
  // key depends only on drow, as 64 i is a multiple of 16).
  const int drow = 8 * wave + (lane >> 3);
  const int dchunk = (lane & 7) ^ swz_key(drow);
  const uint16_t* ap = a.A + a_row0 * K + 8 * dchunk;
  int aoff[R::A_ROUNDS];
#pragma unroll
  for (int i = 0; i < R::A_ROUNDS; ++i) {
    const int r = 64 * i + drow;
    aoff[i] = r < rows ? r : rows - 1;  // rows past the segment: any valid row
  }
  // weight blocks of tile n are (el * n_tiles + n) * nk + kt: consecutive
  // tiles of the run are one contiguous stream
  const char* wblk = reinterpret_cast<const char*>(a.Wp) +
                     (size_t)(el * a.n_tiles_n + n0) * nk * kBStage + drow * kRowBytes +
                     16 * (lane & 7);
  // weight-tile rows of this lane's two MFMA column blocks
  const int jb0 = MODE == MODE_SWIGLU ? wn * 32 + l32 : wn * 64 + l32;
  const int jb1 = MODE == MODE_SWIGLU ? 128 + wn * 32 + l32 : wn * 64 + 32 + l32;

  f32x16 acc0[MI > 0 ? MI : 1], acc1[MI > 0 ? MI : 1];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[i][r] = 0.f;
      acc1[i][r] = 0.f;
    }
  }

  // K chunks past K hold zeros in the weight blocks, so the activation side
  // may load anything finite there: clamp the offset into the row.
#define ISSUE(G, SLOT)                                                             \
  {                                                                                \
    char* st_ = smem + (SLOT) * R::STAGE;                                          \
    const int k0_ = ((G) % nk) * BK;                                               \
    const int ko_ = k0_ + 8 * dchunk < K ? k0_ : K - 8 - 8 * dchunk;               \
    _Pragma("unroll") for (int i_ = 0; i_ < R::A_ROUNDS; ++i_)                     \
      dma16(ap + (int64_t)aoff[i_] * K + ko_, st_ + (64 * i_ + 8 * wave) * kRowBytes); \
    const char* wb_ = wblk + (size_t)(G) * kBStage;                                \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                               \
      dma16(wb_ + i_ * 64 * kRowBytes, st_ + R::A_BYTES + (64 * i_ + 8 * wave) * kRowBytes); \
  }

#pragma unroll
  for (int p = 0; p < R::NST - 1; ++p) ISSUE(p < nstage ? p : nstage - 1, p);

  bool drained = false;  // the previous iteration ended a tile with stores
  for (int g = 0; g < nstage; ++g) {
    // This wavefront's part of stage g has landed.  After an epilogue the
    // vector-memory counter also holds its stores, so wait for everything.
    if (drained)
      wait_vmcnt<0>();
    else
      wait_vmcnt<(R::NST - 2) * R::LOADS>();
    // Everyone's part landed and stage g-1 is consumed (its LDS reads fed
    // MFMAs, so they completed).  A bare s_barrier: __syncthreads() would add
    // a release fence, i.e. wait for *all* outstanding loads -- including the
    // stages prefetched ahead -- and serialize the pipeline.
    __builtin_amdgcn_s_barrier();
    {
      // refill the slot of stage g-1; past the end, reload the last stage
      // (in bounds, never read) so every iteration issues the same count
      const int gn = g + R::NST - 1;
      ISSUE(gn < nstage ? gn : nstage - 1, gn % R::NST);
    }
    drained = false;
    if (MI > 0) {
      __builtin_amdgcn_sched_barrier(0);
      const char* sa = smem + (g % R::NST) * R::STAGE;
      const char* sbt = sa + R::A_BYTES;
      // Operand fragments: each activation fragment is re-read for step s + 1
      // right after the two MFMAs of step s that consume it, and the two
      // weight fragments of step s + 1 at the start of step s, so every LDS
      // read has a whole step of MFMAs to land while only one set of
      // activation fragments is live (the accumulators need the registers).
      u32x4 fa[MI > 0 ? MI : 1], fb[2][2];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = *(const u32x4*)(sa + swz(32 * (first + i) + l32, lg));
      fb[0][0] = *(const u32x4*)(sbt + swz(jb0, lg));
      fb[0][1] = *(const u32x4*)(sbt + swz(jb1, lg));
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_) {
        const int cur = s_ & 1;
        const int chn = 2 * (s_ + 1) + lg;
        if (s_ < 3) {
          fb[cur ^ 1][0] = *(const u32x4*)(sbt + swz(jb0, chn));
          fb[cur ^ 1][1] = *(const u32x4*)(sbt + swz(jb1, chn));
        }
        const bf16x8 b0 = as_bf16x8(fb[cur][0]);
        const bf16x8 b1 = as_bf16x8(fb[cur][1]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const bf16x8 af = as_bf16x8(fa[i]);
          acc0[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b0, acc0[i], 0, 0, 0);
          acc1[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b1, acc1[i], 0, 0, 0);
          if (s_ < 3) fa[i] = *(const u32x4*)(sa + swz(32 * (first + i) + l32, chn));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if ((g % nk) == nk - 1) {
        // Epilogue of tile n0 + g / nk.  acc[i][r] is row 8 (r / 4) + 4 lg +
        // r % 4 of row block first + i, column l32 of its 32-column block.
        // Rows r and r + 1 (r even) are adjacent: lanes 2j and 2j + 1 swap
        // one value so that the even lane writes columns (2j, 2j+1) of row r
        // and the odd lane the same columns of row r + 1, 4 bytes each.
        const int nt = n0 + g / nk;
        const int n_base = MODE == MODE_SWIGLU ? nt * 128 + wn * 32 : nt * 256 + wn * 64;
        const bool odd = lane & 1;
        const int col = n_base + (l32 & ~1);
        // Opaque copy of the row length: without it the compiler hoists every
        // row address of the epilogue out of the tile loop and spills them.
        int nout = a.Nout;
        asm volatile("" : "+s"(nout));
        uint16_t* out = a.Out + o_row0 * nout;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int row = 32 * (first + i) + 8 * (r >> 2) + 4 * lg + (r & 3) + (odd ? 1 : 0);
#pragma unroll
            for (int cb = 0; cb < (MODE == MODE_SWIGLU ? 1 : 2); ++cb) {
              float v0, v1;
              if (MODE == MODE_SWIGLU) {
                v0 = silu_f(acc0[i][r]) * acc1[i][r];
                v1 = silu_f(acc0[i][r + 1]) * acc1[i][r + 1];
              } else {
                v0 = cb == 0 ? acc0[i][r] : acc1[i][r];
                v1 = cb == 0 ? acc0[i][r + 1] : acc1[i][r + 1];
                if (MODE == MODE_GELU) {
                  v0 = gelu_erf(v0);
                  v1 = gelu_erf(v1);
                }
              }
              const float send = odd ? v0 : v1;
              const float got = __shfl_xor(send, 1);
              const float lo = odd ? got : v0;  // column col
              const float hi = odd ? v1 : got;  // column col + 1
              const int c = col + 32 * cb;
              if (row < rows && c < nout)
                *(unsigned int*)(out + (row * nout + c)) = pack_bf16x2(lo, hi);
              // one pair at a time: keeps the epilogue's temporaries from
              // piling up next to the live accumulators
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc0[i][r] = 0.f;
            acc1[i][r] = 0.f;
          }
        }
        drained = true;
      }
    } else if ((g % nk) == nk - 1) {
      drained = true;
    }
  }
#undef ISSUE
  wait_vmcnt<0>();
  __syncthreads();
}

// Row blocks are split between the two wavefront rows: the first takes
// ceil(NS / 2) blocks, the second the rest.
template <int MODE, int NS>
__device__ __forceinline__ void gemm_tiles(const GemmArgs& a, char* smem, int el, int n0,
                                           int ntile, int64_t a_row0, int64_t o_row0, int rows) {
  if ((threadIdx.x >> 8) == 0)
    gemm_run<MODE, NS, (NS + 1) / 2>(a, smem, el, n0, ntile, a_row0, o_row0, rows, 0);
  else
    gemm_run<MODE, NS, NS / 2>(a, smem, el, n0, ntile, a_row0, o_row0, rows, (NS + 1) / 2);
}

// Persistent over a contiguous range of tiles (expert-major, then row slice,
// then output tile).  Consecutive tiles of one expert and row slice are one
// pipelined run; the weight blocks of a run are contiguous in memory.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  int t0, t1;
  if (a.remap) {
    // one tile each: consecutive tiles (same expert) on the same XCD, which
    // then reads that expert's activation rows from HBM once
    const int bid = blockIdx.x;
    const int per = a.total / kXcd;
    t0 = bid < per * kXcd ? (bid % kXcd) * per + bid / kXcd : bid;
    t1 = t0 + 1;
  } else {
    t0 = blockIdx.x * a.per_wg;
    t1 = t0 + a.per_wg < a.total ? t0 + a.per_wg : a.total;
  }
  const int loc = a.eo[a.e_begin];
  for (int t = t0; t < t1;) {
    const int n_t = t % a.n_tiles_n;
    const int em = t / a.n_tiles_n;  // expert and row slice
    const int m_t = em % a.m_tiles;
    const int el = em / a.m_tiles;
    const int run = (t1 - t < a.n_tiles_n - n_t) ? t1 - t : a.n_tiles_n - n_t;
    t += run;
    const int e = a.e_begin + el;
    const int rb = a.eo[e];
    const int M = a.eo[e + 1] - rb;
    const int m0 = m_t * BM;
    if (m0 >= M) continue;
    const int64_t a_row0 = (int64_t)(rb - (a.a_local ? loc : 0) + m0);
    const int64_t o_row0 = (int64_t)(rb - (a.o_local ? loc : 0) + m0);
    const int rows = M - m0 < BM ? M - m0 : BM;
    switch ((rows + 31) >> 5) {
      case 1: gemm_tiles<MODE, 1>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 2: gemm_tiles<MODE, 2>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 3: gemm_tiles<MODE, 3>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 4: gemm_tiles<MODE, 4>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 5: gemm_tiles<MODE, 5>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 6: gemm_tiles<MODE, 6>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 7: gemm_tiles<MODE, 7>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      default: gemm_tiles<MODE, 8>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
    }
  }
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// One workgroup per CU (the LDS ring takes all 160 KB).  A launch with no
// more tiles than CUs gives each workgroup one tile and groups an expert's
// tiles on one XCD; a larger one hands each workgroup a contiguous range.
template <int MODE>
hipError_t launch_gemm(GemmArgs g, hipStream_t s) {
  if (g.total <= 0) return hipSuccess;
  const int cus = device_cus();
  int grid;
  if (g.total <= cus) {
    g.remap = 1;
    g.per_wg = 1;
    grid = g.total;
  } else {
    g.remap = 0;
    g.per_wg = (g.total + cus - 1) / cus;
    grid = (g.total + g.per_wg - 1) / g.per_wg;
  }
  hipLaunchKernelGGL(grouped_gemm_kernel<MODE>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

// Blocked weight layout: for expert e, output tile nt, stage kt, one 32 KB
// block of 256 rows x 8 chunks of 16 B; chunk p of row j holds K chunk
// p ^ swz_key(j) of the row's weight-matrix row (zeros past N or K).  Row j is
// weight row nt*256 + j (GELU, plain), or W1 row nt*128 + j for j < 128 and
// W3 row nt*128 + j - 128 otherwise (SwiGLU).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ W0,
                                                           const uint16_t* __restrict__ W1,
                                                           int n_exp, int Nw, int K, int n_tiles,
                                                           int nk, int swiglu,
                                                           uint16_t* __restrict__ out) {
  const int64_t total = (int64_t)n_exp * n_tiles * nk * kTileRows * 8;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int p = (int)(q & 7);
    const int j = (int)((q >> 3) & (kTileRows - 1));
    int64_t rest = q >> 11;
    const int kt = (int)(rest % nk);
    rest /= nk;
    const int nt = (int)(rest % n_tiles);
    const int e = (int)(rest / n_tiles);
    const int k = kt * BK + 8 * (p ^ swz_key(j));
    int n;
    const uint16_t* src;
    if (swiglu) {
      n = nt * 128 + (j & 127);
      src = j < 128 ? W0 : W1;
    } else {
      n = nt * 256 + j;
      src = W0;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < Nw && k < K) v = *(const u32x4*)(src + ((int64_t)e * Nw + n) * K + k);
    *(u32x4*)(out + q * 8) = v;
  }
}

struct Geo {
  int n_tiles, nk;
  size_t bytes;
};
Geo geo(int n_local, int N, int K, bool swiglu) {
  Geo g;
  g.n_tiles = swiglu ? (N + 127) / 128 : (N + 255) / 256;
  g.nk = (K + BK - 1) / BK;
  g.bytes = (size_t)n_local * g.n_tiles * g.nk * kBStage;
  return g;
}

}  // namespace

size_t packed_weights_bytes(int n_local, int d, int f, bool swiglu) {
  return geo(n_local, f, d, swiglu).bytes + geo(n_local, d, f, false).bytes;
}

hipError_t launch_pack_weights(const uint16_t* W1, const uint16_t* W3, const uint16_t* W2,
                               int n_local, int d, int f, bool swiglu, void* wp, hipStream_t s) {
  if (n_local <= 0) return hipSuccess;
  const Geo g1 = geo(n_local, f, d, swiglu), g2 = geo(n_local, d, f, false);
  uint16_t* o1 = static_cast<uint16_t*>(wp);
  uint16_t* o2 = reinterpret_cast<uint16_t*>(static_cast<char*>(wp) + g1.bytes);
  auto blocks = [](size_t bytes) {
    int64_t g = (int64_t)(bytes / 16 + 255) / 256;
    return (unsigned)(g > (1 << 20) ? (1 << 20) : g);
  };
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks(g1.bytes)), dim3(256), 0, s, W1,
                     swiglu ? W3 : nullptr, n_local, f, d, g1.n_tiles, g1.nk, swiglu ? 1 : 0, o1);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks(g2.bytes)), dim3(256), 0, s, W2, nullptr,
                     n_local, d, f, g2.n_tiles, g2.nk, 0, o2);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const uint16_t* packed, const int32_t* expert_offset, int e_begin,
                             int n_local, int rows_max, int d, int f, bool swiglu, const void* wp,
                             uint16_t* H, uint16_t* ret, hipStream_t s) {
  if (n_local <= 0 || rows_max <= 0) return hipSuccess;
  const int m_tiles = (rows_max + BM - 1) / BM;
  const Geo geo1 = geo(n_local, f, d, swiglu), geo2 = geo(n_local, d, f, false);
  GemmArgs g1{};
  g1.A = packed;
  g1.eo = expert_offset;
  g1.Wp = static_cast<const uint16_t*>(wp);
  g1.Out = H;
  g1.a_local = 0;
  g1.o_local = 1;
  g1.e_begin = e_begin;
  g1.K = d;
  g1.Nout = f;
  g1.n_tiles_n = geo1.n_tiles;
  g1.nk = geo1.nk;
  g1.m_tiles = m_tiles;
  g1.total = n_local * m_tiles * g1.n_tiles_n;
  hipError_t err = swiglu ? launch_gemm<MODE_SWIGLU>(g1, s) : launch_gemm<MODE_GELU>(g1, s);
  if (err != hipSuccess) return err;

  GemmArgs g2{};
  g2.A = H;
  g2.eo = expert_offset;
  g2.Wp = reinterpret_cast<const uint16_t*>(static_cast<const char*>(wp) + geo1.bytes);
  g2.Out = ret;
  g2.a_local = 1;
  g2.o_local = 0;
  g2.e_begin = e_begin;
  g2.K = f;
  g2.Nout = d;
  g2.n_tiles_n = geo2.n_tiles;
  g2.nk = geo2.nk;
  g2.m_tiles = m_tiles;
  g2.total = n_local * m_tiles * g2.n_tiles_n;
  return launch_gemm<MODE_PLAIN>(g2, s);
}

}  // namespace moek
