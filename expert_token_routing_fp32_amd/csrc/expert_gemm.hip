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
//   GEMM1  H   = act(X . W1^T)              (GELU)   or
//          H   = silu(X . W1^T) * (X . W3^T) (SwiGLU, both products in one tile)
//   GEMM2  Out = H . W2^T
// with W stored output-major ([N][K], the contraction index contiguous), so
// both operands of every MFMA are read along K.
//
// Tile: 256 rows x 256 output columns (128 for SwiGLU), K stages of 64.
//  * The rows of one expert are usually <= 256 (C is 160 / 256 / 1280 / 2048 in
//    the workloads), so one tile row covers the whole segment and every weight
//    byte is fetched from HBM once.  Only the 32-row blocks that hold rows run
//    MFMAs; the rest are skipped with a wavefront-uniform branch.
//  * The activation tile (256 x 64 bf16 = 32 KB) is shared by the four
//    wavefronts through LDS, double buffered, 16-byte chunks XOR-swizzled by
//    row so that the 32 lanes reading one MFMA operand hit distinct banks.
//  * Each wavefront owns 64 output columns (two 32-column MFMA blocks) and
//    reads its weight fragments straight from global memory into registers in
//    the MFMA operand layout (lane = column, 8 contiguous k): nothing else
//    reads them, so LDS would only add a copy.  The next stage is in flight
//    while the current one computes.
//  * Accumulators: 2 column blocks x 8 row blocks x 16 fp32 = 256 per lane,
//    one wavefront per SIMD; latency is hidden by the explicit prefetch.
//  * Tiles are numbered so that those sharing an expert's activations land
//    on the same XCD (workgroups are dealt round-robin over the 8 XCDs), so
//    the activation rows are read once per L2.
#include "moe_kernels.h"

namespace moek {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = 256;
constexpr int BK = 64;
constexpr int MSUB = BM / 32;
constexpr int kXcd = 8;

enum { MODE_GELU = 0, MODE_SWIGLU = 1, MODE_PLAIN = 2 };

struct GemmArgs {
  const uint16_t* A;         // rows of length K
  const int32_t* eo;         // expert_offset [E+1]
  const uint16_t* W0;        // [n_exp][Nw][K]
  const uint16_t* W1;        // [n_exp][Nw][K] (SwiGLU second matrix) or null
  uint16_t* Out;             // rows of length Nout
  int a_local, o_local;      // row index relative to expert_offset[e_begin]
  int e_begin;
  int K, Nw, Nout;
  int n_tiles_n, m_tiles, total;
};

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.7071067811865475f));
}
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One tile with NS active 32-row blocks (NS = ceil(rows / 32), 1..8).  All
// loops are static, so the accumulators stay in AGPRs without copies.
template <int MODE, int NS>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, uint16_t* __restrict__ As, int el,
                                          int n_t, int64_t a_row0, int64_t o_row0, int rows) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, lg = lane >> 5;
  const int K = a.K;

  // weight rows (output columns) this lane feeds, one per 32-column block
  int ncol0, ncol1;
  const uint16_t* wsrc0 = a.W0 + (size_t)el * a.Nw * K;
  const uint16_t* wsrc1;
  if (MODE == MODE_SWIGLU) {
    ncol0 = ncol1 = n_t * 128 + wave * 32 + l32;
    wsrc1 = a.W1 + (size_t)el * a.Nw * K;
  } else {
    ncol0 = n_t * 256 + wave * 64 + l32;
    ncol1 = ncol0 + 32;
    wsrc1 = wsrc0;
  }
  // Loads are unconditional from clamped (always valid) addresses; lanes
  // outside the matrix then select zero.  A branch around a load would force
  // a wait for it before the join.
  const bool bok0 = ncol0 < a.Nw, bok1 = ncol1 < a.Nw;
  const uint16_t* bp0 = wsrc0 + (size_t)(bok0 ? ncol0 : a.Nw - 1) * K + 8 * lg;
  const uint16_t* bp1 = wsrc1 + (size_t)(bok1 ? ncol1 : a.Nw - 1) * K + 8 * lg;

  // activation loader: thread owns 16-byte chunk ac of rows ar + 32 i
  const int ac = tid & 7, ar = tid >> 3;
  const uint16_t* ap = a.A + a_row0 * K + 8 * ac;
  int aoff[NS];
  bool aok[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = ar + 32 * i;
    aok[i] = r < rows;
    aoff[i] = (aok[i] ? r : rows - 1);
  }

  f32x16 acc0[NS], acc1[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[i][r] = 0.f;
      acc1[i][r] = 0.f;
    }
  }
  u32x4 bA[4][2], bB[4][2], av[NS];
  const u32x4 zero = {0u, 0u, 0u, 0u};

#define LOAD_B(BUF, K0)                                                   \
  _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_) {                     \
    const int kk_ = (K0) + 16 * s_ + 8 * lg;                              \
    const int ko_ = kk_ < K ? (K0) + 16 * s_ : K - 8 - 8 * lg;            \
    const u32x4 t0_ = *(const u32x4*)(bp0 + ko_);                         \
    const u32x4 t1_ = *(const u32x4*)(bp1 + ko_);                         \
    BUF[s_][0] = (bok0 && kk_ < K) ? t0_ : zero;                          \
    BUF[s_][1] = (bok1 && kk_ < K) ? t1_ : zero;                          \
  }
#define LOAD_A(K0)                                                        \
  {                                                                       \
    const bool kin_ = (K0) + 8 * ac < K;                                  \
    const int ko_ = kin_ ? (K0) : K - 8 - 8 * ac;                         \
    _Pragma("unroll") for (int i_ = 0; i_ < NS; ++i_) {                   \
      const u32x4 t_ = *(const u32x4*)(ap + (int64_t)aoff[i_] * K + ko_); \
      av[i_] = (aok[i_] && kin_) ? t_ : zero;                             \
    }                                                                     \
  }
#define STORE_A(BUFI)                                                     \
  _Pragma("unroll") for (int i_ = 0; i_ < NS; ++i_) {                     \
    const int r_ = ar + 32 * i_;                                          \
    *(u32x4*)&As[(BUFI) * (BM * BK) + r_ * BK + ((ac ^ (r_ & 7)) << 3)] = av[i_]; \
  }
#define COMPUTE(BUFI, BUF)                                                \
  _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_) {                     \
    const bf16x8 b0_ = as_bf16x8(BUF[s_][0]);                             \
    const bf16x8 b1_ = as_bf16x8(BUF[s_][1]);                             \
    const int ch_ = 2 * s_ + lg;                                          \
    _Pragma("unroll") for (int i_ = 0; i_ < NS; ++i_) {                   \
      const int r_ = 32 * i_ + l32;                                       \
      const bf16x8 af_ = as_bf16x8(                                       \
          *(const u32x4*)&As[(BUFI) * (BM * BK) + r_ * BK + ((ch_ ^ (r_ & 7)) << 3)]); \
      acc0[i_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_, b0_, acc0[i_], 0, 0, 0); \
      acc1[i_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_, b1_, acc1[i_], 0, 0, 0); \
    }                                                                     \
  }

  // Two stages per iteration so that the two register sets of weight
  // fragments swap statically.  Prefetches past the last stage reload the
  // last stage (in bounds, never consumed), which keeps the loop free of
  // branches around loads.
  const int nk = (K + BK - 1) / BK;
  LOAD_A(0);
  LOAD_B(bA, 0);
  STORE_A(0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    const int k1 = (kt + 1) * BK;
    LOAD_A(k1);
    LOAD_B(bB, k1);
    COMPUTE(0, bA);
    STORE_A(1);
    __syncthreads();
    const int k2 = (kt + 2 < nk ? kt + 2 : nk - 1) * BK;
    LOAD_A(k2);
    LOAD_B(bA, k2);
    COMPUTE(1, bB);
    STORE_A(0);
    __syncthreads();
  }
  if (kt < nk) {
    COMPUTE(0, bA);
    __syncthreads();
  }
#undef LOAD_B
#undef LOAD_A
#undef STORE_A
#undef COMPUTE

  // Epilogue, one 32-row block at a time: the wavefront parks its fp32
  // accumulators in LDS (acc[i][r] is row 8 (r / 4) + 4 lg + r % 4 of block
  // i, column l32 of its 32-column block), then reads them back row-wise,
  // applies the activation and writes 16-byte bf16 chunks.  The A buffers are
  // free: every wavefront has passed the last barrier of the main loop.
  constexpr int LD = 68;  // padded row of 64 fp32
  float* scr = reinterpret_cast<float*>(As) + wave * (32 * LD);
  const int n_base = MODE == MODE_SWIGLU ? n_t * 128 + wave * 32 : n_t * 256 + wave * 64;
  uint16_t* out = a.Out + o_row0 * a.Nout;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * lg + (r & 3);
      scr[row * LD + l32] = acc0[i][r];
      scr[row * LD + 32 + l32] = acc1[i][r];
    }
    __builtin_amdgcn_wave_barrier();
    if (MODE == MODE_SWIGLU) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int row = it * 16 + (lane >> 2), c = lane & 3;
        const float* g = scr + row * LD + 8 * c;
        const f32x4 g0 = *(const f32x4*)g, g1 = *(const f32x4*)(g + 4);
        const f32x4 u0 = *(const f32x4*)(g + 32), u1 = *(const f32x4*)(g + 36);
        float h[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] = silu_f(g0[q]) * u0[q];
          h[q + 4] = silu_f(g1[q]) * u1[q];
        }
        const int grow = 32 * i + row, gcol = n_base + 8 * c;
        if (grow < rows && gcol < a.Nout) *(u32x4*)(out + (int64_t)grow * a.Nout + gcol) = pack8(h);
      }
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = it * 8 + (lane >> 3), c = lane & 7;
        const float* g = scr + row * LD + 8 * c;
        const f32x4 v0 = *(const f32x4*)g, v1 = *(const f32x4*)(g + 4);
        float h[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] = MODE == MODE_GELU ? gelu_erf(v0[q]) : v0[q];
          h[q + 4] = MODE == MODE_GELU ? gelu_erf(v1[q]) : v1[q];
        }
        const int grow = 32 * i + row, gcol = n_base + 8 * c;
        if (grow < rows && gcol < a.Nout) *(u32x4*)(out + (int64_t)grow * a.Nout + gcol) = pack8(h);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * BK];

  // tile id: consecutive ids (same expert, neighbouring column tiles) share an XCD
  const int bid = blockIdx.x;
  const int per = a.total / kXcd;
  int tile = bid < per * kXcd ? (bid % kXcd) * per + bid / kXcd : bid;
  const int n_t = tile % a.n_tiles_n;
  tile /= a.n_tiles_n;
  const int m_t = tile % a.m_tiles;
  const int el = tile / a.m_tiles;
  const int e = a.e_begin + el;
  const int rb = a.eo[e];
  const int M = a.eo[e + 1] - rb;
  const int m0 = m_t * BM;
  if (m0 >= M) return;
  const int loc = a.eo[a.e_begin];
  const int64_t a_row0 = (int64_t)(rb - (a.a_local ? loc : 0) + m0);
  const int64_t o_row0 = (int64_t)(rb - (a.o_local ? loc : 0) + m0);
  const int rows = M - m0 < BM ? M - m0 : BM;
  switch ((rows + 31) >> 5) {
    case 1: gemm_tile<MODE, 1>(a, As, el, n_t, a_row0, o_row0, rows); break;
    case 2: gemm_tile<MODE, 2>(a, As, el, n_t, a_row0, o_row0, rows); break;
    case 3: gemm_tile<MODE, 3>(a, As, el, n_t, a_row0, o_row0, rows); break;
    case 4: gemm_tile<MODE, 4>(a, As, el, n_t, a_row0, o_row0, rows); break;
    case 5: gemm_tile<MODE, 5>(a, As, el, n_t, a_row0, o_row0, rows); break;
    case 6: gemm_tile<MODE, 6>(a, As, el, n_t, a_row0, o_row0, rows); break;
    case 7: gemm_tile<MODE, 7>(a, As, el, n_t, a_row0, o_row0, rows); break;
    default: gemm_tile<MODE, 8>(a, As, el, n_t, a_row0, o_row0, rows); break;
  }
}

template <int MODE>
hipError_t launch_gemm(GemmArgs g, hipStream_t s) {
  if (g.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_kernel<MODE>, dim3(g.total), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_ffn(const uint16_t* packed, const int32_t* expert_offset, int e_begin,
                             int n_local, int rows_max, int d, int f, bool swiglu,
                             const uint16_t* W1, const uint16_t* W3, const uint16_t* W2,
                             uint16_t* H, uint16_t* ret, hipStream_t s) {
  if (n_local <= 0 || rows_max <= 0) return hipSuccess;
  const int m_tiles = (rows_max + BM - 1) / BM;
  GemmArgs g1{};
  g1.A = packed;
  g1.eo = expert_offset;
  g1.W0 = W1;
  g1.W1 = swiglu ? W3 : nullptr;
  g1.Out = H;
  g1.a_local = 0;
  g1.o_local = 1;
  g1.e_begin = e_begin;
  g1.K = d;
  g1.Nw = f;
  g1.Nout = f;
  g1.n_tiles_n = swiglu ? (f + 127) / 128 : (f + 255) / 256;
  g1.m_tiles = m_tiles;
  g1.total = n_local * m_tiles * g1.n_tiles_n;
  hipError_t err = swiglu ? launch_gemm<MODE_SWIGLU>(g1, s) : launch_gemm<MODE_GELU>(g1, s);
  if (err != hipSuccess) return err;

  GemmArgs g2{};
  g2.A = H;
  g2.eo = expert_offset;
  g2.W0 = W2;
  g2.W1 = nullptr;
  g2.Out = ret;
  g2.a_local = 1;
  g2.o_local = 0;
  g2.e_begin = e_begin;
  g2.K = f;
  g2.Nw = d;
  g2.Nout = d;
  g2.n_tiles_n = (d + 255) / 256;
  g2.m_tiles = m_tiles;
  g2.total = n_local * m_tiles * g2.n_tiles_n;
  return launch_gemm<MODE_PLAIN>(g2, s);
}

}  // namespace moek
