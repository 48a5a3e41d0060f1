// Grouped expert MLP on bf16 matrix cores (gfx950 MFMA 32x32x16).
//
// "Expert Parallelism" (narrativegoldmine.com), "Components and
// Architecture", Expert GEMM: each expert is a standard transformer MLP run on
// the tokens routed to it, with no communication during the compute phase;
// "Formal Algorithm": the work is proportional to received tokens times the
// expert FFN cost.
//
// Two launches per call, each a grouped GEMM over the experts' contiguous
// packed segments (rows [expert_offset[e], expert_offset[e+1])), with the
// weights as [in, out] matrices (W1, W3 [d][f], W2 [f][d]):
//   GEMM1  H   = act(X . W1)              (GELU)   or
//          H   = silu(X . W1) * (X . W3)  (SwiGLU, both products in one tile)
//   GEMM2  Out = H . W2
//
// Weight streaming.  With ~100-2000 rows per expert the GEMMs of the smaller
// workloads are bound by reading the weights from HBM once.  Weights are
// therefore kept in a blocked layout (moe_pack_weights, once per model): for
// every expert, 256-column output tile and 64-wide K stage, one contiguous
// 32 KB block holding, in order, each wavefront's MFMA operand fragments
// (1 KB per fragment: 64 lanes x 16 bytes).  A wavefront loads its fragments
// straight into registers, front to back, as whole 1 KB requests from
// consecutive addresses; every weight byte is read once.  Tails (N or K not
// a multiple of 256 / 64, and K padded to a whole pipeline group) are zero
// in the blocks, so the MFMAs need no masking.
//
// Tile: up to 256 rows x 256 output columns (128 hidden units of W1 and W3
// for SwiGLU), K stages of 64; 4 wavefronts, one per SIMD, each owning 64
// weight columns and all row blocks (accumulators in the AGPRs, up to 256).
//  * One tile usually covers a whole expert segment (C is 160 / 256 in the
//    HBM-bound workloads); only the 32-row blocks that hold rows run MFMAs
//    (the block count is a template parameter chosen per tile).
//  * Weights: global -> registers, kP - 1 stages ahead (8 KB per wavefront
//    per stage).  Activations: global -> LDS by buffer loads that write LDS
//    directly (no register staging) into a kP-slot ring, bank-swizzled;
//    every activation fragment read from LDS feeds two MFMAs.
//  * Persistent, two schedules.  Weight-streaming launches: each workgroup
//    runs a contiguous range of tiles; tiles of one expert that share its
//    activation rows sit on the same XCD (workgroups are dealt round-robin
//    over the 8 XCDs), so the activation rows are read from HBM about once
//    per expert and then from L2.  Matrix-core-bound launches (hundreds of
//    rows per expert): chunks of consecutive tiles are dealt round-robin
//    over the XCDs, so each XCD works on a compact patch of one expert at a
//    time and every XCD gets a share of every expert.
#include "launch.h"
#include "moe_kernels.h"

namespace moek {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int BM = 256;                   // rows per tile
constexpr int BK = 64;                    // K per stage
constexpr int kRowBytes = BK * 2;         // one K slice of a row: 128 B
constexpr int kTileRows = 256;            // weight rows per tile
constexpr int kWStage = kTileRows * kRowBytes;  // 32 KB of weights per tile and stage
constexpr int kP = 4;                     // pipeline depth (stages in flight + 1)
constexpr int kLdsBytes = 160 * 1024;
constexpr int kXcd = 8;

// MODE_DGELU / MODE_DSWIGLU (backward): the tile's products are dH, the
// gradient of the hidden activation; the epilogue reads the pre-activations
// Z of the same rows and writes dZ = dH * gelu'(Z), or dZ1 = dH Z3 silu'(Z1)
// and dZ3 = dH silu(Z1) (at columns u and f + u of a 2f-wide row).
enum { MODE_GELU = 0, MODE_SWIGLU = 1, MODE_PLAIN = 2, MODE_DGELU = 3, MODE_DSWIGLU = 4 };

struct GemmArgs {
  const uint16_t* A;         // rows of length K
  const int32_t* eo;         // expert_offset [E+1]
  const uint16_t* Wp;        // blocked weights of this GEMM
  uint16_t* Out;             // rows of length Nout
  int a_local, o_local;      // row index relative to expert_offset[e_begin]
  int e_begin;
  int K, Nout;
  int n_tiles_n, nk;
  int n_local;               // experts e_begin .. e_begin + n_local - 1
  // backward epilogues: pre-activations Z (rows as Out's, zw per row) and
  // the output row stride (Nout is then the valid column count, f)
  const uint16_t* Z;
  int zw;
  int ldo;
  // gather (optional): row r of the A operand is row gidx[r] of A, a matrix
  // of src_rows rows (the forward's first GEMM reads the token rows of x
  // through pack_src instead of a packed copy)
  const int32_t* gidx;
  int64_t src_rows;
  // GELU / SwiGLU launch, optional: the pre-activations themselves, stored
  // as the plain launch of the same weights would store them (rows as
  // Out's, zs_w per row), for a backward pass that then need not recompute
  // them
  uint16_t* Zs;
  int zs_w;
};

// GELU with the exact-erf definition, 0.5 z (1 + erf(z / sqrt 2)).  erf is
// evaluated with Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (absolute error <= 1.5e-7, far below the bf16 rounding of
// the stored activation): for x >= 0, erf(x) = 1 - q with
// q = (a1 t + a2 t^2 + ... + a5 t^5) e^{-x^2}, t = 1 / (1 + p x), and erf is
// odd.  With x = |z| / sqrt 2 this gives GELU(z) = z - z q / 2 for z >= 0
// and z q / 2 for z < 0.  The constants p / sqrt 2 and log2(e) / 2 are
// folded in, and the reciprocal and exponential are single hardware
// instructions (v_rcp_f32, v_exp_f32: about 1 ulp), once per hidden
// activation in the epilogue.
__device__ __forceinline__ float gelu_erf(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164188f, az, 1.0f));  // p / sqrt 2
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  // e^{-z^2 / 2} = 2^{-(log2 e / 2) z^2}
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752f);
  const float r = 0.5f * z * (p * e);
  return z >= 0.0f ? z - r : r;
}
// silu(z) = z / (1 + e^{-z}), with e^{-z} = 2^{-z log2 e} and a hardware
// reciprocal
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504f));
}
// GELU'(z) = Phi(z) + z phi(z).  With the same erf approximation (A & S
// 7.1.26, x = |z| / sqrt 2): Phi(z) = 1 - q / 2 for z >= 0 and q / 2 for
// z < 0, q = poly(t) e^{-z^2 / 2}; phi(z) = e^{-z^2 / 2} / sqrt(2 pi).
__device__ __forceinline__ float dgelu_erf(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164188f, az, 1.0f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752f);
  const float hq = 0.5f * p * e;
  const float Phi = z >= 0.0f ? 1.0f - hq : hq;
  return fmaf(z * 0.39894228f, e, Phi);
}
// column of hidden unit u's W1 product in the recomputed SwiGLU
// pre-activations (the GEMM1 tile order: per 128 units, four 64-column
// groups of 32 W1 then 32 W3 products)
__device__ __forceinline__ int zcol_w1(int u) {
  return (u >> 7) * 256 + ((u >> 5) & 3) * 64 + (u & 31);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds; lds must be wavefront-uniform), from byte
// offset off of the buffer rs; offsets past the buffer's size read zeros.
// The buffer form rather than global_load_lds: the compiler counts a pending
// global_load_lds against the LDS-read counter as well, and then has to wait
// for every outstanding LDS read (lgkmcnt(0)) before each MFMA step instead
// of only the ones that step consumes.
// The LDS address is a 32-bit offset: converting a generic pointer instead
// costs a null check (three scalar instructions) per load.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t off, uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(uintptr_t)lds, 16, off, 0, 0, 0);
}
// 32-bit LDS offset of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_off(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One accumulator element, read out of the accumulation registers where it
// is used (left alone, the compiler copies every accumulator of the tile to
// ordinary registers at the start of the epilogue).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
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

// Activation ring for a tile of NS row blocks: kP slots of the size of an
// 8-block tile's 64-wide K slice, holding the tile's 32 NS rows (one 32-row
// DMA round per block).  The slots sit at the same offsets whatever NS is,
// so a run's prologue, which writes slots 0 .. kP - 2, never touches the
// last slot of the run before (that one may still be read).
template <int NS>
struct Ring {
  static constexpr int A_BYTES = 8 * 32 * kRowBytes;
  static constexpr int LOADS = NS + 8;  // vector-memory loads per thread per stage
};
static_assert(kP * Ring<8>::A_BYTES <= kLdsBytes, "activation ring exceeds LDS");
// LDS past the ring: the tile scheduler's scan arrays (4 (1029 + 1025) bytes),
// then the epilogue's staging area, 32 rows x 64 bf16 columns per wavefront
constexpr int kStageOff = kP * Ring<8>::A_BYTES + 8448;
// staged row of 64 bf16 columns, padded by 16 bytes: the 8-byte writes of
// the 32 rows of a block then spread over the banks, and rows stay 16-byte
// aligned for the read-back
constexpr int kStgRow = 64 * 2 + 16;
static_assert(kStageOff + (kThreads / 64) * 32 * kStgRow <= kLdsBytes, "staging area exceeds LDS");
static_assert((kP - 2) * Ring<8>::LOADS < 64, "vmcnt range");

// Weight fragment load.  Streaming launches (each weight byte used by one
// tile) mark it non-temporal so it does not push the activation rows out of
// L2; matrix-core-bound launches share weight tiles between row slices
// through L2, so there it is an ordinary load.
template <bool NT>
__device__ __forceinline__ u32x4 load_w(const char* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

// A run of `ntile` consecutive output tiles (n0 .. n0+ntile-1) of one expert
// and one row slice of `rows` <= 32 NS rows.  Wavefront w (one per SIMD)
// owns the 64 weight rows 64w .. 64w+63 of each tile -- two 32-column MFMA
// blocks -- and all NS row blocks: 2 NS accumulators of 16 registers.  The
// weight fragment is the matrix instruction's first operand, so an
// accumulator holds the transposed block: register r of lane l is row l % 32
// of the block, column 8 (r / 4) + 4 (l / 32) + r % 4 -- four consecutive
// columns of one row in registers 4q .. 4q + 3.
//
// The run is one pipeline over ntile * nk stages of 64 K; nk is a multiple
// of kP, so tile ends fall on the last step of the unrolled group and the
// register set and ring slot of a stage are compile-time constants.  Stage
// g + kP - 1 is issued while stage g is multiplied:
//   weights     global -> registers, the wavefront's own 8 KB (eight 1 KB
//               fragment loads, non-temporal), set (g + kP - 1) % kP;
//   activations global -> LDS by DMA, slot (g + kP - 1) % kP.
// Vector-memory loads complete in issue order, so waiting until at most
// (kP - 2) stages' loads are outstanding means stage g has landed.  After an
// epilogue the counter also holds stores, which are not ordered with the
// loads: then wait for everything.
//
// Matrix-core-bound launches (NT false) wait one stage further, for stage
// g + 1 as well, at the start of stage g; each wavefront can then read stage
// g + 1's first activation fragments right after its last MFMAs of stage g,
// so the next stage's MFMAs start as soon as the barrier is passed instead
// of after an LDS round trip.  Their loads hit L2 often enough that two
// stages of lead suffice; the weight-streaming launches keep the deeper
// lead, which the loaded HBM latency needs.
template <int MODE, int NS, bool NT>
__device__ __forceinline__ void gemm_run(const GemmArgs& a, char* __restrict__ smem, int el,
                                         int n0, int ntile, int64_t a_row0, int64_t o_row0,
                                         int rows) {
  using R = Ring<NS>;
  const int lane = threadIdx.x & 63;
  // wavefront-uniform, so that every address below that depends only on it
  // lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lg = lane >> 5;
  const int K = a.K;
  const int nk = a.nk;
  const int nstage = ntile * nk;

  // DMA lane geometry: round i fills rows 32 i + 8 wave + lane/8, LDS chunk
  // lane % 8, which holds K chunk (lane % 8) ^ swz_key(row) (the key depends
  // only on drow, as 32 i is a multiple of 16).  Global addresses are a
  // scalar base plus a 32-bit per-lane byte offset (a row slice is far below
  // 4 GB).
  const int drow = 8 * wave + (lane >> 3);
  const int dcol = 8 * ((lane & 7) ^ swz_key(drow));  // K offset of the lane's chunk
  // the row slice as one buffer (rows x K bf16), or with a gather the whole
  // source matrix, each lane's row through the index.  Only the first GEMM
  // (GELU / SwiGLU) gathers: in the other modes the gather is compiled out,
  // since a possible index load leaves a wait for every outstanding memory
  // operation where the two ways of forming the row offset meet -- with the
  // previous tile's epilogue stores still in flight, at every tile.
  constexpr bool kCanGather = MODE == MODE_GELU || MODE == MODE_SWIGLU;
  const bool gat = kCanGather && a.gidx != nullptr;
  const char* abase = reinterpret_cast<const char*>(gat ? a.A : a.A + a_row0 * K);
  const rsrc_t ars =
      make_rsrc(abase, 2u * (uint32_t)(gat ? a.src_rows : (int64_t)rows) * (uint32_t)K);
  uint32_t arow[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = 32 * i + drow;
    const int rr = r < rows ? r : rows - 1;  // past the segment: any valid row
    arow[i] = 2u * (uint32_t)(gat ? a.gidx[a_row0 + rr] : rr) * (uint32_t)K;
  }
  // this wavefront's weight fragments: stage G of the run at G * kWStage
  const char* wbase = reinterpret_cast<const char*>(a.Wp) +
                      (size_t)(el * a.n_tiles_n + n0) * nk * kWStage + wave * 8192;
  const uint32_t wlane = 16u * lane;

  u32x4 bw[kP][8];

  // Issue state, all scalar: the next stage to issue is K stage iss_k of the
  // weight block at iss_w; once the last stage is issued the pointers stop
  // and further issues reload it (in bounds, never read), so every step
  // issues the same number of loads.
  int iss_k = 0, iss_left = nstage;
  // this wavefront's rows of ring slot 0; made opaque once per stage below,
  // so that the per-slot, per-round LDS addresses are recomputed where they
  // are used instead of all being hoisted into scalar registers
  uint32_t lds_w = lds_off(smem) + 8 * wave * kRowBytes;
  const char* iss_w = wbase;
  // K chunks past K (and whole padding stages) have zero weights, so the
  // activation side may load anything finite there: clamp into the row.
#define ISSUE(SLOT)                                                                \
  {                                                                                \
    const uint32_t st_ = lds_w + (SLOT) * R::A_BYTES;                              \
    const int kc_ = iss_k * BK + dcol;                                             \
    const uint32_t cb_ = 2u * (uint32_t)(kc_ < K ? kc_ : K - 8);                   \
    _Pragma("unroll") for (int i_ = 0; i_ < NS; ++i_)                              \
      dma16(ars, arow[i_] + cb_, st_ + 32 * i_ * kRowBytes);                       \
    const char* wb_ = iss_w + wlane;                                               \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) bw[SLOT][j_] = load_w<NT>(wb_ + 1024 * j_); \
    if (iss_left > 1) {                                                            \
      --iss_left;                                                                  \
      iss_w += kWStage;                                                            \
      iss_k = iss_k + 1 == nk ? 0 : iss_k + 1;                                     \
    }                                                                              \
  }

#pragma unroll
  for (int p = 0; p < kP - 1; ++p) ISSUE(p);
  // activation fragments of the current MFMA step, one per row block
  constexpr bool PRE = !NT;
  u32x4 fa[NS];
  if (PRE) {
    // stages 0 and 1 have landed; the first fragments of stage 0
    wait_vmcnt<(kP - 3) * R::LOADS>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < NS; ++i) fa[i] = *(const u32x4*)(smem + swz(32 * i + l32, lg));
  }

  for (int tile = n0; tile < n0 + ntile; ++tile) {
  // accumulators live only inside one tile (carried across the tile loop
  // they would be kept in a second copy)
  f32x16 acc[2][NS];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][i][r] = 0.f;
  for (int kk = 0; kk < nk; kk += kP) {
#pragma unroll
    for (int u = 0; u < kP; ++u) {
      wait_vmcnt<(PRE ? kP - 3 : kP - 2) * R::LOADS>();
      // every wavefront's part of slot u (PRE: and of slot u + 1) has landed
      // and slot u - 1 is consumed (its LDS reads fed MFMAs).  A bare s_barrier: a
      // __syncthreads() fence would wait for the whole prefetch.
      __builtin_amdgcn_s_barrier();
      asm volatile("" : "+s"(lds_w));
      // Stage g + kP - 1 is issued spread between this stage's MFMAs, not as
      // one burst: part q (NS activation rounds, then 8 weight fragments)
      // follows MFMA pair q * 4NS / NL.  With one wavefront per SIMD, a load
      // whose issue stalls (memory queues full) stalls the matrix core too;
      // spread out, the stalls fall in the gaps between MFMAs.
      constexpr int NL = NS + 8;
      const uint32_t ist_ = lds_w + ((u + kP - 1) % kP) * R::A_BYTES;
      const int ikc_ = iss_k * BK + dcol;
      const uint32_t icb_ = 2u * (uint32_t)(ikc_ < K ? ikc_ : K - 8);
      const char* iwb_ = iss_w + wlane;
      __builtin_amdgcn_sched_barrier(0);
      const char* sa = smem + u * R::A_BYTES;
      // Activation fragments are re-read for step s + 1 right after the two
      // MFMAs of step s that consume them (PRE: after step 3, the next
      // stage's step 0 from slot u + 1).
      const char* sn = smem + ((u + 1) % kP) * R::A_BYTES;
      if (!PRE) {
#pragma unroll
        for (int i = 0; i < NS; ++i) fa[i] = *(const u32x4*)(sa + swz(32 * i + l32, lg));
      }
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_) {
        const bf16x8 b0 = as_bf16x8(bw[u][2 * s_]);
        const bf16x8 b1 = as_bf16x8(bw[u][2 * s_ + 1]);
        const int chn = 2 * (s_ + 1) + lg;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const bf16x8 af = as_bf16x8(fa[i]);
          acc[0][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, af, acc[0][i], 0, 0, 0);
          acc[1][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, af, acc[1][i], 0, 0, 0);
          if (s_ < 3) fa[i] = *(const u32x4*)(sa + swz(32 * i + l32, chn));
          else if (PRE) fa[i] = *(const u32x4*)(sn + swz(32 * i + l32, lg));
#pragma unroll
          for (int q = 0; q < NL; ++q) {
            if (q * 4 * NS / NL == s_ * NS + i) {
              if (q < NS)
                dma16(ars, arow[q < NS ? q : 0] + icb_, ist_ + 32 * q * kRowBytes);
              else
                bw[(u + kP - 1) % kP][q - NS] = load_w<NT>(iwb_ + 1024 * (q - NS));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (iss_left > 1) {
        --iss_left;
        iss_w += kWStage;
        iss_k = iss_k + 1 == nk ? 0 : iss_k + 1;
      }
    }
  }
  if constexpr (MODE == MODE_DGELU || MODE == MODE_DSWIGLU) {
    // Backward epilogue of tile `tile`: the products are dH for hidden units
    // 256 tile + 64 wave + 32 c + (column in the block).  They are staged
    // through LDS as bf16 exactly like the plain epilogue's outputs (32 rows
    // x 64 units per wavefront); then each lane takes 16-byte row segments (8 units of one
    // row), loads the matching pre-activations Z as 16-byte vectors and
    // writes dZ = dH * gelu'(Z), or dZ1 = dH Z3 silu'(Z1) and dZ3 = dH
    // silu(Z1) at columns u and f + u, as 16-byte stores.
    int ldo = a.ldo;
    asm volatile("" : "+s"(ldo));
    uint16_t* out = a.Out + o_row0 * ldo;
    const uint16_t* zb = a.Z + o_row0 * a.zw;
    const int nval = a.Nout;
    char* stg = smem + kStageOff + wave * 32 * kStgRow;
    const int col0 = tile * 256 + 64 * wave;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc_read(acc[c][i][4 * q + j]);
          *(uint2*)(stg + l32 * kStgRow + (32 * c + 8 * q + 4 * lg) * 2) =
              uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // one segment at a time (not unrolled: the loads of all four would
      // be hoisted together and crowd the live accumulators)
#pragma unroll 1
      for (int qq = 0; qq < 32 * 8 / 64; ++qq) {
        const int sgi = lane + 64 * qq;
        const int rin = sgi / 8, sg8 = sgi % 8;
        const int row = 32 * i + rin, u0 = col0 + 8 * sg8;
        if (row < rows && u0 < nval) {
          float dh[8], z1[8], o1[8];
          unpack8(*(const u32x4*)(stg + rin * kStgRow + sg8 * 16), dh);
          const uint16_t* zr = zb + (int64_t)row * a.zw;
          if (MODE == MODE_DGELU) {
            unpack8(*(const u32x4*)(zr + u0), z1);
#pragma unroll
            for (int e = 0; e < 8; ++e) o1[e] = dh[e] * dgelu_erf(z1[e]);
            *(u32x4*)(out + ((int64_t)row * ldo + u0)) = pack8(o1);
          } else {
            float z3[8], o3[8];
            const uint16_t* zp = zr + zcol_w1(u0);
            unpack8(*(const u32x4*)zp, z1);
            unpack8(*(const u32x4*)(zp + 32), z3);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float sg = __builtin_amdgcn_rcpf(
                  1.0f + __builtin_amdgcn_exp2f(z1[e] * -1.44269504f));
              o1[e] = dh[e] * z3[e] * sg * fmaf(z1[e], 1.0f - sg, 1.0f);
              o3[e] = dh[e] * z1[e] * sg;
            }
            *(u32x4*)(out + ((int64_t)row * ldo + u0)) = pack8(o1);
            *(u32x4*)(out + ((int64_t)row * ldo + nval + u0)) = pack8(o3);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
        // Epilogue of tile `tile`.  Registers 4q .. 4q + 3 of acc[c][i] are
        // columns 32 c + 8 q + 4 lg .. + 3 of row l32 of row block i (of the
        // wavefront's weight block c); the activation is applied, the four
        // values are converted to bf16 and written to LDS as one 8-byte
        // piece.  Each 32-row block is staged that way (in a part of LDS the
        // ring does not use now) and leaves as 16-byte row segments, so
        // every store writes whole 128-byte lines.  The staging area is
        // private to the wavefront and lies past the ring, so no barrier
        // guards it.
        const int nt = tile;
        // Opaque copy of the row length: without it the compiler hoists every
        // row address of the epilogue out of the tile loop and spills them.
        int nout = a.Nout;
        asm volatile("" : "+s"(nout));
        uint16_t* out = a.Out + o_row0 * nout;
        // output columns of this wavefront: 64 (SwiGLU: 32 hidden units)
        constexpr int WCOLS = MODE == MODE_SWIGLU ? 32 : 64;
        char* stg = smem + kStageOff + wave * 32 * kStgRow;
        const int col0 = MODE == MODE_SWIGLU ? nt * 128 + 32 * wave : nt * 256 + 64 * wave;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (MODE != MODE_PLAIN && a.Zs) {
            // the pre-activations of block i first, through the same
            // staging area, exactly as the plain launch stores its outputs
            // (both weight blocks, 64 columns per wavefront); non-temporal,
            // as only a later backward pass reads them
            int zs_w = a.zs_w;
            asm volatile("" : "+s"(zs_w));
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = acc_read(acc[c][i][4 * q + j]);
                *(uint2*)(stg + l32 * kStgRow + (32 * c + 8 * q + 4 * lg) * 2) =
                    uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
              }
            __builtin_amdgcn_sched_barrier(0);
            uint16_t* zo = a.Zs + o_row0 * zs_w;
            const int zc0 = nt * 256 + 64 * wave;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int sgi = lane + 64 * q;
              const int rin = sgi / 8, sg = sgi % 8;
              const u32x4 v = *(const u32x4*)(stg + rin * kStgRow + sg * 16);
              const int row = 32 * i + rin, col = zc0 + 8 * sg;
              if (row < rows && col < zs_w)
                __builtin_nontemporal_store(v, (u32x4*)(zo + (row * zs_w + col)));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int c = 0; c < (MODE == MODE_SWIGLU ? 1 : 2); ++c) {
            // SwiGLU: block 0 holds the W1 products and block 1 the W3
            // products of the same hidden units, in the same lanes and
            // registers.  Two 4-column pieces at a time: their dependency
            // chains (read-out, activation with exp2 and reciprocal,
            // conversion) interleave while the temporaries stay few.
#pragma unroll
            for (int q0 = 0; q0 < 4; q0 += 2) {
              float v[2][4];
#pragma unroll
              for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const int r = 4 * (q0 + g) + j;
                  if (MODE == MODE_SWIGLU) {
                    v[g][j] = silu_f(acc_read(acc[0][i][r])) * acc_read(acc[1][i][r]);
                  } else {
                    v[g][j] = acc_read(acc[c][i][r]);
                    if (MODE == MODE_GELU) v[g][j] = gelu_erf(v[g][j]);
                  }
                }
#pragma unroll
              for (int g = 0; g < 2; ++g)
                *(uint2*)(stg + l32 * kStgRow + (32 * c + 8 * (q0 + g) + 4 * lg) * 2) =
                    uint2{pack_bf16x2(v[g][0], v[g][1]), pack_bf16x2(v[g][2], v[g][3])};
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // block i: 32 rows x WCOLS columns, 16-byte segments
          constexpr int SPR = WCOLS / 8;  // segments per row
#pragma unroll
          for (int q = 0; q < 32 * SPR / 64; ++q) {
            const int sgi = lane + 64 * q;
            const int rin = sgi / SPR, sg = sgi % SPR;
            const u32x4 v = *(const u32x4*)(stg + rin * kStgRow + sg * 16);
            const int row = 32 * i + rin, col = col0 + 8 * sg;
            // The hidden activations H (GELU / SwiGLU launch) are read back
            // only by the second GEMM, after the whole launch: stored
            // non-temporally they do not displace the weights and
            // activation rows the launch is streaming (uniform routing:
            // FFN 261 -> 240 us).  The FFN output stays a normal store: the
            // combine reads it next, often still from cache.
            if (row < rows && col < nout) {
              if (MODE == MODE_PLAIN)
                *(u32x4*)(out + (row * nout + col)) = v;
              else
                __builtin_nontemporal_store(v, (u32x4*)(out + (row * nout + col)));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
  }
  }
#undef ISSUE
  // No wait for the epilogue's stores, and no barrier: the stores drain
  // while the next run's loads are issued.  The stage waits stay correct
  // with stores in the counter -- at most N operations outstanding means at
  // most N loads outstanding, and loads complete in issue order -- and the
  // next run's prologue writes only ring slots 0 .. kP - 2, which every
  // wavefront finished reading before the barrier of this run's last stage
  // (its epilogue staging area is its own).
}

// Persistent over an equal share of the active tiles.  Expert el has
// ceil(M_el / BM) row slices of its M_el rows, each with n_tiles_n output
// tiles; tiles are ordered (expert, row slice, output tile), so consecutive
// tiles of one expert and row slice form a pipelined run over contiguous
// weight blocks.  Every workgroup counts the active tiles itself from
// expert_offset (a scan of one value per expert in LDS), so experts with no
// rows cost nothing and skewed routing does not idle workgroups.
constexpr int kRingBytes = kP * Ring<8>::A_BYTES;
static_assert(kRingBytes + 4 * (1029 + 1025) <= kStageOff, "LDS budget");

// Row slice m_t of an expert's M rows, cut into nsl = ceil(M / BM) slices:
// the ceil(M / 32) row blocks are dealt as evenly as possible (the first
// nb % nsl slices take one block more), so that no slice is a thin tail
// whose stages would cost as much as a full slice's.  The slice count is the
// same as with full slices and a trailing remainder; nsl = ceil(nb / 8), so
// no slice exceeds 8 blocks.
__device__ __forceinline__ void row_slice(int M, int nsl, int m_t, int& m0, int& rows) {
  const int nb = (M + 31) >> 5;
  const int q = nb / nsl, r = nb - q * nsl;
  m0 = 32 * (m_t * q + (m_t < r ? m_t : r));
  const int span = 32 * (q + (m_t < r ? 1 : 0));
  rows = M - m0 < span ? M - m0 : span;
}

template <int MODE, bool XS>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  // pre[el] = active (expert, row slice) pairs of the experts before el
  int* pre = reinterpret_cast<int*>(smem + kRingBytes);
  int* wsum = pre + 1025;  // per-wavefront totals (4)
  int* eos = wsum + 4;     // expert_offset[e_begin .. e_begin + n_local]
  const int nl = a.n_local;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    // thread tid scans experts [4 tid, 4 tid + 4) (n_local <= 1024)
    int cnt[4], run_ = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int el = 4 * tid + j;
      int m = 0;
      if (el < nl) {
        const int lo = a.eo[a.e_begin + el], hi = a.eo[a.e_begin + el + 1];
        eos[el] = lo;
        if (el == nl - 1) eos[nl] = hi;
        m = (hi - lo + BM - 1) / BM;
      }
      cnt[j] = run_;
      run_ += m;
    }
    // inclusive scan of the per-thread totals inside the wavefront
    int incl = run_;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = incl - run_;
    for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * tid + j < nl) pre[4 * tid + j] = base + cnt[j];
    if (tid == kThreads - 1) pre[nl] = base + run_;
    __syncthreads();
  }
  const int64_t total = (int64_t)pre[nl] * a.n_tiles_n;
  const int G = gridDim.x, b = blockIdx.x;
  const int loc0 = eos[0];
  if (XS) {
    // Matrix-core-bound launches (hundreds of rows per expert): tiles are
    // ordered (expert, output tile, row slice) and cut into 8 equal
    // contiguous ranges, one per XCD (the workgroups b with b % 8 == x sit
    // on XCD x: workgroups are dealt round-robin over the 8 XCDs); the nx
    // workgroups of an XCD take its tiles in turn, nx consecutive tiles at a
    // time.  At any moment an XCD then works on a compact patch of one
    // expert -- few row slices x few output tiles -- so the activation
    // slices and weight tiles it streams are shared through its L2, an
    // expert's weights are read by one or two XCDs only, and every XCD gets
    // the same number of tiles (experts differ in rows, so whole experts
    // per XCD would not balance, and dealing chunks of nx tiles round-robin
    // leaves the XCDs a chunk apart when the chunk count is not a multiple
    // of 8).
    const int x = b % kXcd, j = b / kXcd;
    const int nx = G / kXcd;  // workgroups per XCD (G >= 8)
    if (j >= nx) return;      // the G % 8 extra workgroups take no tiles
    const int64_t xe = total * (x + 1) / kXcd;
    for (int64_t t = total * x / kXcd + j; t < xe; t += nx) {
      const int p = (int)(t / a.n_tiles_n);
      int lo = 0, hi = nl - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= p) lo = mid; else hi = mid - 1;
      }
      const int el = lo;
      const int mel = pre[el + 1] - pre[el];  // row slices of this expert
      const int64_t loc_t = t - (int64_t)pre[el] * a.n_tiles_n;
      const int n_t = (int)(loc_t / mel), m_t = (int)(loc_t - (int64_t)n_t * mel);
      const int rb = eos[el];
      int m0, rows;
      row_slice(eos[el + 1] - rb, mel, m_t, m0, rows);
      const int64_t a_row0 = (int64_t)(rb - (a.a_local ? loc0 : 0) + m0);
      const int64_t o_row0 = (int64_t)(rb - (a.o_local ? loc0 : 0) + m0);
      switch ((rows + 31) >> 5) {
        case 1: gemm_run<MODE, 1, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        case 2: gemm_run<MODE, 2, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        case 3: gemm_run<MODE, 3, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        case 4: gemm_run<MODE, 4, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        case 5: gemm_run<MODE, 5, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        case 6: gemm_run<MODE, 6, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        case 7: gemm_run<MODE, 7, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
        default: gemm_run<MODE, 8, false>(a, smem, el, n_t, 1, a_row0, o_row0, rows); break;
      }
    }
    return;
  }
  // Weight-streaming launches: a contiguous range per workgroup, the ranges
  // of neighbouring logical ids (mostly one expert's tiles) on the same XCD.
  const int nper = G / kXcd;
  const int L = b < nper * kXcd ? (b % kXcd) * nper + b / kXcd : b;
  const int64_t t0 = total * L / G, t1 = total * (L + 1) / G;
  if (t0 >= t1) return;
  const int loc = loc0;
  // expert of the first pair: the last el with pre[el] <= p (binary search;
  // experts without rows share their pre value with the next one)
  int el = 0;
  {
    const int p = (int)(t0 / a.n_tiles_n);
    int lo = 0, hi = nl - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= p) lo = mid; else hi = mid - 1;
    }
    el = lo;
  }
  for (int64_t t = t0; t < t1;) {
    const int p = (int)(t / a.n_tiles_n);
    const int n_t = (int)(t - (int64_t)p * a.n_tiles_n);
    while (pre[el + 1] <= p) ++el;
    const int m_t = p - pre[el];
    const int run = (int)(t1 - t < a.n_tiles_n - n_t ? t1 - t : a.n_tiles_n - n_t);
    t += run;
    const int rb = eos[el];
    int m0, rows;
    row_slice(eos[el + 1] - rb, pre[el + 1] - pre[el], m_t, m0, rows);
    const int64_t a_row0 = (int64_t)(rb - (a.a_local ? loc : 0) + m0);
    const int64_t o_row0 = (int64_t)(rb - (a.o_local ? loc : 0) + m0);
    switch ((rows + 31) >> 5) {
      case 1: gemm_run<MODE, 1, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 2: gemm_run<MODE, 2, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 3: gemm_run<MODE, 3, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 4: gemm_run<MODE, 4, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 5: gemm_run<MODE, 5, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 6: gemm_run<MODE, 6, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      case 7: gemm_run<MODE, 7, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
      default: gemm_run<MODE, 8, true>(a, smem, el, n_t, run, a_row0, o_row0, rows); break;
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

// One workgroup per CU (the LDS ring takes most of the 160 KB), no more
// workgroups than there could be tiles.  e0 / e1 (optional) take the
// dispatch's start / end timestamps; with no tiles they are recorded as
// markers.  Without events the plain launch is used: the timestamped launch
// leaves a gap of about 5 us on each side of the kernel (measured in kernel
// traces; the plain launches follow each other with none).
template <int MODE>
hipError_t launch_gemm(GemmArgs g, int m_tiles, bool mfma_bound, hipStream_t s,
                       hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const int64_t bound = (int64_t)g.n_local * m_tiles * g.n_tiles_n;
  if (bound <= 0) {
    hipError_t e = hipSuccess;
    if (e0) e = hipEventRecord(e0, s);
    if (e == hipSuccess && e1) e = hipEventRecord(e1, s);
    return e;
  }
  const int cus = device_cus();
  const int grid = bound < cus ? (int)bound : cus;
  if (mfma_bound && grid >= kXcd)
    launch_timed(grouped_gemm_kernel<MODE, true>, dim3(grid), dim3(kThreads), 0, s, e0, e1, g);
  else
    launch_timed(grouped_gemm_kernel<MODE, false>, dim3(grid), dim3(kThreads), 0, s, e0, e1, g);
  return hipGetLastError();
}

// Blocked weight layout, in the order the wavefronts load it: for expert e,
// output tile nt and stage kt (nk stages, padded to a multiple of kP), one
// 32 KB block; inside it wavefront w's 8 KB, then MFMA step s's 2 KB, then
// column block cb's 1 KB, then lane l's 16 bytes = K values
// kt*64 + 16 s + 8 (l / 32) .. +7 of weight-tile row j = 64 w + 32 cb + l % 32
// (zeros past N or K).  Tile row j is output column nt*256 + j (GELU,
// plain); for SwiGLU, block cb = 0 of wavefront w holds the W1 columns of
// hidden units nt*128 + 32 w .. +31 and block cb = 1 the W3 columns of the
// same units, so both products of a hidden unit land in the same lane.
// The source matrices are [in, out] per expert (W[e][k][n], K rows of Nw
// columns: x . W), so a lane gathers its 8 K values from 8 rows; lanes
// l % 32 read consecutive columns of one row, 64 bytes together.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ W0,
                                                           const uint16_t* __restrict__ W1,
                                                           int n_exp, int Nw, int K, int n_tiles,
                                                           int nk, int swiglu,
                                                           uint16_t* __restrict__ out) {
  const int64_t total = (int64_t)n_exp * n_tiles * nk * (kWStage / 16);
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int l = (int)(q & 63);
    const int cb = (int)((q >> 6) & 1);
    const int s = (int)((q >> 7) & 3);
    const int w = (int)((q >> 9) & 3);
    int64_t rest = q >> 11;
    const int kt = (int)(rest % nk);
    rest /= nk;
    const int nt = (int)(rest % n_tiles);
    const int e = (int)(rest / n_tiles);
    const int k = kt * BK + 16 * s + 8 * (l >> 5);
    int n;
    const uint16_t* src;
    if (swiglu) {
      n = nt * 128 + 32 * w + (l & 31);
      src = cb == 0 ? W0 : W1;
    } else {
      n = nt * 256 + 64 * w + 32 * cb + (l & 31);
      src = W0;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < Nw && k < K) {
      // K is a multiple of 8, so k < K covers k .. k + 7
      const uint16_t* col = src + ((int64_t)e * K + k) * Nw + n;
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = col[(int64_t)i * Nw];
      v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                h[6] | (h[7] << 16)};
    }
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
  const int nk = (K + BK - 1) / BK;
  g.nk = (nk + kP - 1) / kP * kP;
  g.bytes = (size_t)n_local * g.n_tiles * g.nk * kWStage;
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

namespace {
// expert_offset {0, B} of the shared expert: one lane per entry
__global__ void shared_offsets_kernel(int32_t* __restrict__ eo, int32_t B) {
  const int i = threadIdx.x;
  if (i < 2) eo[i] = i == 0 ? 0 : B;
}
}  // namespace

hipError_t launch_shared_ffn(const uint16_t* x, int64_t B, int d, int f, bool swiglu,
                             const void* wp, uint16_t* H, int32_t* eo, uint16_t* out,
                             hipStream_t s, hipEvent_t ev_stop, uint16_t* zsave) {
  if (B <= 0) return ev_stop ? hipEventRecord(ev_stop, s) : hipSuccess;
  hipLaunchKernelGGL(shared_offsets_kernel, dim3(1), dim3(64), 0, s, eo, (int32_t)B);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_expert_ffn(x, eo, 0, 1, (int)B, (int)B, d, f, swiglu, wp, H, out, s, nullptr,
                           ev_stop, nullptr, nullptr, nullptr, nullptr, 0, zsave);
}

hipError_t launch_expert_ffn(const uint16_t* packed, const int32_t* expert_offset, int e_begin,
                             int n_local, int rows_max, int rows_hint, int d, int f, bool swiglu,
                             const void* wp, uint16_t* H, uint16_t* ret, hipStream_t s,
                             hipEvent_t ev_start, hipEvent_t ev_stop, hipEvent_t ev_mid_end,
                             hipEvent_t ev_mid_start, const uint16_t* gx, const int32_t* gidx,
                             int64_t gx_rows, uint16_t* zsave) {
  if (n_local <= 0 || rows_max <= 0) {
    hipError_t e = hipSuccess;
    for (hipEvent_t ev : {ev_start, ev_mid_end, ev_mid_start, ev_stop})
      if (e == hipSuccess && ev) e = hipEventRecord(ev, s);
    return e;
  }
  // a 256-column tile does 2 * rows FLOP per weight byte; above ~384 rows per
  // expert the matrix cores, not the weight stream, set the pace (the
  // MI355X bf16 / HBM ridge is ~310 FLOP per byte)
  const bool mfma_bound = rows_hint >= 384;
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
  g1.n_local = n_local;
  if (gidx) {
    g1.A = gx;
    g1.gidx = gidx;
    g1.src_rows = gx_rows;
  }
  g1.Zs = zsave;
  g1.zs_w = expert_ffn_zw(f, swiglu);
  hipError_t err = swiglu ? launch_gemm<MODE_SWIGLU>(g1, m_tiles, mfma_bound, s, ev_start, ev_mid_end)
                          : launch_gemm<MODE_GELU>(g1, m_tiles, mfma_bound, s, ev_start, ev_mid_end);
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
  g2.n_local = n_local;
  return launch_gemm<MODE_PLAIN>(g2, m_tiles, mfma_bound, s, ev_mid_start, ev_stop);
}

}  // namespace moek

// ---------------------------------------------------------------------------
// Backward pass on the same grouped GEMM.
namespace moek {
namespace {

// Blocked layout (as pack_weights_kernel's) from output-major sources:
// weight-tile row n of K stage kt holds value(n, k) = srcA[e][n][k] for
// k < Ka and srcB[e][n][k - Ka] beyond (rows of Ka values; Ka a multiple of
// 8, so a lane's 8 K values come from one source as one 16-byte load).
__global__ __launch_bounds__(256) void pack_weights_nmajor_kernel(
    const uint16_t* __restrict__ srcA, const uint16_t* __restrict__ srcB, int Ka, int n_exp,
    int Nw, int K, int n_tiles, int nk, uint16_t* __restrict__ out) {
  const int64_t total = (int64_t)n_exp * n_tiles * nk * (kWStage / 16);
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int l = (int)(q & 63);
    const int cb = (int)((q >> 6) & 1);
    const int s = (int)((q >> 7) & 3);
    const int w = (int)((q >> 9) & 3);
    int64_t rest = q >> 11;
    const int kt = (int)(rest % nk);
    rest /= nk;
    const int nt = (int)(rest % n_tiles);
    const int e = (int)(rest / n_tiles);
    const int k = kt * BK + 16 * s + 8 * (l >> 5);
    const int n = nt * 256 + 64 * w + 32 * cb + (l & 31);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < Nw && k < K) {
      const uint16_t* src = k < Ka ? srcA : srcB;
      const int kk = k < Ka ? k : k - Ka;
      v = *(const u32x4*)(src + ((int64_t)e * Nw + n) * Ka + kk);
    }
    *(u32x4*)(out + q * 8) = v;
  }
}

int zw_of(int f, bool swiglu) { return swiglu ? geo(1, f, 8, true).n_tiles * 256 : f; }

// the two blocked backward matrices: dH's (N = f, K = d; rows of W2) and
// dX's (N = d, K = f or 2 f; rows of W1, then W3)
Geo geo_b1(int n_local, int d, int f) { return geo(n_local, f, d, false); }
Geo geo_b2(int n_local, int d, int f, bool swiglu) {
  return geo(n_local, d, swiglu ? 2 * f : f, false);
}

GemmArgs ffn_args(const uint16_t* A, const int32_t* eo, const void* Wp, uint16_t* Out,
                  int a_local, int o_local, int e_begin, int K, int Nout, const Geo& g,
                  int n_local) {
  GemmArgs a{};
  a.A = A;
  a.eo = eo;
  a.Wp = static_cast<const uint16_t*>(Wp);
  a.Out = Out;
  a.a_local = a_local;
  a.o_local = o_local;
  a.e_begin = e_begin;
  a.K = K;
  a.Nout = Nout;
  a.n_tiles_n = g.n_tiles;
  a.nk = g.nk;
  a.n_local = n_local;
  a.ldo = Nout;
  return a;
}

}  // namespace

int expert_ffn_zw(int f, bool swiglu) { return zw_of(f, swiglu); }

size_t packed_weights_bwd_bytes(int n_local, int d, int f, bool swiglu) {
  return geo_b1(n_local, d, f).bytes + geo_b2(n_local, d, f, swiglu).bytes;
}

hipError_t launch_pack_weights_bwd(const uint16_t* W1, const uint16_t* W3, const uint16_t* W2,
                                   int n_local, int d, int f, bool swiglu, void* wpb,
                                   hipStream_t s) {
  if (n_local <= 0) return hipSuccess;
  const Geo g1 = geo_b1(n_local, d, f), g2 = geo_b2(n_local, d, f, swiglu);
  uint16_t* o1 = static_cast<uint16_t*>(wpb);
  uint16_t* o2 = reinterpret_cast<uint16_t*>(static_cast<char*>(wpb) + g1.bytes);
  auto blocks = [](size_t bytes) {
    int64_t g = (int64_t)(bytes / 16 + 255) / 256;
    return (unsigned)(g > (1 << 20) ? (1 << 20) : g);
  };
  // dH = dret W2^T: value(n, k) = W2[e][n][k], n < f, k < d
  hipLaunchKernelGGL(pack_weights_nmajor_kernel, dim3(blocks(g1.bytes)), dim3(256), 0, s, W2,
                     nullptr, d, n_local, f, d, g1.n_tiles, g1.nk, o1);
  // dX = [dZ1 | dZ3] [W1 | W3]^T: value(n, k) = W1[e][n][k] (k < f), W3[e][n][k - f]
  hipLaunchKernelGGL(pack_weights_nmajor_kernel, dim3(blocks(g2.bytes)), dim3(256), 0, s, W1,
                     swiglu ? W3 : nullptr, f, n_local, d, swiglu ? 2 * f : f, g2.n_tiles, g2.nk,
                     o2);
  return hipGetLastError();
}

hipError_t launch_ffn_recompute(const uint16_t* xloc, const int32_t* expert_offset, int e_begin,
                                int n_local, int rows_max, int rows_hint, int d, int f,
                                bool swiglu, const void* wp, uint16_t* Z, hipStream_t s) {
  if (n_local <= 0 || rows_max <= 0) return hipSuccess;
  const Geo g1 = geo(n_local, f, d, swiglu);
  GemmArgs a = ffn_args(xloc, expert_offset, wp, Z, 1, 1, e_begin, d, zw_of(f, swiglu), g1,
                        n_local);
  return launch_gemm<MODE_PLAIN>(a, (rows_max + BM - 1) / BM, rows_hint >= 384, s);
}

hipError_t launch_ffn_dact(const uint16_t* dret, const int32_t* expert_offset, int e_begin,
                           int n_local, int rows_max, int rows_hint, int d, int f, bool swiglu,
                           const void* wpb, const uint16_t* Z, uint16_t* dZ, hipStream_t s) {
  if (n_local <= 0 || rows_max <= 0) return hipSuccess;
  const Geo g = geo_b1(n_local, d, f);
  GemmArgs a = ffn_args(dret, expert_offset, wpb, dZ, 0, 1, e_begin, d, f, g, n_local);
  a.Z = Z;
  a.zw = zw_of(f, swiglu);
  a.ldo = swiglu ? 2 * f : f;
  const int mt = (rows_max + BM - 1) / BM;
  return swiglu ? launch_gemm<MODE_DSWIGLU>(a, mt, rows_hint >= 384, s)
                : launch_gemm<MODE_DGELU>(a, mt, rows_hint >= 384, s);
}

hipError_t launch_ffn_dgrad(const uint16_t* dZ, const int32_t* expert_offset, int e_begin,
                            int n_local, int rows_max, int rows_hint, int d, int f, bool swiglu,
                            const void* wpb, uint16_t* dxp, hipStream_t s) {
  if (n_local <= 0 || rows_max <= 0) return hipSuccess;
  const Geo g1 = geo_b1(n_local, d, f), g2 = geo_b2(n_local, d, f, swiglu);
  const void* w2 = static_cast<const char*>(wpb) + g1.bytes;
  GemmArgs a = ffn_args(dZ, expert_offset, w2, dxp, 1, 0, e_begin, swiglu ? 2 * f : f, d, g2,
                        n_local);
  return launch_gemm<MODE_PLAIN>(a, (rows_max + BM - 1) / BM, rows_hint >= 384, s);
}

}  // namespace moek
