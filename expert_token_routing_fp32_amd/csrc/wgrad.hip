// Grouped "K-fragment" GEMM on bf16 matrix cores for the backward pass:
//   C_g[m][n] = sum_s sum_k A_s,g(m, k) B_s,g(n, k)        (fp32 accumulation)
// over groups g (experts, or slices of a long contraction) and up to six
// operand pairs s (segments) that share the contraction length K_g.  Used
// for the weight gradients of the experts (the contraction runs over an
// expert's rows: dW2 = H^T dret, [dW1 | dW3] = X^T [dZ1 | dZ3]) and for the
// router's gradients (dWg and the bias gradient over the tokens, dx =
// dlogits Wg^T over the experts), the fp32 router operands split exactly
// into bf16 parts.
//
// Operands are in the RB8 layout: fragment (kg, m) -- the 8 values
// k = 8 kg .. 8 kg + 7 of row m -- is the 16 bytes at ((kg W + m) 8)
// elements from the group's base, so one k group of 256 consecutive rows is
// 4 KB of contiguous memory.  K_g is padded with zero fragments to a
// multiple of 32.
//
// Tile 256 x 256, K in stages of 32, per workgroup of 4 wavefronts (one
// per SIMD, one workgroup per CU, persistent over a range of tiles): each
// wavefront computes all 256 rows against its own 64 columns (8 x 2 blocks
// of v_mfma_f32_32x32x16_bf16, accumulators in the AGPRs).  A, shared by
// the four, goes global -> LDS by buffer loads that write LDS directly into
// a 4-slot ring (wavefront w loads k group w, 4 loads of 64 x 16 bytes per
// stage); each wavefront's B fragments go global -> registers into a 4-slot
// register ring (4 loads per stage); both three stages ahead, loads past a
// group's data reading zeros.  Vector-memory loads complete in issue order,
// so waiting until one stage's loads are outstanding means the two oldest
// stages have landed; one barrier per stage then makes every wavefront's A
// parts visible and frees the slot the next issue overwrites.
#include "moe_kernels.h"

namespace moek {
namespace {

typedef __bf16 kb16x8 __attribute__((ext_vector_type(8)));
typedef float kf32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void k_lds_void_t;

constexpr int KBM = 256, KBN = 256;
constexpr int KPL = 256;                   // 16-byte chunks per k group in LDS
constexpr int KSLOT = 4 * KPL * 16;        // one stage of A in LDS: 16 KB
constexpr int KR = 4;                      // ring slots (LDS for A, registers for B)
constexpr int KLOADS = 4 + 4;              // loads per wavefront per stage: A to LDS, B
constexpr int KSTG_ROW = 64 + 4;           // floats per row of the epilogue staging (padded)
constexpr int KSTG_WAVE = 32 * KSTG_ROW * 4;  // a wavefront's staging area: 32 rows x 64 columns

struct KArgsDev {
  const uint16_t* A[6];
  const uint16_t* Bm[6];
  int nseg;
  int a_w, b_w;              // RB8 widths (columns) of A and B
  int64_t a_es, b_es;        // per-group element offsets
  int64_t a_bytes, b_bytes;  // bytes of each segment's operand from its base
  const int32_t* eo;         // K_g = eo[e_begin + g + 1] - eo[e_begin + g] when set
  int e_begin;
  int Kc;                    // otherwise this K (split-K: group g takes rows g Kc ..
  int Ktot;                  // .. min((g + 1) Kc, Ktot) when Ktot > 0)
  int tiles_m, tiles_n;
  int groups;
  int mode;                  // 0: fp32 store to C0 / C1; 1: (acc + add) stored as bf16 / fp32
  float* C0;
  int64_t ldc0, c0_es;
  int M0, N0;
  float* C1;
  int64_t ldc1, c1_es;
  int r1, col1, M1, N1;
  const float* add;
  int64_t ld_add;
  void* xo;
  int x_bf16;
};

template <int N>
__device__ __forceinline__ void k_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// lds: a 32-bit LDS offset (a generic pointer would cost a null check per load)
__device__ __forceinline__ void k_dma16(rsrc_t rs, uint32_t off, uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (k_lds_void_t*)(uintptr_t)lds, 16, off, 0, 0, 0);
}

// one accumulator element, read out of the accumulation registers where it
// is used
__device__ __forceinline__ float kacc(float x) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
  return v;
}

// one output element
__device__ __forceinline__ void kstore(const KArgsDev& a, int g, int m, int n, float v) {
  if (a.mode == 0) {
    if (m < a.M0 && n < a.N0) {
      a.C0[(int64_t)g * a.c0_es + (int64_t)m * a.ldc0 + n] = v;
    } else if (a.C1) {
      const int mm = m - a.r1, nn = n - a.col1;
      if (mm >= 0 && mm < a.M1 && nn >= 0 && nn < a.N1)
        a.C1[(int64_t)g * a.c1_es + (int64_t)mm * a.ldc1 + nn] = v;
    }
  } else if (m < a.M0 && n < a.N0) {
    const float o = v + (a.add ? a.add[(int64_t)m * a.ld_add + n] : 0.f);
    const int64_t off = (int64_t)m * a.ldc0 + n;
    if (a.x_bf16)
      static_cast<uint16_t*>(a.xo)[off] = (uint16_t)f32_to_bf16(o);
    else
      static_cast<float*>(a.xo)[off] = o;
  }
}

// four consecutive output elements (n .. n + 3) of row m: one 16-byte fp32
// store (8-byte bf16) when they all fall inside C0 (or the stored output)
// and the destination is aligned, element by element otherwise
__device__ __forceinline__ void kstore4(const KArgsDev& a, int g, int m, int n, f32x4 v) {
  if (a.mode == 0) {
    if (m < a.M0 && n + 3 < a.N0 && (a.ldc0 & 3) == 0) {
      float* p = a.C0 + (int64_t)g * a.c0_es + (int64_t)m * a.ldc0 + n;
      if ((reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
        *reinterpret_cast<f32x4*>(p) = v;
        return;
      }
    } else if (a.C1 && n >= a.N0 && (a.ldc1 & 3) == 0) {
      // all four in the second output (dW3 beside dW1)
      const int mm = m - a.r1, nn = n - a.col1;
      if (mm >= 0 && mm < a.M1 && nn >= 0 && nn + 3 < a.N1) {
        float* p = a.C1 + (int64_t)g * a.c1_es + (int64_t)mm * a.ldc1 + nn;
        if ((reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
          *reinterpret_cast<f32x4*>(p) = v;
          return;
        }
      }
    }
  } else if (m < a.M0 && n + 3 < a.N0 && (a.ldc0 & 3) == 0 && (a.ld_add & 3) == 0) {
    const int64_t off = (int64_t)m * a.ldc0 + n;
    const float* ap = a.add ? a.add + (int64_t)m * a.ld_add + n : nullptr;
    if ((!ap || (reinterpret_cast<uintptr_t>(ap) & 15u) == 0)) {
      f32x4 o = v;
      if (ap) o += *reinterpret_cast<const f32x4*>(ap);
      if (a.x_bf16) {
        uint16_t* q = static_cast<uint16_t*>(a.xo) + off;
        if ((reinterpret_cast<uintptr_t>(q) & 7u) == 0) {
          *reinterpret_cast<u32x2*>(q) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          return;
        }
      } else {
        float* q = static_cast<float*>(a.xo) + off;
        if ((reinterpret_cast<uintptr_t>(q) & 15u) == 0) {
          *reinterpret_cast<f32x4*>(q) = o;
          return;
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) kstore(a, g, m, n + u, v[u]);
}

// bytes of an operand readable from group g's base (0 past the end)
__device__ __forceinline__ uint32_t kbytes(int64_t total, int64_t es, int g) {
  const int64_t left = total - 2 * es * g;
  return left > 0 ? (uint32_t)(left < 0x7fffffffLL ? left : 0x7fffffffLL) : 0u;
}

// A tile: 256 x 256 outputs of group g at (m0, n0), nst stages of 32 k
// (nks per segment).
struct KTile {
  int g, m0, n0, nks, nst;
};

__device__ __forceinline__ KTile ktile(const KArgsDev& a, int64_t t) {
  const int tiles = a.tiles_m * a.tiles_n;
  KTile r;
  r.g = (int)(t / tiles);
  const int tile = (int)(t % tiles);
  r.m0 = tile / a.tiles_n * KBM;
  r.n0 = tile % a.tiles_n * KBN;
  int K;
  if (a.eo) {
    K = a.eo[a.e_begin + r.g + 1] - a.eo[a.e_begin + r.g];
    K = (K + 31) / 32 * 32;
  } else {
    K = a.Kc;
    if (a.Ktot > 0) {
      const int left = a.Ktot - r.g * a.Kc;
      K = left < K ? left : K;
      K = K > 0 ? K : 0;
    }
  }
  r.nks = K / 32;
  r.nst = r.nks * a.nseg;
  return r;
}

// Block row I of the accumulators (32 rows x this wavefront's 64 columns)
// through the wavefront's staging area `stg`: written in the accumulator
// layout, read back as rows -- RV[t] holds row 4 t + lane / 16, columns
// 4 (lane % 16) .. + 3 of the block row.  All eight reads are issued before
// any is used (one read per use, each waited for, would serialize the LDS
// latency).  LDS operations of one wavefront complete in order, so the
// reads see the writes and the next block row's writes wait for the reads.
#define KSTAGE_ROWS(I, RV)                                                               \
  {                                                                                      \
    _Pragma("unroll") for (int j_ = 0; j_ < 2; ++j_)                                     \
      _Pragma("unroll") for (int q_ = 0; q_ < 4; ++q_)                                   \
        *reinterpret_cast<f32x4*>(stg + l32 * KSTG_ROW + 32 * j_ + 8 * q_ + 4 * lh) =    \
            f32x4{kacc(acc[I][j_][4 * q_]), kacc(acc[I][j_][4 * q_ + 1]),                \
                  kacc(acc[I][j_][4 * q_ + 2]), kacc(acc[I][j_][4 * q_ + 3])};           \
    asm volatile("" ::: "memory");                                                       \
    _Pragma("unroll") for (int t_ = 0; t_ < 8; ++t_)                                     \
      RV[t_] = *reinterpret_cast<const f32x4*>(stg + (4 * t_ + (lane >> 4)) * KSTG_ROW + \
                                               4 * (lane & 15));                         \
    __builtin_amdgcn_sched_barrier(0);                                                   \
  }

// Epilogue of the tile (g, m0, n0): the B fragment is the matrix
// instruction's first operand, so acc[i][j] holds the block transposed:
// registers 4q .. 4q + 3 of lane l are C[m][n .. n + 3] with m = m0 + 32 i +
// l % 32 and n = n0 + 64 wave + 32 j + 8 q + 4 (l / 32) -- four consecutive
// columns of one row.  The common case -- a mode-0 tile wholly inside one of
// the two outputs, rows 16-byte aligned -- stores unconditionally; other
// tiles go element by element through kstore4.
__device__ __forceinline__ void kgemm_epilogue(const KArgsDev& a, char* smem, kf32x16 (&acc)[8][2],
                                               int g, int m0, int n0, int wave, int lane) {
  const int l32 = lane & 31, lh = lane >> 5;
  float* fbase = nullptr;
  int64_t fld = 0;
  if (a.mode == 0 && m0 + KBM <= a.M0) {
    if (n0 + KBN <= a.N0 && (a.ldc0 & 3) == 0) {
      fbase = a.C0 + (int64_t)g * a.c0_es + (int64_t)m0 * a.ldc0 + n0;
      fld = a.ldc0;
    } else if (a.C1 && n0 >= a.N0 && (a.ldc1 & 3) == 0 && m0 - a.r1 >= 0 &&
               m0 + KBM - a.r1 <= a.M1 && n0 - a.col1 >= 0 && n0 + KBN - a.col1 <= a.N1) {
      fbase = a.C1 + (int64_t)g * a.c1_es + (int64_t)(m0 - a.r1) * a.ldc1 + (n0 - a.col1);
      fld = a.ldc1;
    }
    if (reinterpret_cast<uintptr_t>(fbase) & 15u) fbase = nullptr;
  }
  // mode 1 (out = acc + add, stored as bf16 or fp32) on a full tile with
  // 16-byte aligned rows: unconditional vector loads and stores too
  if (a.mode == 1 && m0 + KBM <= a.M0 && n0 + KBN <= a.N0 && (a.ldc0 & 3) == 0 &&
      (!a.add || (a.ld_add & 3) == 0)) {
    const float* ab = a.add ? a.add + (int64_t)m0 * a.ld_add + n0 : nullptr;
    const int64_t o0 = (int64_t)m0 * a.ldc0 + n0;
    const bool al = (!ab || (reinterpret_cast<uintptr_t>(ab) & 15u) == 0) &&
                    (a.x_bf16 ? (reinterpret_cast<uintptr_t>(static_cast<uint16_t*>(a.xo) + o0) & 7u) == 0
                              : (reinterpret_cast<uintptr_t>(static_cast<float*>(a.xo) + o0) & 15u) == 0);
    if (al) {
      // opaque, so that the per-row offsets are not hoisted out of the tile
      // loop (and spilled)
      int64_t ldo = a.ldc0, lda = a.ld_add;
      asm volatile("" : "+s"(ldo), "+s"(lda));
      // rows through the staging area as in the mode-0 case below; the
      // addend rows are loaded first, so their latency overlaps the staging
      float* stg = reinterpret_cast<float*>(smem + KR * KSLOT + wave * KSTG_WAVE);
      const int rr = lane >> 4, cc = 4 * (lane & 15);
      const int64_t orow = o0 + (int64_t)rr * ldo + 64 * wave + cc;
      const float* ar = ab ? ab + (int64_t)rr * lda + 64 * wave + cc : nullptr;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f32x4 ad[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          ad[t] = ar ? *reinterpret_cast<const f32x4*>(ar + (int64_t)(32 * i + 4 * t) * lda)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 rv[8];
        KSTAGE_ROWS(i, rv)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const f32x4 v = rv[t] + ad[t];
          const int64_t off = orow + (int64_t)(32 * i + 4 * t) * ldo;
          if (a.x_bf16)
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.xo) + off) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          else
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.xo) + off) = v;
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
  }
  if (fbase) {
    // Each block row goes through the wavefront's own staging area in LDS
    // (outside the ring, so no barrier) and is stored 4 rows x 256
    // contiguous bytes per instruction.  Stored straight from the
    // accumulators, every instruction would touch 32 rows with 32 bytes
    // each, and the stores, issued at a fraction of the rate, would take as
    // long as a quarter of the tile's matrix work.
    float* stg = reinterpret_cast<float*>(smem + KR * KSLOT + wave * KSTG_WAVE);
    // opaque, so that the per-row offsets are not all hoisted out of the
    // tile loop (and spilled)
    asm volatile("" : "+s"(fld));
    const int rr = lane >> 4, cc = 4 * (lane & 15);
    float* ob = fbase + 64 * wave + (int64_t)rr * fld + cc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 rv[8];
      KSTAGE_ROWS(i, rv)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<f32x4*>(ob + (int64_t)(32 * i + 4 * t) * fld) = rv[t];
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  // other tiles: each 32 x 32 block through the wavefront's staging area;
  // the unrolled part only moves registers to LDS, and the stores, with
  // their bounds and destinations, run in a plain loop of 4 rounds in which
  // lanes write consecutive columns
  float* stg = reinterpret_cast<float*>(smem + KR * KSLOT + wave * KSTG_WAVE);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(stg + l32 * 32 + 8 * q + 4 * lh) =
            f32x4{kacc(acc[i][j][4 * q]), kacc(acc[i][j][4 * q + 1]), kacc(acc[i][j][4 * q + 2]),
                  kacc(acc[i][j][4 * q + 3])};
      // LDS operations of one wavefront complete in order; the compiler
      // barrier keeps the reads below the writes (and the next block's
      // writes below these reads)
      asm volatile("" ::: "memory");
      const int mb = m0 + 32 * i, nb = n0 + 64 * wave + 32 * j;
      // four rounds: lane -> row 8 r + lane / 8, columns 4 (lane % 8) .. + 3
#pragma unroll 1
      for (int r = 0; r < 4; ++r) {
        const int row = 8 * r + (lane >> 3), c4 = 4 * (lane & 7);
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + row * 32 + c4);
        kstore4(a, g, mb + row, nb + c4, v);
      }
      asm volatile("" ::: "memory");
    }
}


#undef KSTAGE_ROWS

// Persistent: one workgroup per CU walks the tiles, ordered (group, tile)
// and cut into 8 equal contiguous ranges, one per XCD (workgroups are dealt
// round-robin over the XCDs), so an XCD works on few groups at a time and
// their operands are shared through its L2.  (One launch of a workgroup per
// tile left a fifth of the CUs idle: the in-order dispatch of workgroups
// waits for the XCD whose turn it is.)
__global__ __launch_bounds__(256, 1) void kgemm_kernel(KArgsDev a) {
  __shared__ __attribute__((aligned(16))) char smem[KR * KSLOT + 4 * KSTG_WAVE];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const int tiles = a.tiles_m * a.tiles_n;
  const int64_t total = (int64_t)tiles * a.groups;
  const int G = gridDim.x, b = blockIdx.x;
  int64_t t0, t1, step;
  if (G >= 8) {
    const int x = b % 8, j = b / 8, nx = G / 8;
    if (j >= nx) return;
    t0 = total * x / 8 + j;
    t1 = total * (x + 1) / 8;
    step = nx;
  } else {
    t0 = b;
    t1 = total;
    step = G;
  }
  if (t0 >= t1) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lo16 = 16u * lane;
  const int l32 = lane & 31, lh = lane >> 5;
  KTile ct = ktile(a, t0);
  // The segment's descriptors are built when the segment changes (csg = -1
  // for a new tile), not on every stage: their base pointers come from the
  // kernel arguments through scalar loads whose wait would otherwise open
  // every stage.
  int csg = -1;
  rsrc_t ra, rb;
  // Each wavefront computes all 256 rows of the tile against its own 64
  // columns n0 + 64 wave .. + 63: A (shared by the four) comes through LDS,
  // B (this wavefront's alone) straight from memory into registers.
  // B fragments of a stage: [slot][half][column block]
  u32x4 bq[KR][2][2];
  // Issue of the next stage into slot SLOT (after the last stage the issues
  // reload it, and nobody reads it again, so every stage issues the same
  // loads), in 8 parts: A's k group `wave` (rows m0 .. m0 + 255, parts 0-3,
  // 64 chunks each) into LDS slot SLOT, then this wavefront's B fragments
  // (the lane's k groups 2 h + lh; parts 4-7) into registers bq[SLOT].
  // KSEG sets the stage's descriptors and offsets; KPART issues one part.
  // The stages of a tile are issued in order, so the stage (is_st), its
  // segment (is_seg) and its k step in the segment (is_k) are counters
  // advanced by one per issue, up to the last stage: no division of the
  // stage index by the steps per segment (a scalar division of some 70
  // instructions ahead of every stage's barrier).
  uint32_t ia_la = 0, ia_oa = 0, ia_kq = 0;
  int is_st = 0, is_k = 0, is_seg = 0;
#define KSEG(SLOT)                                                                     \
  {                                                                                    \
    ia_kq = (uint32_t)is_k * 4;                                                        \
    if (is_seg != csg) {                                                               \
      ra = make_rsrc(a.A[is_seg] + (int64_t)ct.g * a.a_es, kbytes(a.a_bytes, a.a_es, ct.g)); \
      rb = make_rsrc(a.Bm[is_seg] + (int64_t)ct.g * a.b_es, kbytes(a.b_bytes, a.b_es, ct.g)); \
      csg = is_seg;                                                                    \
    }                                                                                  \
    if (is_st < ct.nst - 1) {                                                          \
      ++is_st;                                                                         \
      if (++is_k == ct.nks) {                                                          \
        is_k = 0;                                                                      \
        ++is_seg;                                                                      \
      }                                                                                \
    }                                                                                  \
    ia_la = smem_lds + (SLOT) * KSLOT + wave * KPL * 16;                               \
    ia_oa = 16u * ((ia_kq + wave) * (uint32_t)a.a_w + (uint32_t)ct.m0) + lo16;         \
  }
#define KPART(Q, SLOT)                                                                 \
  {                                                                                    \
    if ((Q) < 4) {                                                                     \
      k_dma16(ra, ia_oa + 1024u * ((Q) & 3), ia_la + 1024 * ((Q) & 3));                \
    } else {                                                                           \
      constexpr int h_ = ((Q) - 4) >> 1, j_ = ((Q) - 4) & 1;                           \
      bq[SLOT][h_][j_] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128( \
          rb, 16u * ((ia_kq + 2 * h_ + lh) * (uint32_t)a.b_w +                         \
                     (uint32_t)(ct.n0 + 64 * wave + 32 * j_ + l32)), 0, 0));            \
    }                                                                                  \
  }
#define KISSUE(SLOT)                                                                   \
  {                                                                                    \
    KSEG(SLOT)                                                                         \
    KPART(0, SLOT) KPART(1, SLOT) KPART(2, SLOT) KPART(3, SLOT)                        \
    KPART(4, SLOT) KPART(5, SLOT) KPART(6, SLOT) KPART(7, SLOT)                        \
  }
  // Stage ST in slot U: wait until stages ST and ST + 1 have landed (one
  // stage's loads outstanding: they complete in issue order), a barrier that
  // makes every wavefront's A parts visible and retires the reads of the
  // slot the issue below refills; then 16 groups of 2 MFMAs (half h, row
  // block i) with, after group (h, i), the LDS read of the fragment that
  // group frees -- the second half's during the first, the next stage's
  // first half during the second -- and after every second group one part
  // of the issue of stage ST + KR - 1, spread so that a load whose issue
  // stalls does not hold the matrix core for long.
#define KGROUP(U, H, I)                                                                \
  {                                                                                    \
    _Pragma("unroll") for (int j_ = 0; j_ < 2; ++j_)                                   \
      acc[I][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                            \
          __builtin_bit_cast(kb16x8, bq[U][H][j_]), fa[H][I], acc[I][j_], 0, 0, 0);    \
    if ((H) == 0)                                                                      \
      fa[1][I] = __builtin_bit_cast(kb16x8, sa_[(2 + lh) * KPL + l32 + (I) * 32]);     \
    else                                                                               \
      fa[0][I] = __builtin_bit_cast(kb16x8, sn_[lh * KPL + l32 + (I) * 32]);            \
    if ((I) & 1) KPART(4 * (H) + ((I) >> 1), ((U) + KR - 1) % KR)                      \
    __builtin_amdgcn_sched_barrier(0);                                                 \
  }
#define KSTAGE(ST, U)                                                                  \
  {                                                                                    \
    k_wait_vmcnt<(KR - 3) * KLOADS>();                                                 \
    asm volatile("" ::: "memory");                                                     \
    __builtin_amdgcn_s_barrier();                                                      \
    asm volatile("" ::: "memory");                                                     \
    KSEG(((U) + KR - 1) % KR)                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                 \
    const u32x4* sa_ = reinterpret_cast<const u32x4*>(smem + (U) * KSLOT);             \
    const u32x4* sn_ = reinterpret_cast<const u32x4*>(smem + (((U) + 1) % KR) * KSLOT); \
    KGROUP(U, 0, 0) KGROUP(U, 0, 1) KGROUP(U, 0, 2) KGROUP(U, 0, 3)                    \
    KGROUP(U, 0, 4) KGROUP(U, 0, 5) KGROUP(U, 0, 6) KGROUP(U, 0, 7)                    \
    KGROUP(U, 1, 0) KGROUP(U, 1, 1) KGROUP(U, 1, 2) KGROUP(U, 1, 3)                    \
    KGROUP(U, 1, 4) KGROUP(U, 1, 5) KGROUP(U, 1, 6) KGROUP(U, 1, 7)                    \
  }

  for (int64_t t = t0; t < t1; t += step) {
    if (t != t0) {
      ct = ktile(a, t);
      csg = -1;
    }
    is_st = is_k = is_seg = 0;
    if (ct.nst > 0) {
      KISSUE(0)
      KISSUE(1)
      KISSUE(2)
    }
    kf32x16 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (ct.nst > 0) {
      const int nst = ct.nst;
      // A fragments: fa[0] the current stage's first half, read during the
      // previous stage; fa[1] its second half
      kb16x8 fa[2][8];
      // stage 0 has landed (stage 1 may not yet): the first half's fragments
      k_wait_vmcnt<2 * KLOADS>();
      __builtin_amdgcn_s_barrier();
      {
        const u32x4* s0_ = reinterpret_cast<const u32x4*>(smem);
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[0][i] = __builtin_bit_cast(kb16x8, s0_[lh * KPL + l32 + i * 32]);
      }
      // whole groups of KR stages (register slots fixed at compile time),
      // then the remainder
      const int nfull = nst - nst % KR;
      for (int st0 = 0; st0 < nfull; st0 += KR) {
        KSTAGE(st0, 0)
        KSTAGE(st0 + 1, 1)
        KSTAGE(st0 + 2, 2)
        KSTAGE(st0 + 3, 3)
      }
      if (nst - nfull > 0) KSTAGE(nfull, 0)
      if (nst - nfull > 1) KSTAGE(nfull + 1, 1)
      if (nst - nfull > 2) KSTAGE(nfull + 2, 2)
      // The reloads past the end land before the epilogue.  Left in flight,
      // they reach the next tile's first stages on the path through the
      // remainder stages above, and the compiler, which cannot tell that
      // path's register slots from the loop's, then waits for nearly all of
      // the two stages ahead at the start of every group of KR stages.
      k_wait_vmcnt<0>();
      // every wavefront is done reading the ring before the next tile's
      // loads refill it (each wavefront's loads land in issue order, and the
      // epilogue does not use the ring)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    kgemm_epilogue(a, smem, acc, ct.g, ct.m0, ct.n0, wave, lane);
  }
#undef KSTAGE
#undef KGROUP
#undef KISSUE
#undef KPART
#undef KSEG
}

}  // namespace

hipError_t launch_kgemm(const KGemm& q, hipStream_t s) {
  if (q.groups <= 0 || q.M <= 0 || q.N <= 0) return hipSuccess;
  KArgsDev a{};
  if (q.nseg < 1 || q.nseg > 6) return hipErrorInvalidValue;
  for (int i = 0; i < q.nseg; ++i) {
    a.A[i] = q.A[i];
    a.Bm[i] = q.B[i];
  }
  a.nseg = q.nseg;
  a.a_w = q.a_w;
  a.b_w = q.b_w;
  a.a_es = q.a_es;
  a.b_es = q.b_es;
  a.a_bytes = q.a_bytes;
  a.b_bytes = q.b_bytes;
  a.eo = q.eo;
  a.e_begin = q.e_begin;
  a.Kc = (q.K + 31) / 32 * 32;
  a.Ktot = q.Ktot > 0 ? (q.Ktot + 31) / 32 * 32 : 0;
  a.tiles_m = (q.M + KBM - 1) / KBM;
  a.tiles_n = (q.N + KBN - 1) / KBN;
  a.mode = q.mode;
  a.C0 = q.C0;
  a.ldc0 = q.ldc0;
  a.c0_es = q.c0_es;
  a.M0 = q.M0;
  a.N0 = q.N0;
  a.C1 = q.C1;
  a.ldc1 = q.ldc1;
  a.c1_es = q.c1_es;
  a.r1 = q.r1;
  a.col1 = q.col1;
  a.M1 = q.M1;
  a.N1 = q.N1;
  a.add = q.add;
  a.ld_add = q.ld_add;
  a.xo = q.xo;
  a.x_bf16 = q.x_bf16;
  // every byte offset inside one group's operand is 32-bit: the groups'
  // extents (or the whole operand for one group) stay below 2 GB, and so
  // do the offsets the tiles reach (k groups x width x 16 bytes)
  const int64_t ga = q.a_es > 0 ? 2 * q.a_es : q.a_bytes;
  const int64_t gb = q.b_es > 0 ? 2 * q.b_es : q.b_bytes;
  if (ga > 0x7fffffffLL || gb > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t kmax = q.eo ? 0 : a.Kc;
  if (kmax > 0 && ((int64_t)kmax / 8 * q.a_w * 16 > 0x7fffffffLL ||
                   (int64_t)kmax / 8 * q.b_w * 16 > 0x7fffffffLL))
    return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles > 2147483647 || q.groups > 65535) return hipErrorInvalidValue;
  a.groups = q.groups;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t total = tiles * q.groups;
  const int grid = (int)(total < cus ? total : cus);
  hipLaunchKernelGGL(kgemm_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moek
