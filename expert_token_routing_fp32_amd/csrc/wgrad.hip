// Grouped "K-fragment" GEMM on bf16 matrix cores for the backward pass:
//   C_g[m][n] = sum_s sum_k A_s,g(m, k) B_s,g(n, k)        (fp32 accumulation)
// over groups g (experts) and up to six operand pairs s (segments) that
// share the contraction length K_g.  Used for the weight gradients of the
// experts (the contraction runs over an expert's rows: dW2 = H^T dret,
// [dW1 | dW3] = X^T [dZ1 | dZ3]) and for the router's gradients (dWg and the
// bias gradient over the tokens, dx = dlogits Wg^T over the experts), the
// fp32 router operands split exactly into bf16 parts.
//
// Operands are read as 16-byte K fragments: fragment (kg, m) -- the 8
// values k = 8 kg .. 8 kg + 7 of row m -- at element base + kg sg + m sm.
// Two layouts give that:
//   RB8  (sm = 8, sg = 8 W): 8 consecutive rows of one column contiguous
//        (the re-layout kernels write it), for contractions over rows;
//   ROW  (sm = ld, sg = 8): plain row-major with K contiguous.
// K_g (rows of expert g, or a constant) is padded with zero fragments to a
// multiple of 32 in the operands.
//
// Tile 128 x 128 x 32 per workgroup of 4 wavefronts (2 x 2, each 64 x 64 =
// 2 x 2 blocks of v_mfma_f32_32x32x16_bf16); LDS double buffer, one
// barrier per 32-deep stage; the next stage's global loads are in flight
// while the current one is multiplied.
#include "moe_kernels.h"

namespace moek {
namespace {

typedef __bf16 kb16x8 __attribute__((ext_vector_type(8)));
typedef float kf32x16 __attribute__((ext_vector_type(16)));

constexpr int KBM = 128, KBN = 128;
// 16-byte chunks per LDS plane (one 8-deep k group): 128 + 4 pad, so that
// the four planes start 16 banks apart (the row-major store pattern writes
// four planes' chunks of one row together)
constexpr int KPL = 132;

struct KArgsDev {
  const uint16_t* A[6];
  const uint16_t* Bm[6];
  int nseg;
  int64_t a_sm, a_sg, a_es;
  int64_t b_sm, b_sg, b_es;
  int Ma, Nb;
  const int32_t* eo;  // K_g = eo[e_begin + g + 1] - eo[e_begin + g] when set
  int e_begin;
  int Kc;             // otherwise this K (split-K: group g takes rows g Kc ..
  int Ktot;           // .. min((g + 1) Kc, Ktot) when Ktot > 0)
  int tiles_m, tiles_n;
  int mode;           // 0: fp32 store to C0 / C1; 1: (acc + add) stored as bf16 / fp32
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

// one 16-byte fragment of operand p at (kg, m): clamped to a valid row m
__device__ __forceinline__ u32x4 kfrag(const uint16_t* p, int64_t sm, int64_t sg, int kg, int m) {
  return *(const u32x4*)(p + (int64_t)kg * sg + (int64_t)m * sm);
}

template <bool AROW, bool BROW>
__global__ __launch_bounds__(256) void kgemm_kernel(KArgsDev a) {
  __shared__ __attribute__((aligned(16))) u32x4 sa[2][4 * KPL];
  __shared__ __attribute__((aligned(16))) u32x4 sb[2][4 * KPL];
  const int g = blockIdx.y;
  const int tm = blockIdx.x / a.tiles_n, tn = blockIdx.x % a.tiles_n;
  const int m0 = tm * KBM, n0 = tn * KBN;
  int K;
  if (a.eo) {
    K = a.eo[a.e_begin + g + 1] - a.eo[a.e_begin + g];
    K = (K + 31) / 32 * 32;
  } else {
    K = a.Kc;
    if (a.Ktot > 0) {
      const int left = a.Ktot - g * a.Kc;
      K = left < K ? left : K;
      K = K > 0 ? K : 0;
    }
  }
  const int nks = K / 32;  // stages per segment
  const int nst = nks * a.nseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register mapping of one stage: 512 chunks per operand, two per
  // thread.  RB8: chunk q -> (kg = q / 128, m = q % 128), consecutive
  // threads read consecutive 16-byte chunks of one k group.  ROW: chunk q ->
  // (m = q / 4, kg = q % 4), 64 contiguous bytes of a row per 4 threads.
  int am[2], ak[2], bm_[2], bk[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = tid + 256 * h;
    am[h] = AROW ? q >> 2 : q & 127;
    ak[h] = AROW ? q & 3 : q >> 7;
    bm_[h] = BROW ? q >> 2 : q & 127;
    bk[h] = BROW ? q & 3 : q >> 7;
  }
  int amc[2], bmc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ma = m0 + am[h], nb = n0 + bm_[h];
    amc[h] = ma < a.Ma ? ma : a.Ma - 1;
    bmc[h] = nb < a.Nb ? nb : a.Nb - 1;
  }
  u32x4 ra[2], rb[2];
  auto gload = [&](int st) {
    const int sgm = st / nks, kg0 = (st - sgm * nks) * 4;
    const uint16_t* A = a.A[sgm] + (int64_t)g * a.a_es;
    const uint16_t* Bp = a.Bm[sgm] + (int64_t)g * a.b_es;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = kfrag(A, a.a_sm, a.a_sg, kg0 + ak[h], amc[h]);
      rb[h] = kfrag(Bp, a.b_sm, a.b_sg, kg0 + bk[h], bmc[h]);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sa[buf][ak[h] * KPL + am[h]] = ra[h];
      sb[buf][bk[h] * KPL + bm_[h]] = rb[h];
    }
  };

  kf32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nst > 0) {
    gload(0);
    swrite(0);
    __syncthreads();
  }
  const int l32 = lane & 31, lh = lane >> 5;
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int kgl = 2 * s2 + lh;  // this lane's k group in the stage
      kb16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = __builtin_bit_cast(kb16x8, sa[buf][kgl * KPL + wm * 64 + i * 32 + l32]);
        fb[i] = __builtin_bit_cast(kb16x8, sb[buf][kgl * KPL + wn * 64 + i * 32 + l32]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < nst) swrite(buf ^ 1);
    __syncthreads();
  }

  // epilogue: acc[i][j][r] is C[m][n] with m = m0 + 64 wm + 32 i + 8 (r / 4)
  // + 4 lh + r % 4 and n = n0 + 64 wn + 32 j + l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int n = n0 + 64 * wn + 32 * j + l32;
        const float v = acc[i][j][r];
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
  a.a_sm = q.a_row ? q.a_ld : 8;
  a.a_sg = q.a_row ? 8 : (int64_t)8 * q.a_w;
  a.a_es = q.a_es;
  a.b_sm = q.b_row ? q.b_ld : 8;
  a.b_sg = q.b_row ? 8 : (int64_t)8 * q.b_w;
  a.b_es = q.b_es;
  a.Ma = q.a_rows;
  a.Nb = q.b_rows;
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
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles > 2147483647 || q.groups > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles, (unsigned)q.groups);
  if (q.a_row && q.b_row)
    hipLaunchKernelGGL((kgemm_kernel<true, true>), grid, dim3(256), 0, s, a);
  else if (q.a_row)
    hipLaunchKernelGGL((kgemm_kernel<true, false>), grid, dim3(256), 0, s, a);
  else if (q.b_row)
    hipLaunchKernelGGL((kgemm_kernel<false, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kgemm_kernel<false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moek
