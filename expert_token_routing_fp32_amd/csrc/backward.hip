// Backward pass of the MoE layer: the bandwidth-bound steps and the
// operand re-layouts of the weight-gradient GEMMs.
//
// "Expert Parallelism" (narrativegoldmine.com), "About": the sparsely gated
// layer is trained by backpropagation with an auxiliary load-balancing loss;
// "Formal Algorithm": the auxiliary loss is added to the training loss.  The
// loss is L = <dy, y> + aux_coef * sum_e f_e P_e; the top-k choice and the
// capacity decision are held fixed (no gradient flows through a selection),
// so a dropped assignment gets no gradient at all.
//
//   combine_bwd   one wavefront per token: dret[dest[t,j]] = w[t,j] dy[t]
//                 (bf16) and dw[t,j] = <dy[t], ret[dest[t,j]]> (fp32 dot,
//                 butterfly sum in a fixed order)
//   route_bwd     one token per group of L lanes (the router's geometry):
//                 softmax again in fp32, dp = sum_j [idx = e] dw_j
//                 + aux_coef n_e / B^2, dl = p (dp - <p, dp>) / tau
//   gather_rows   X_loc[r] = x[pack_src[lo + r]] for the local experts'
//                 packed rows (bf16; fp32 x rounded to nearest even)
//   relayout_rb8  row-major rows of one expert segment -> the "RB8" layout
//                 the weight-gradient GEMM reads: element (r, c) of a
//                 segment of W columns at ((r / 8) W + c) 8 + r % 8, so
//                 that 8 consecutive rows of one column (one matrix-core
//                 K fragment) are 16 contiguous bytes; rows past the
//                 segment's end up to the next multiple of 32 are zero.
//                 Optionally the activation H = act(Z) is formed on the way
//                 (Z recomputed by the forward GEMM1 without activation).
//   split_rows    fp32 -> bf16 parts hi, mid, lo (v = hi + mid + lo exactly
//                 where the remainders stay normal), row-major with zero
//                 columns up to a multiple of 32, or in the RB8 layout
//   unpack_sum    dx_acc[t] = sum_j dXp[dest[t,j]] (+ dy[t] with the
//                 residual), fp32, fixed j order
#include "launch.h"
#include "moe_kernels.h"

namespace moek {
namespace {

unsigned bgrid(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > (1 << 20)) g = 1 << 20;
  if (g < 1) g = 1;
  return (unsigned)g;
}

__device__ __forceinline__ void load8(const void* p, bool bf16, int64_t off, float* f) {
  if (bf16) {
    unpack8(*(const u32x4*)((const uint16_t*)p + off), f);
  } else {
    const float* q = (const float*)p + off;
    const f32x4 a = *(const f32x4*)q;
    const f32x4 b = *(const f32x4*)(q + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f[u] = a[u];
      f[u + 4] = b[u];
    }
  }
}

// ---- combine backward --------------------------------------------------
// Block: 4 tokens, one wavefront each; the wavefront walks the row in
// 512-column pieces (one 16-byte chunk per lane), reading dy once and each
// kept row of ret once.  Per-lane partial dots of the k choices are summed
// across the wavefront by a fixed butterfly at the end.
template <bool XBF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const void* __restrict__ dy, const uint16_t* __restrict__ ret,
    const int32_t* __restrict__ dest, const float* __restrict__ w, int64_t B, int k, int d,
    int64_t kmax, uint16_t* __restrict__ dret, float* __restrict__ dw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= B) return;
  int r_[16];
  float w_[16], dot[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    r_[j] = -1;
    w_[j] = 0.f;
    dot[j] = 0.f;
    if (j < k) {
      const int r = dest[t * k + j];
      r_[j] = (r >= 0 && r < kmax) ? r : -1;
      w_[j] = w[t * k + j];
    }
  }
  const int cpr = d / 8;
  for (int c = lane; c < cpr; c += 64) {
    float g[8];
    load8(dy, XBF16, t * d + c * 8, g);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k && r_[j] >= 0) {
        const int64_t o = (int64_t)r_[j] * d + c * 8;
        float v[8], s[8];
        unpack8(__builtin_nontemporal_load((const u32x4*)(ret + o)), v);
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc = fmaf(g[u], v[u], acc);
          s[u] = w_[j] * g[u];
        }
        dot[j] += acc;
        *(u32x4*)(dret + o) = pack8(s);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      float v = dot[j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) dw[t * k + j] = r_[j] >= 0 ? v : 0.f;
    }
  }
}

// ---- route backward ----------------------------------------------------
// L lanes per token, V logits per lane (V <= 16), as the router.
template <int L, int V>
__global__ __launch_bounds__(256) void route_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, const int32_t* __restrict__ load, float aux_scale,
    int64_t B, int E, int k, float inv_tau, float* __restrict__ dl) {
  const int li = threadIdx.x % L;
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / L;
  if (t >= B) return;  // all L lanes of a token leave together
  const float* row = logits + t * E;
  float v[V], dp[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = li + u * L;
    v[u] = e < E ? row[e] : -INFINITY;
    dp[u] = (e < E && load) ? aux_scale * (float)load[e] : 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    const float g = dw[t * k + j];
    if (e >= 0 && e < E && e % L == li) {
#pragma unroll
      for (int u = 0; u < V; ++u)
        if (u == e / L) dp[u] += g;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < V; ++u) m = fmaxf(m, v[u]);
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, L));
  float ex[V], s = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    ex[u] = li + u * L < E ? expf((v[u] - m) * inv_tau) : 0.f;
    s += ex[u];
  }
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, L);
  const float inv_s = 1.0f / s;
  float pd = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u) pd = fmaf(ex[u] * inv_s, dp[u], pd);
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) pd += __shfl_xor(pd, off, L);
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = li + u * L;
    if (e < E) dl[t * E + e] = ex[u] * inv_s * (dp[u] - pd) * inv_tau;
  }
}

// ---- gather of the local experts' input rows ----------------------------
// One wavefront per row, one lane per 16-byte chunk; rows past the local
// count (known on the device) are skipped.
template <bool XBF16>
__global__ __launch_bounds__(256) void gather_rows_kernel(const void* __restrict__ x,
                                                          const int32_t* __restrict__ pack_src,
                                                          const int32_t* __restrict__ eo,
                                                          int e_begin, int e_end, int64_t B,
                                                          int d, int64_t rows_max,
                                                          uint16_t* __restrict__ out) {
  const int64_t lo = eo[e_begin], hi = eo[e_end];
  const int64_t n = hi - lo < rows_max ? hi - lo : rows_max;
  const int cpr = d / 8;
  for (int64_t rb = blockIdx.x; rb * 4 < n; rb += gridDim.x) {
    const int64_t r = rb * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= n) continue;
    const int64_t t = pack_src[lo + r];
    if (t < 0 || t >= B) continue;
    for (int c = threadIdx.x & 63; c < cpr; c += 64) {
      float f[8];
      if (XBF16) {
        *(u32x4*)(out + r * d + c * 8) = *(const u32x4*)((const uint16_t*)x + t * d + c * 8);
      } else {
        load8(x, false, t * d + c * 8, f);
        *(u32x4*)(out + r * d + c * 8) = pack8(f);
      }
    }
  }
}

// ---- RB8 re-layout ----------------------------------------------------------
// GELU with the exact-erf definition (erf by Abramowitz & Stegun formula
// 7.1.26, as in the expert GEMM's epilogue); silu(z) = z / (1 + e^-z).
__device__ __forceinline__ float b_gelu(float z) {
  const float az = fabsf(z);
  const float t = 1.0f / fmaf(0.23164188f, az, 1.0f);
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = exp2f(z * z * -0.72134752f);
  const float r = 0.5f * z * (p * e);
  return z >= 0.0f ? z - r : r;
}
__device__ __forceinline__ float b_silu(float z) { return z / (1.0f + exp2f(z * -1.44269504f)); }

enum { RL_COPY = 0, RL_GELU = 1, RL_SWIGLU = 2 };

// Column of unit u in the recomputed SwiGLU pre-activations (the forward
// GEMM1's interleaved tile layout: per 128 hidden units, four groups of 64
// columns, 32 of W1's products then 32 of W3's).
__device__ __forceinline__ int zcol1(int u) { return (u >> 7) * 256 + ((u >> 5) & 3) * 64 + (u & 31); }

// Block: one 8-row group x 256 columns of one segment.  Phase 1: 256
// threads load the 8 x 256 tile as 16-byte row pieces into LDS; phase 2:
// thread i reads column i's 8 values and writes them as one 16-byte chunk.
// grid.x: n_seg * groups_per_seg (groups past a segment's zero padding
// exit); grid.y: column tiles (at most 257).  Segment s holds source rows
// [seg_lo(s), seg_hi(s)) (relative to src), from expert_offset when eo is
// given, else one segment of rows_const rows.  With ridx (and eo, rel), row
// r of the segments is row ridx[expert_offset[e_begin] + r] of src (the
// local experts' rows of x through pack_src, with no gathered copy); an
// index outside [0, src_rows) reads as a zero row.
template <int MODE>
__global__ __launch_bounds__(256) void relayout_rb8_kernel(
    const uint16_t* __restrict__ src, int64_t src_ld, const int32_t* __restrict__ eo,
    int e_begin, int rel, int64_t rows_const, int gps, int W, int src_w, int one_col,
    uint16_t* __restrict__ out, int64_t out_seg, const int32_t* __restrict__ ridx,
    int64_t src_rows) {
  __shared__ uint16_t tile[8][256 + 8];
  const int seg = blockIdx.x / gps, g = blockIdx.x % gps;
  int64_t lo, n, base = 0;
  if (eo) {
    // rel: src holds the local rows only (row 0 = expert_offset[e_begin]);
    // otherwise src is indexed by the absolute packed row
    base = rel ? eo[e_begin] : 0;
    lo = eo[e_begin + seg] - base;
    n = eo[e_begin + seg + 1] - eo[e_begin + seg];
  } else {
    lo = 0;
    n = rows_const;
  }
  const int64_t npad = (n + 31) / 32 * 32;
  if ((int64_t)g * 8 >= npad) return;
  const int c0 = blockIdx.y * 256;
  // phase 1: row rr = tid / 32, columns c0 + 8 (tid % 32) .. +7
  {
    const int rr = threadIdx.x >> 5, cc = (threadIdx.x & 31) * 8;
    const int64_t r = (int64_t)g * 8 + rr;
    const int c = c0 + cc;
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = 0.f;
    int64_t sr = lo + r;
    if (ridx && r < n) {
      sr = ridx[base + lo + r];
      if (sr < 0 || sr >= src_rows) sr = -1;
    }
    if (r < n && sr >= 0) {
      const uint16_t* rowp = src + sr * src_ld;
      if (MODE == RL_COPY) {
        if (c + 8 <= src_w) {
          unpack8(*(const u32x4*)(rowp + c), v);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (c + u < src_w) v[u] = bf16_lo(rowp[c + u]);
        }
      } else if (MODE == RL_GELU) {
        if (c < W) {  // W (= f) is a multiple of 8
          unpack8(*(const u32x4*)(rowp + c), v);
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = bf16_lo(f32_to_bf16(b_gelu(v[u])));
        }
      } else {
        if (c < W) {
          float z1[8], z3[8];
          const int p1 = zcol1(c);
          unpack8(*(const u32x4*)(rowp + p1), z1);
          unpack8(*(const u32x4*)(rowp + p1 + 32), z3);
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = bf16_lo(f32_to_bf16(b_silu(z1[u]) * z3[u]));
        }
      }
    }
    // the optional constant column (ones) past the source's columns
    if (one_col >= 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c + u == one_col) v[u] = (r < n) ? 1.0f : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[rr][cc + u] = (uint16_t)f32_to_bf16(v[u]);
  }
  __syncthreads();
  const int c = c0 + threadIdx.x;
  if (c >= W) return;
  uint32_t h[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) h[u] = tile[u][threadIdx.x];
  const u32x4 q = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16)};
  *(u32x4*)(out + (int64_t)seg * out_seg + (((int64_t)g * W + c) * 8)) = q;
}

// ---- fp32 -> bf16 parts -----------------------------------------------------
// v = hi + mid + lo: hi = v truncated to bf16, mid = the remainder truncated,
// lo = what is left (exact while the remainders stay in the normal range).
__device__ __forceinline__ void split3f(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = __float_as_uint(v) >> 16;
  const float r1 = v - __uint_as_float(hi << 16);
  mid = __float_as_uint(r1) >> 16;
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16(r2);
}

// Row-major: out_p [rows][Wp] (Wp = cols rounded up to 32, zeros past cols);
// one thread per 8 output columns.
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ src,
                                                         int64_t rows, int cols, int Wp,
                                                         uint16_t* __restrict__ o0,
                                                         uint16_t* __restrict__ o1,
                                                         uint16_t* __restrict__ o2) {
  const int cpr = Wp / 8;
  const int64_t total = rows * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cpr;
    const int c = (int)(i - r * cpr) * 8;
    uint32_t a[8], b[8], e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = c + u < cols ? src[r * cols + c + u] : 0.f;
      split3f(v, a[u], b[u], e[u]);
    }
    const int64_t o = r * Wp + c;
    *(u32x4*)(o0 + o) = u32x4{a[0] | (a[1] << 16), a[2] | (a[3] << 16), a[4] | (a[5] << 16),
                              a[6] | (a[7] << 16)};
    if (o1)
      *(u32x4*)(o1 + o) = u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16),
                                b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
    if (o2)
      *(u32x4*)(o2 + o) = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
  }
}

// RB8 of an fp32 [rows][cols] matrix (one segment, W = Wp columns, rows
// padded with zeros to a multiple of 32), split into parts; one thread per
// (8-row group, column).  one_col >= 0: that column is 1 (in part hi).
__global__ __launch_bounds__(256) void split_rb8_kernel(const float* __restrict__ src,
                                                        int64_t rows, int cols, int64_t ld,
                                                        int trans, int Wp, int one_col,
                                                        uint16_t* __restrict__ o0,
                                                        uint16_t* __restrict__ o1,
                                                        uint16_t* __restrict__ o2) {
  const int64_t groups = (rows + 31) / 32 * 4;
  const int64_t total = groups * Wp;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t g = i / Wp;
    const int c = (int)(i - g * Wp);
    uint32_t a[8], b[8], e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t r = g * 8 + u;
      float v = 0.f;
      if (r < rows)
        v = c < cols ? (trans ? src[(int64_t)c * ld + r] : src[r * ld + c])
                     : (c == one_col ? 1.0f : 0.f);
      split3f(v, a[u], b[u], e[u]);
    }
    const int64_t o = i * 8;
    *(u32x4*)(o0 + o) = u32x4{a[0] | (a[1] << 16), a[2] | (a[3] << 16), a[4] | (a[5] << 16),
                              a[6] | (a[7] << 16)};
    if (o1)
      *(u32x4*)(o1 + o) = u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16),
                                b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
    if (o2)
      *(u32x4*)(o2 + o) = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
  }
}

// ---- dispatch backward (the pack's transpose) -----------------------------
// Same grid as the combine: one wavefront per token, one lane per 8 columns.
template <bool XBF16, bool RES>
__global__ __launch_bounds__(256) void unpack_sum_kernel(
    const uint16_t* __restrict__ dxp, const int32_t* __restrict__ dest,
    const void* __restrict__ dy, int64_t B, int k, int d, int64_t kmax,
    float* __restrict__ dx_acc) {
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
        float f[8];
        unpack8(__builtin_nontemporal_load((const u32x4*)(dxp + (int64_t)r * d + c * 8)), f);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += f[u];
      }
    }
    if (RES) {
      float g[8];
      load8(dy, XBF16, t * d + c * 8, g);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += g[u];
    }
    float* o = dx_acc + t * d + c * 8;
    *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

// shared expert backward: its rows are the tokens in order (pack_src[t] = t,
// expert_offset {0, B}), and its output gradient is dy (bf16) itself
__global__ __launch_bounds__(256) void shared_bwd_prep_kernel(int32_t* __restrict__ pack_src,
                                                              int32_t* __restrict__ eo,
                                                              const u32x4* __restrict__ dy,
                                                              u32x4* __restrict__ dret, int64_t B,
                                                              int64_t nchunks) {
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t st = (int64_t)gridDim.x * 256;
  if (i0 < 2) eo[i0] = i0 == 0 ? 0 : (int32_t)B;
  for (int64_t i = i0; i < B; i += st) pack_src[i] = (int32_t)i;
  for (int64_t i = i0; i < nchunks; i += st) dret[i] = dy[i];
}

// acc[i] += v[i] (bf16), 8 elements per thread (n a multiple of 8)
__global__ __launch_bounds__(256) void add_bf16_kernel(float* __restrict__ acc,
                                                       const uint16_t* __restrict__ v,
                                                       int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * 256) {
    float f[8];
    unpack8(*(const u32x4*)(v + i * 8), f);
    float4* a = reinterpret_cast<float4*>(acc + i * 8);
    float4 a0 = a[0], a1 = a[1];
    a0.x += f[0]; a0.y += f[1]; a0.z += f[2]; a0.w += f[3];
    a1.x += f[4]; a1.y += f[5]; a1.z += f[6]; a1.w += f[7];
    a[0] = a0;
    a[1] = a1;
  }
}

__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int G,
                                                        int M0, int N, float* __restrict__ out0,
                                                        float* __restrict__ out1) {
  const int64_t per = (int64_t)(M0 + 1) * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per;
       i += (int64_t)gridDim.x * 256) {
    float v = 0.f;
    for (int g = 0; g < G; ++g) v += part[(int64_t)g * per + i];
    const int64_t m = i / N;
    if (m < M0) out0[i] = v;
    else if (out1) out1[i - (int64_t)M0 * N] = v;
  }
}

}  // namespace

hipError_t launch_sum_parts(const float* part, int G, int M0, int N, float* out0, float* out1,
                            hipStream_t s) {
  const int64_t per = (int64_t)(M0 + 1) * N;
  hipLaunchKernelGGL(sum_parts_kernel, dim3(bgrid(per, 256)), dim3(256), 0, s, part, G, M0, N,
                     out0, out1);
  return hipGetLastError();
}

// zeros by a kernel (not a memset node: callers may capture the stream)
hipError_t launch_shared_bwd_prep(int32_t* pack_src, int32_t* eo, const uint16_t* dy,
                                  uint16_t* dret, int64_t B, int d, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int64_t nchunks = B * d / 8;
  hipLaunchKernelGGL(shared_bwd_prep_kernel, dim3(bgrid(nchunks > B ? nchunks : B, 256)),
                     dim3(256), 0, s, pack_src, eo, reinterpret_cast<const u32x4*>(dy),
                     reinterpret_cast<u32x4*>(dret), B, nchunks);
  return hipGetLastError();
}

hipError_t launch_add_bf16(float* acc, const uint16_t* v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(add_bf16_kernel, dim3(bgrid(n / 8, 256)), dim3(256), 0, s, acc, v, n / 8);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0 || !p) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(bgrid(n, 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, bool x_bf16, const uint16_t* ret,
                              const int32_t* dest, const float* w, int64_t B, int k, int d,
                              int64_t kmax, uint16_t* dret, float* dw, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const unsigned g = (unsigned)((B + 3) / 4);
  if (x_bf16)
    hipLaunchKernelGGL(combine_bwd_kernel<true>, dim3(g), dim3(256), 0, s, dy, ret, dest, w, B,
                       k, d, kmax, dret, dw);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<false>, dim3(g), dim3(256), 0, s, dy, ret, dest, w, B,
                       k, d, kmax, dret, dw);
  return hipGetLastError();
}

template <int L, int V>
static void launch_route_bwd_t(const float* logits, const int32_t* idx, const float* dw,
                               const int32_t* load, float aux_scale, int64_t B, int E, int k,
                               float inv_tau, float* dl, hipStream_t s) {
  const int64_t threads = B * L;
  hipLaunchKernelGGL((route_bwd_kernel<L, V>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, logits, idx, dw, load, aux_scale, B, E, k, inv_tau, dl);
}

hipError_t launch_route_bwd(const float* logits, const int32_t* idx, const float* dw,
                            const int32_t* load, float aux_coef, int64_t B, int E, int k,
                            float tau, float* dl, hipStream_t s) {
  if (B == 0) return hipSuccess;
  // the auxiliary term aux_coef * f_e / B with f_e = n_e / B
  const float aux_scale = (float)((double)aux_coef / ((double)B * (double)B));
  const int32_t* ld = aux_coef != 0.0f ? load : nullptr;
  const float it = 1.0f / tau;
  if (E <= 8) launch_route_bwd_t<8, 1>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else if (E <= 16) launch_route_bwd_t<16, 1>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else if (E <= 32) launch_route_bwd_t<32, 1>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else if (E <= 64) launch_route_bwd_t<64, 1>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else if (E <= 128) launch_route_bwd_t<64, 2>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else if (E <= 256) launch_route_bwd_t<64, 4>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else if (E <= 512) launch_route_bwd_t<64, 8>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  else launch_route_bwd_t<64, 16>(logits, idx, dw, ld, aux_scale, B, E, k, it, dl, s);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, bool x_bf16, const int32_t* pack_src,
                              const int32_t* eo, int e_begin, int e_end, int64_t B, int d,
                              int64_t rows_max, uint16_t* out, hipStream_t s) {
  if (rows_max <= 0 || e_end <= e_begin) return hipSuccess;
  const unsigned g = bgrid(rows_max, 4);
  if (x_bf16)
    hipLaunchKernelGGL(gather_rows_kernel<true>, dim3(g), dim3(256), 0, s, x, pack_src, eo,
                       e_begin, e_end, B, d, rows_max, out);
  else
    hipLaunchKernelGGL(gather_rows_kernel<false>, dim3(g), dim3(256), 0, s, x, pack_src, eo,
                       e_begin, e_end, B, d, rows_max, out);
  return hipGetLastError();
}

int64_t rb8_rows(int64_t rows) { return (rows + 31) / 32 * 32; }

hipError_t launch_relayout_rb8(int mode, const uint16_t* src, int64_t src_ld, const int32_t* eo,
                               int e_begin, int rel, int n_seg, int64_t rows_cap, int W,
                               int src_w, int one_col, uint16_t* out, hipStream_t s,
                               const int32_t* ridx, int64_t src_rows) {
  if (n_seg <= 0 || rows_cap <= 0) return hipSuccess;
  const int64_t R8 = rb8_rows(rows_cap);
  const int gps = (int)(R8 / 8);
  const int64_t gx = (int64_t)n_seg * gps;
  if (gx > 2147483647 || (W + 255) / 256 > 65535) return hipErrorInvalidValue;
  const dim3 g((unsigned)gx, (unsigned)((W + 255) / 256));
  const int64_t out_seg = R8 * W;
  switch (mode) {
    case RL_GELU:
      hipLaunchKernelGGL(relayout_rb8_kernel<RL_GELU>, g, dim3(256), 0, s, src, src_ld, eo,
                         e_begin, rel, rows_cap, gps, W, src_w, one_col, out, out_seg,
                         ridx, src_rows);
      break;
    case RL_SWIGLU:
      hipLaunchKernelGGL(relayout_rb8_kernel<RL_SWIGLU>, g, dim3(256), 0, s, src, src_ld, eo,
                         e_begin, rel, rows_cap, gps, W, src_w, one_col, out, out_seg,
                         ridx, src_rows);
      break;
    default:
      hipLaunchKernelGGL(relayout_rb8_kernel<RL_COPY>, g, dim3(256), 0, s, src, src_ld, eo,
                         e_begin, rel, rows_cap, gps, W, src_w, one_col, out, out_seg,
                         ridx, src_rows);
  }
  return hipGetLastError();
}

hipError_t launch_split_rows(const float* src, int64_t rows, int cols, int Wp, uint16_t* o0,
                             uint16_t* o1, uint16_t* o2, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_rows_kernel, dim3(bgrid(rows * (Wp / 8), 256)), dim3(256), 0, s, src,
                     rows, cols, Wp, o0, o1, o2);
  return hipGetLastError();
}

hipError_t launch_split_rb8(const float* src, int64_t rows, int cols, int64_t ld, bool trans,
                            int Wp, int one_col, uint16_t* o0, uint16_t* o1, uint16_t* o2,
                            hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t total = (rows + 31) / 32 * 4 * Wp;
  hipLaunchKernelGGL(split_rb8_kernel, dim3(bgrid(total, 256)), dim3(256), 0, s, src, rows, cols,
                     ld, trans ? 1 : 0, Wp, one_col, o0, o1, o2);
  return hipGetLastError();
}

hipError_t launch_unpack_sum(const uint16_t* dxp, const int32_t* dest, const void* dy,
                             bool x_bf16, bool residual, int64_t B, int k, int d, int64_t kmax,
                             float* dx_acc, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int64_t ntb = (B + 3) / 4;
  const dim3 g((unsigned)((d / 8 + 63) / 64), (unsigned)(ntb < 65535 ? ntb : 65535));
  if (residual) {
    if (x_bf16)
      hipLaunchKernelGGL((unpack_sum_kernel<true, true>), g, dim3(256), 0, s, dxp, dest, dy, B,
                         k, d, kmax, dx_acc);
    else
      hipLaunchKernelGGL((unpack_sum_kernel<false, true>), g, dim3(256), 0, s, dxp, dest, dy, B,
                         k, d, kmax, dx_acc);
  } else {
    hipLaunchKernelGGL((unpack_sum_kernel<true, false>), g, dim3(256), 0, s, dxp, dest, dy, B, k,
                       d, kmax, dx_acc);
  }
  return hipGetLastError();
}

}  // namespace moek
