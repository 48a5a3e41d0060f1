// Expert-choice routing: every expert picks its top-C tokens of the batch.
//
// "Expert Parallelism" (narrativegoldmine.com), "Major Variants and
// Families", expert choice routing.  The rule implemented: the selection
// runs per expert over the batch, not per token over the experts; expert e
// keeps the C_e tokens with the highest scores in its column, so every
// expert gets the same row count and a token can end up with several
// experts or with none.
//
// Scores are the router probabilities p_te = softmax(g_t / tau)_e in fp32;
// among equal scores the lower token wins; an expert's rows are packed in
// token order, experts one after the other (C_e = min(C, B) rows each); the
// weight of a chosen pair is p_te.  Kernels:
//   probs_kernel      softmax per token (the router's lane geometry), written
//                     transposed, probs_t[e][t], so that one expert's scores
//                     are contiguous
//   ec_select_kernel  one workgroup per expert: a 4-pass radix select over
//                     the fp32 bit patterns (non-negative floats order like
//                     their bits) finds the C_e-th largest score T; then one
//                     ordered pass over the tokens takes every score > T and
//                     the first (C_e - #greater) scores == T, numbering the
//                     chosen tokens in token order (ballot prefix counts)
//   ec_pack_kernel    gather: one wavefront per packed row
//   ec_combine_kernel one wavefront per token and 512 columns: the token's
//                     rows for up to 64 experts at a time are gathered by
//                     lane, then the chosen experts are walked in expert
//                     order (ballot, lowest set lane first), fp32 sums
#include "moe_kernels.h"

namespace moek {
namespace {

constexpr int kProbThreads = 256;
constexpr int kSelThreads = 1024;

template <int L, int V>
__global__ __launch_bounds__(kProbThreads) void probs_kernel(const float* __restrict__ logits,
                                                             int64_t B, int E, float inv_tau,
                                                             float* __restrict__ probs_t) {
  const int tid = threadIdx.x, li = tid % L;
  const int64_t t = ((int64_t)blockIdx.x * kProbThreads + tid) / L;
  // all L lanes of a token share t, so a token's lanes are all in or all out
  if (t >= B) return;
  const float* row = logits + t * E;
  float v[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = li + u * L;
    v[u] = e < E ? row[e] : -INFINITY;
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
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = li + u * L;
    if (e < E) probs_t[(int64_t)e * B + t] = ex[u] * inv_s;
  }
}

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// hist[digit] += 1 for every valid lane, one LDS atomic per distinct digit
// in the wavefront: 8 ballots find the lanes sharing a lane's digit (the
// scores of one expert cluster around 1/E, so most lanes share the top
// digits and per-lane atomics on one address would serialize)
__device__ __forceinline__ void hist_add(int* hist, unsigned digit, bool valid) {
  const int lane = threadIdx.x & 63;
  unsigned long long m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (digit >> b) & 1u;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  if (valid && (m & lanes_below(lane)) == 0) atomicAdd(&hist[digit], __popcll(m));
}

// Block-wide exclusive prefix of a 0/1 flag over the block's threads in
// thread order; returns this thread's prefix and writes the block total to
// *tot.
__device__ __forceinline__ int block_flag_prefix(bool f, int* wcnt, int* tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long b = __ballot(f);
  const int in_wave = __popcll(b & lanes_below(lane));
  if (lane == 0) wcnt[wave] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int c = wcnt[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();
  *tot = all;
  return before + in_wave;
}

// COL_LDS: the expert's column of scores is first copied into LDS (one pass
// with every load in flight), and the five passes below read it there
// instead of paying the memory latency once per chunk and pass.
template <bool COL_LDS>
__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(
    const float* __restrict__ probs_t, int64_t B, int Ce, int32_t* __restrict__ sel_t,
    int32_t* __restrict__ pack_src, float* __restrict__ pack_w) {
  __shared__ int hist[256];
  __shared__ int wcnt[kSelThreads / 64];
  __shared__ int bsum[4];
  __shared__ unsigned s_prefix;
  __shared__ int s_need;
  extern __shared__ unsigned colbuf[];
  const int e = blockIdx.x, tid = threadIdx.x;
  const unsigned* gkey = reinterpret_cast<const unsigned*>(probs_t + (int64_t)e * B);
  if (COL_LDS) {
    for (int64_t t = tid; t < B; t += kSelThreads) colbuf[t] = gkey[t];
    __syncthreads();
  }
  const unsigned* key = COL_LDS ? colbuf : gkey;
  // threshold T: the Ce-th largest key; need = how many keys == T to take
  unsigned prefix = 0u, mask = 0u;
  int need = Ce;
  if (Ce > 0 && Ce < B) {
    for (int dgt = 3; dgt >= 0; --dgt) {
      const int sh = 8 * dgt;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      // every lane of a wavefront runs the same trip count (the ballots)
      for (int64_t t0 = 0; t0 < B; t0 += kSelThreads) {
        const int64_t t = t0 + tid;
        const unsigned kk = t < B ? key[t] : 0u;
        hist_add(hist, (kk >> sh) & 255u, t < B && (kk & mask) == prefix);
      }
      __syncthreads();
      // the bin holding the need-th largest key: thread i < 256 takes bin
      // 255 - i, so an inclusive prefix over i counts the keys in bins >= b;
      // exactly one bin has fewer than need above it and need or more up to
      // and including it
      int h = 0, incl = 0;
      const int lane = tid & 63, wave = tid >> 6;
      if (tid < 256) {
        h = hist[255 - tid];
        incl = h;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(incl, off);
          if (lane >= off) incl += v;
        }
        if (lane == 63) bsum[wave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < wave; ++w) incl += bsum[w];
        const int above = incl - h;
        if (above < need && incl >= need) {
          s_prefix = prefix | ((unsigned)(255 - tid) << sh);
          s_need = need - above;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      need = s_need;
      mask |= 255u << sh;
      __syncthreads();
    }
  }
  const unsigned T = prefix;
  const bool all = Ce >= B;
  // ordered pass: take key > T, and the first `need` keys == T
  int eq_before = 0, sel_before = 0;
  for (int64_t t0 = 0; t0 < B; t0 += kSelThreads) {
    const int64_t t = t0 + tid;
    const bool live = t < B;
    const unsigned kk = live ? key[t] : 0u;
    const bool eq = live && !all && Ce > 0 && kk == T;
    int eq_tot;
    const int eq_rank = eq_before + block_flag_prefix(eq, wcnt, &eq_tot);
    const bool take = live && Ce > 0 && (all || kk > T || (eq && eq_rank < need));
    int sel_tot;
    const int row_in = sel_before + block_flag_prefix(take, wcnt, &sel_tot);
    if (live) {
      const int row = e * Ce + row_in;
      sel_t[(int64_t)e * B + t] = take ? row : -1;
      if (take) {
        pack_src[row] = (int32_t)t;
        pack_w[row] = __uint_as_float(kk);
      }
    }
    eq_before += eq_tot;
    sel_before += sel_tot;
  }
}

// packed[r] = bf16(x[pack_src[r]]): one wavefront per row, one lane per
// 16-byte chunk, 4 rows per block, the column piece in the grid's x
template <bool XBF16>
__global__ __launch_bounds__(256) void ec_pack_kernel(const void* __restrict__ x,
                                                      const int32_t* __restrict__ pack_src,
                                                      int64_t rows, int d,
                                                      uint16_t* __restrict__ packed) {
  const int cpr = d / 8;
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t nrb = (rows + 3) / 4;
  for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    const int64_t r = rb * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= rows || c >= cpr) continue;
    const int64_t t = pack_src[r];
    u32x4 v;
    if (XBF16) {
      v = *(const u32x4*)((const uint16_t*)x + t * d + c * 8);
    } else {
      const float* xf = (const float*)x + t * d + c * 8;
      const f32x4 a = *(const f32x4*)xf;
      const f32x4 b = *(const f32x4*)(xf + 4);
      const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      v = pack8(f);
    }
    __builtin_nontemporal_store(v, (u32x4*)(packed + r * d + c * 8));
  }
}

template <bool XBF16, bool RES>
__global__ __launch_bounds__(256) void ec_combine_kernel(
    const uint16_t* __restrict__ ret, const int32_t* __restrict__ sel_t,
    const float* __restrict__ pack_w, const void* __restrict__ xres, void* __restrict__ y,
    int64_t B, int E, int d) {
  const int cpr = d / 8;
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 64 + lane;
  const int64_t ntb = (B + 3) / 4;
  for (int64_t tb = blockIdx.y; tb < ntb; tb += gridDim.y) {
    const int64_t t = tb * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= B) continue;
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int r_lane = e < E ? sel_t[(int64_t)e * B + t] : -1;
      unsigned long long m = __ballot(r_lane >= 0);
      while (m) {
        const int l = __ffsll((long long)m) - 1;  // lowest lane = lowest expert
        m &= m - 1;
        const int r = __builtin_amdgcn_readlane(r_lane, l);
        const float wr = pack_w[r];
        if (c < cpr) {
          float f[8];
          unpack8(__builtin_nontemporal_load((const u32x4*)(ret + (int64_t)r * d + c * 8)), f);
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[u] = fmaf(wr, f[u], acc[u]);
        }
      }
    }
    if (c >= cpr) continue;
    if (RES) {
      float xr[8];
      if (XBF16) {
        unpack8(*(const u32x4*)((const uint16_t*)xres + t * d + c * 8), xr);
      } else {
        const float* xf = (const float*)xres + t * d + c * 8;
        const f32x4 a = *(const f32x4*)xf;
        const f32x4 b = *(const f32x4*)(xf + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) { xr[u] = a[u]; xr[u + 4] = b[u]; }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += xr[u];
    }
    if (XBF16) {
      // non-temporal, as in the token-choice combine: nothing reads y again
      __builtin_nontemporal_store(pack8(acc), (u32x4*)((uint16_t*)y + t * d + c * 8));
    } else {
      float* yf = (float*)y + t * d + c * 8;
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)yf);
      __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, (f32x4*)(yf + 4));
    }
  }
}

template <int L, int V>
void launch_probs_t(const float* logits, int64_t B, int E, float inv_tau, float* probs_t,
                    hipStream_t s) {
  const int64_t threads = B * L;
  hipLaunchKernelGGL((probs_kernel<L, V>), dim3((unsigned)((threads + kProbThreads - 1) /
                                                           kProbThreads)),
                     dim3(kProbThreads), 0, s, logits, B, E, inv_tau, probs_t);
}

// expert_offset[i] = i * Ce: one lane per entry
__global__ void ec_offsets_kernel(int32_t* __restrict__ eo, int E, int Ce) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i <= E) eo[i] = i * Ce;
}

dim3 row_grid(int64_t rows, int d) {
  const int64_t nrb = (rows + 3) / 4;
  return dim3((unsigned)((d / 8 + 63) / 64), (unsigned)(nrb < 65535 ? nrb : 65535));
}

}  // namespace

hipError_t launch_router_probs(const float* logits, int64_t B, int E, float tau, float* probs_t,
                               hipStream_t s) {
  if (B == 0) return hipSuccess;
  const float it = 1.0f / tau;
  if (E <= 1) launch_probs_t<1, 1>(logits, B, E, it, probs_t, s);
  else if (E <= 2) launch_probs_t<2, 1>(logits, B, E, it, probs_t, s);
  else if (E <= 4) launch_probs_t<4, 1>(logits, B, E, it, probs_t, s);
  else if (E <= 8) launch_probs_t<8, 1>(logits, B, E, it, probs_t, s);
  else if (E <= 16) launch_probs_t<16, 1>(logits, B, E, it, probs_t, s);
  else if (E <= 32) launch_probs_t<16, 2>(logits, B, E, it, probs_t, s);
  else if (E <= 64) launch_probs_t<16, 4>(logits, B, E, it, probs_t, s);
  else if (E <= 128) launch_probs_t<16, 8>(logits, B, E, it, probs_t, s);
  else if (E <= 256) launch_probs_t<16, 16>(logits, B, E, it, probs_t, s);
  else if (E <= 512) launch_probs_t<16, 32>(logits, B, E, it, probs_t, s);
  else launch_probs_t<64, 16>(logits, B, E, it, probs_t, s);
  return hipGetLastError();
}

hipError_t launch_expert_choice(const float* probs_t, int64_t B, int E, int Ce, int32_t* sel_t,
                                int32_t* expert_offset, int32_t* pack_src, float* pack_w,
                                hipStream_t s) {
  if (expert_offset)
    hipLaunchKernelGGL(ec_offsets_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, s,
                       expert_offset, E, Ce);
  if (B == 0 || E == 0) return hipGetLastError();
  // the column in LDS up to 36864 tokens (144 KB beside the small arrays)
  if (B <= 36864)
    hipLaunchKernelGGL((ec_select_kernel<true>), dim3(E), dim3(kSelThreads), (size_t)B * 4, s,
                       probs_t, B, Ce, sel_t, pack_src, pack_w);
  else
    hipLaunchKernelGGL((ec_select_kernel<false>), dim3(E), dim3(kSelThreads), 0, s, probs_t, B,
                       Ce, sel_t, pack_src, pack_w);
  return hipGetLastError();
}

hipError_t launch_ec_pack(const void* x, bool x_bf16, const int32_t* pack_src, int64_t rows,
                          int d, uint16_t* packed, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 g = row_grid(rows, d);
  if (x_bf16)
    hipLaunchKernelGGL((ec_pack_kernel<true>), g, dim3(256), 0, s, x, pack_src, rows, d, packed);
  else
    hipLaunchKernelGGL((ec_pack_kernel<false>), g, dim3(256), 0, s, x, pack_src, rows, d, packed);
  return hipGetLastError();
}

hipError_t launch_ec_combine(const uint16_t* ret, const int32_t* sel_t, const float* pack_w,
                             const void* x_res, bool x_bf16, void* y, int64_t B, int E, int d,
                             hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 g = row_grid(B, d);
  if (x_bf16) {
    if (x_res)
      hipLaunchKernelGGL((ec_combine_kernel<true, true>), g, dim3(256), 0, s, ret, sel_t, pack_w,
                         x_res, y, B, E, d);
    else
      hipLaunchKernelGGL((ec_combine_kernel<true, false>), g, dim3(256), 0, s, ret, sel_t, pack_w,
                         x_res, y, B, E, d);
  } else {
    if (x_res)
      hipLaunchKernelGGL((ec_combine_kernel<false, true>), g, dim3(256), 0, s, ret, sel_t, pack_w,
                         x_res, y, B, E, d);
    else
      hipLaunchKernelGGL((ec_combine_kernel<false, false>), g, dim3(256), 0, s, ret, sel_t,
                         pack_w, x_res, y, B, E, d);
  }
  return hipGetLastError();
}

}  // namespace moek
