// Routing-health signals of one batch: per-expert mean router probability,
// token fraction, utilisation and drops, the Switch auxiliary loss, routing
// entropy and load entropy.
//
// "Expert Parallelism" (inferensys.com glossary), "Practitioner Guidance":
// expert utilisation and routing entropy are first-class health signals.
// "Expert Parallelism" (narrativegoldmine.com), "Components and
// Architecture", auxiliary load-balancing loss (the Switch form): computed
// here as sum_e f_e P_e, f_e the share of tokens that chose expert e and P_e
// its mean router probability.
// "Expert Parallelism" (theinfinity.ai), figure text: each expert's bar is
// the share of its capacity in use.
//
// Three launches, all deterministic (every sum in a fixed order):
//   stats_partial  L lanes per token (the router's lane geometry), V logits
//                  per lane; per token the softmax and its entropy
//                  ln S - (sum_e e^z z) / S with z = (g - max g) / tau; each
//                  block sums p over its token range per expert and the
//                  entropies in fp32, into column e (and E) of a
//                  column-major [E + 1][blocks] table
//   stats_column   one wavefront per column: the block partials loaded
//                  coalesced and added in double by a fixed butterfly
//   stats_final    one block: P_e, f_e, kept / C, drops and the scalar
//                  signals (fixed-tree sums in double)
// The logits are read once (B E 4 bytes); everything else is O(E) per block.
#include "moe_kernels.h"

namespace moek {
namespace {

constexpr int kStatThreads = 256;
constexpr int kFinalThreads = 1024;
constexpr int kMaxStatBlocks = 512;

template <int L, int V>
__global__ __launch_bounds__(kStatThreads) void stats_partial_kernel(
    const float* __restrict__ logits, int64_t B, int E, float inv_tau, int64_t tpb,
    float* __restrict__ part) {
  constexpr int G = kStatThreads / L;  // tokens per pass
  __shared__ float red[kStatThreads * V];
  __shared__ float hred[G];
  const int tid = threadIdx.x, li = tid % L, g = tid / L;
  float acc[V];
#pragma unroll
  for (int u = 0; u < V; ++u) acc[u] = 0.f;
  float hacc = 0.f;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t1 = t0 + tpb < B ? t0 + tpb : B;
  // the L lanes of a token run the same trip count, so the segment-wide
  // shuffles below always see all of their lanes
  for (int64_t t = t0 + g; t < t1; t += G) {
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
    float ex[V], s = 0.f, a = 0.f;
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const bool ok = li + u * L < E;
      const float z = ok ? (v[u] - m) * inv_tau : 0.f;
      ex[u] = ok ? expf(z) : 0.f;
      s += ex[u];
      a += ex[u] * z;
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) {
      s += __shfl_xor(s, off, L);
      a += __shfl_xor(a, off, L);
    }
    const float inv_s = 1.0f / s;
#pragma unroll
    for (int u = 0; u < V; ++u) acc[u] += ex[u] * inv_s;
    if (li == 0) hacc += logf(s) - a * inv_s;
  }
  // red[g][e] with e = li + u L
#pragma unroll
  for (int u = 0; u < V; ++u) red[g * (L * V) + u * L + li] = acc[u];
  if (li == 0) hred[g] = hacc;
  __syncthreads();
  const int nblk = gridDim.x;
  for (int e = tid; e < E; e += kStatThreads) {
    float sum = 0.f;
    for (int gg = 0; gg < G; ++gg) sum += red[gg * (L * V) + e];
    part[(int64_t)e * nblk + blockIdx.x] = sum;
  }
  if (tid == 0) {
    float sum = 0.f;
    for (int gg = 0; gg < G; ++gg) sum += hred[gg];
    part[(int64_t)E * nblk + blockIdx.x] = sum;
  }
}

// Column c of the partial table (c < E: expert c; c == E: entropies), one
// wavefront each: lane l adds blocks l, l + 64, ... in double, then a
// butterfly over the 64 lanes (the same pairing every time).
__global__ __launch_bounds__(256) void stats_column_kernel(const float* __restrict__ part,
                                                           int nblk, int ncol,
                                                           double* __restrict__ colsum) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= ncol) return;
  const float* col = part + (int64_t)c * nblk;
  double s = 0.0;
  for (int b = lane; b < nblk; b += 64) s += (double)col[b];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) colsum[c] = s;
}

// fixed-order sum over the block (deterministic): a butterfly inside each
// wavefront, then the 16 wavefront totals in wavefront order
template <typename T>
__device__ T block_sum(T v, T* sh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((tid & 63) == 0) sh[tid >> 6] = v;
  __syncthreads();
  T r = 0;
#pragma unroll
  for (int w = 0; w < kFinalThreads / 64; ++w) r += sh[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kFinalThreads) void stats_final_kernel(
    const double* __restrict__ colsum, int64_t B, int E, int k, int C,
    const int32_t* __restrict__ load, const int32_t* __restrict__ count,
    float* __restrict__ prob_mean, float* __restrict__ token_frac,
    float* __restrict__ utilization, int32_t* __restrict__ dropped, double* __restrict__ summary) {
  __shared__ double shd[kFinalThreads / 64];
  __shared__ long long shl[kFinalThreads / 64];
  const int tid = threadIdx.x;
  const double Bd = (double)B;
  double aux = 0.0, lent = 0.0;
  long long drop_t = 0, kept_t = 0;
  for (int e = tid; e < E; e += kFinalThreads) {
    const double P = B > 0 ? colsum[e] / Bd : 0.0;
    const int n = load[e], kept = count[e];
    const double f = B > 0 ? (double)n / Bd : 0.0;
    if (prob_mean) prob_mean[e] = (float)P;
    if (token_frac) token_frac[e] = (float)f;
    if (utilization) utilization[e] = C > 0 ? (float)((double)kept / (double)C) : 0.f;
    if (dropped) dropped[e] = n - kept;
    aux += f * P;
    const double a = B > 0 ? (double)n / (Bd * (double)k) : 0.0;
    if (a > 0.0) lent -= a * log(a);
    drop_t += n - kept;
    kept_t += kept;
  }
  aux = block_sum(aux, shd);
  lent = block_sum(lent, shd);
  drop_t = block_sum(drop_t, shl);
  kept_t = block_sum(kept_t, shl);
  if (tid == 0 && summary) {
    summary[0] = aux;
    summary[1] = B > 0 ? colsum[E] / Bd : 0.0;
    summary[2] = lent;
    summary[3] = (double)drop_t;
    summary[4] = (double)kept_t;
  }
}

// lanes per token (the router's choice): a power of two >= E up to 16
// experts, 16 up to 512, 64 beyond
int stats_lanes(int E) {
  if (E <= 16) {
    int L = 1;
    while (L < E) L <<= 1;
    return L;
  }
  return E <= 512 ? 16 : 64;
}

int stats_blocks(int64_t B, int E) {
  if (B <= 0) return 0;
  const int64_t per_pass = kStatThreads / stats_lanes(E);
  const int64_t want = (B + per_pass - 1) / per_pass;
  return (int)(want < kMaxStatBlocks ? want : kMaxStatBlocks);
}

template <int L, int V>
void launch_partial(const float* logits, int64_t B, int E, float inv_tau, int nblk,
                    int64_t tpb, float* part, hipStream_t s) {
  hipLaunchKernelGGL((stats_partial_kernel<L, V>), dim3(nblk), dim3(kStatThreads), 0, s, logits,
                     B, E, inv_tau, tpb, part);
}

}  // namespace

// partial table [E + 1][blocks] fp32, then the column sums [E + 1] double
static size_t stats_table_bytes(int64_t B, int E) {
  const size_t t = (size_t)stats_blocks(B, E) * (size_t)(E + 1) * sizeof(float);
  return (t + 7) & ~(size_t)7;
}

size_t stats_ws_bytes(int64_t B, int E) {
  return B > 0 ? stats_table_bytes(B, E) + (size_t)(E + 1) * sizeof(double) : 0;
}

hipError_t launch_routing_stats(const float* logits, int64_t B, int E, int k, int C, float tau,
                                const int32_t* load, const int32_t* count, float* prob_mean,
                                float* token_frac, float* utilization, int32_t* dropped,
                                double* summary, void* ws, hipStream_t s) {
  const int nblk = stats_blocks(B, E);
  float* part = static_cast<float*>(ws);
  double* colsum = nullptr;
  if (nblk > 0) {
    colsum = reinterpret_cast<double*>(static_cast<char*>(ws) + stats_table_bytes(B, E));
    const int64_t tpb = (B + nblk - 1) / nblk;
    const float it = 1.0f / tau;
    if (E <= 1) launch_partial<1, 1>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 2) launch_partial<2, 1>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 4) launch_partial<4, 1>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 8) launch_partial<8, 1>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 16) launch_partial<16, 1>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 32) launch_partial<16, 2>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 64) launch_partial<16, 4>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 128) launch_partial<16, 8>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 256) launch_partial<16, 16>(logits, B, E, it, nblk, tpb, part, s);
    else if (E <= 512) launch_partial<16, 32>(logits, B, E, it, nblk, tpb, part, s);
    else launch_partial<64, 16>(logits, B, E, it, nblk, tpb, part, s);
    hipLaunchKernelGGL(stats_column_kernel, dim3((E + 1 + 3) / 4), dim3(256), 0, s, part, nblk,
                       E + 1, colsum);
  }
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kFinalThreads), 0, s, colsum, B, E, k, C,
                     load, count, prob_mean, token_frac, utilization, dropped, summary);
  return hipGetLastError();
}

}  // namespace moek
