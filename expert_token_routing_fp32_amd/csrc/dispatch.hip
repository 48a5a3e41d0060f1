// Capacity-limited slot assignment and the pack that replaces the dispatch
// all-to-all on one GPU.
//
// "Expert Parallelism" (theinfinity.ai), capacity paragraph: every expert
// takes at most C = ceil((B*k/E)*c) assignments and the overflow,
// max(0, n_e - C), is dropped.  "Expert Parallelism and the All-to-All
// Bottleneck", "The Mechanism of Expert Parallelism": the (tokens, hidden)
// activations are repacked so that each row is a token bound for one expert,
// and rows for one destination rank are contiguous ("The All-to-All
// Communication Pattern": experts are placed contiguously, E/D per rank).
//
// Claim order is q = j*B + t.  The q range is cut into tiles; three kernels
// give every assignment its slot without any order-dependent atomic:
//   slot_hist  per-tile expert histogram (LDS atomics only count)
//   slot_scan  per expert, exclusive prefix over tiles -> tile bases; n_e,
//              min(n_e, C), expert_offset (prefix over experts), rank_offset
//   slot_rank  inside a tile: 64-lane ballot match gives each lane its rank
//              among equal experts in its wavefront; per-wavefront counts and
//              bases in LDS carry the order across the four wavefronts and
//              across chunks.  Writes pos, keep, dest, pack_src.
// pack then moves each token row once from x into its kept packed rows.
#include "launch.h"
#include "moe_kernels.h"

namespace moek {
namespace {

constexpr int kSlotThreads = 256;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ unsigned long long lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// lanes of this wavefront holding the same (valid) expert id
__device__ __forceinline__ unsigned long long match_expert(int e, int nbits) {
  unsigned long long m = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__device__ __forceinline__ int load_expert(const int32_t* idx, int64_t q, int64_t B, int k,
                                           int E) {
  const int64_t j = q / B;
  const int64_t t = q - j * B;
  const int e = idx[t * k + j];
  return ((unsigned)e < (unsigned)E) ? e : -1;
}

// Per-tile expert counts: hist[tile][e], or (trans) hist[e][tile] -- each
// expert's counts over the tiles contiguous, for the multi-block scan.
__global__ __launch_bounds__(kSlotThreads) void slot_hist_kernel(const int32_t* __restrict__ idx,
                                                                int64_t B, int k, int E,
                                                                int64_t BK, int tile, int trans,
                                                                int32_t* __restrict__ hist) {
  extern __shared__ int h[];
  for (int e = threadIdx.x; e < E; e += kSlotThreads) h[e] = 0;
  __syncthreads();
  const int64_t q0 = (int64_t)blockIdx.x * tile;
  const int64_t q1 = q0 + tile < BK ? q0 + tile : BK;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += kSlotThreads) {
    const int e = load_expert(idx, q, B, k, E);
    if (e >= 0) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kSlotThreads)
    hist[trans ? (int64_t)e * gridDim.x + blockIdx.x : (int64_t)blockIdx.x * E + e] = h[e];
}

// Multi-block scan of a transposed count table: block e turns row e (expert
// e's counts over the n_tiles tiles) into its exclusive prefix in place and
// writes n_e and min(n_e, C_e).  The expert offsets (a prefix over the
// experts' kept counts) are formed by every rank block from those counts.
__global__ __launch_bounds__(kSlotThreads) void slot_scan_rows_kernel(
    int32_t* __restrict__ histT, int n_tiles, int C, const uint8_t* __restrict__ unavail,
    const int32_t* __restrict__ cap_in, int32_t* __restrict__ expert_load,
    int32_t* __restrict__ expert_count) {
  __shared__ int wsum[kSlotThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  int32_t* row = histT + (int64_t)e * n_tiles;
  int carry = 0;
  for (int t0 = 0; t0 < n_tiles; t0 += kSlotThreads) {
    const int t = t0 + tid;
    const int v = t < n_tiles ? row[t] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int pre = carry + incl - v, all = carry;
#pragma unroll
    for (int w = 0; w < kSlotThreads / 64; ++w) {
      if (w < wave) pre += wsum[w];
      all += wsum[w];
    }
    if (t < n_tiles) row[t] = pre;
    carry = all;
    __syncthreads();
  }
  if (tid == 0) {
    const int ce = cap_in ? cap_in[e] : (unavail && unavail[e]) ? 0 : C;
    if (expert_load) expert_load[e] = carry;
    expert_count[e] = carry < ce ? carry : ce;
  }
}

// One block.  Thread (g, e) of G = 1024/Epad groups walks a contiguous range
// of tiles for expert e.
__global__ __launch_bounds__(kScanThreads) void slot_scan_kernel(
    int32_t* __restrict__ hist, int n_tiles, int E, int Epad, int C,
    const uint8_t* __restrict__ unavail, const int32_t* __restrict__ cap_in, int D,
    int32_t* __restrict__ expert_load, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ rank_offset) {
  __shared__ int gsum[kScanThreads];
  __shared__ int sc[kScanThreads];
  const int tid = threadIdx.x;
  const int G = kScanThreads / Epad;
  const int g = tid / Epad, e = tid % Epad;
  const bool live = g < G && e < E;
  const int tpg = (n_tiles + G - 1) / (G > 0 ? G : 1);
  const int tb = g * tpg;
  const int te = tb + tpg < n_tiles ? tb + tpg : n_tiles;

  int sum = 0;
  if (live)
    for (int t = tb; t < te; ++t) sum += hist[(int64_t)t * E + e];
  gsum[tid] = sum;
  __syncthreads();
  int pre = 0, tot = 0;
  if (live) {
    for (int g2 = 0; g2 < G; ++g2) {
      const int v = gsum[g2 * Epad + e];
      if (g2 < g) pre += v;
      tot += v;
    }
    int run = pre;
    for (int t = tb; t < te; ++t) {
      const int v = hist[(int64_t)t * E + e];
      hist[(int64_t)t * E + e] = run;
      run += v;
    }
  }
  int kept = 0;
  if (g == 0 && e < E) {
    // an unavailable expert keeps nothing; cap_in: per-expert capacities
    const int ce = cap_in ? cap_in[e] : (unavail && unavail[e]) ? 0 : C;
    kept = tot < ce ? tot : ce;
    if (expert_load) expert_load[e] = tot;
    expert_count[e] = kept;
  }
  sc[tid] = (g == 0) ? kept : 0;
  __syncthreads();
  for (int off = 1; off < Epad; off <<= 1) {
    const int v = (tid < Epad && tid >= off) ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  // sc[i] is now the inclusive prefix over experts 0..i
  for (int i = tid; i <= E; i += kScanThreads) expert_offset[i] = i == 0 ? 0 : sc[i - 1];
  for (int r = tid; r <= D; r += kScanThreads) {
    const int i = r * (E / D);
    rank_offset[r] = i == 0 ? 0 : sc[i - 1];
  }
}

// FUSED: `base` holds the per-tile counts of slot_hist_kernel (no scan
// kernel ran), and every block derives what it needs from them itself: its
// tile's per-expert bases (the counts of the tiles before it), the totals
// n_e, min(n_e, C) and the expert offsets; block 0 also writes the scan's
// outputs.  Used when the count table is small (n_tiles x E <= 16384,
// E % 4 == 0): re-reading it in every block then costs less than a separate
// scan launch.  Otherwise `base` is the transposed table of exclusive
// prefixes (slot_scan_rows_kernel), which also wrote the kept counts; every
// block forms the expert offsets from those and block 0 writes them.
template <bool FUSED>
__global__ __launch_bounds__(kSlotThreads) void slot_rank_kernel(
    const int32_t* __restrict__ idx, int64_t B, int k, int E, int nbits, int C,
    const uint8_t* __restrict__ unavail, const int32_t* __restrict__ cap_in, int64_t BK,
    int tile, const int32_t* __restrict__ base, int32_t* __restrict__ pos,
    uint8_t* __restrict__ keep, int32_t* __restrict__ dest, int32_t* __restrict__ pack_src, int n_tiles, int D, int32_t* __restrict__ expert_load,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset_out,
    int32_t* __restrict__ rank_offset) {
  extern __shared__ int sm[];
  int* ebuf = sm;         // [tile] experts in claim order
  int* wb = sm + tile;    // [4][E] per-wavefront counts, then running bases
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t q0 = (int64_t)blockIdx.x * tile;
  const int64_t n = BK - q0 < tile ? BK - q0 : tile;
  for (int i = tid; i < tile; i += kSlotThreads) ebuf[i] = i < n ? load_expert(idx, q0 + i, B, k, E) : -1;
  for (int i = tid; i < 4 * E; i += kSlotThreads) wb[i] = 0;
  // capacity of each expert: C, or 0 for one marked unavailable
  int* cap = wb + 4 * E;
  for (int i = tid; i < E; i += kSlotThreads)
    cap[i] = cap_in ? cap_in[i] : (unavail && unavail[i]) ? 0 : C;
  __syncthreads();
  // FUSED: sbase [E] bases of this tile; soff [E + 1] expert offsets of the
  // kept rows; then scratch
  int* sbase = cap + E;
  int* soff = sbase + E;
  int* wsum = soff + E + 1;
  int kept[4];
  if constexpr (FUSED) {
    int* pb = wsum + 4;               // [G][E] partial sums of the earlier tiles
    int* pt = pb + kSlotThreads * 4;  // [G][E] partial totals
    // thread (g, c): experts 4c .. 4c + 3 (one 16-byte load per tile) over
    // the g-th of G tile groups
    const int E4 = E / 4;
    // at most 16 groups: the second phase sums G partials per expert in one
    // thread, so a large G (few experts) would make it the long pole
    int G = kSlotThreads / E4 > 0 ? kSlotThreads / E4 : 1;
    if (G > 16) G = 16;
    const int b = blockIdx.x;
    for (int i = tid; i < G * E4; i += kSlotThreads) {
      const int g = i / E4, c = i % E4;
      const int tpg = (n_tiles + G - 1) / G;
      const int t0 = g * tpg, t1 = t0 + tpg < n_tiles ? t0 + tpg : n_tiles;
      int sb[4] = {0, 0, 0, 0}, st[4] = {0, 0, 0, 0};
      for (int t = t0; t < t1; ++t) {
        const int4 v = *reinterpret_cast<const int4*>(base + (int64_t)t * E + 4 * c);
        const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          st[u] += vv[u];
          if (t < b) sb[u] += vv[u];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pb[g * E + 4 * c + u] = sb[u];
        pt[g * E + 4 * c + u] = st[u];
      }
    }
    __syncthreads();
    // thread tid: experts 4 tid .. 4 tid + 3 (E <= 1024): bases, totals,
    // kept counts
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      kept[u] = 0;
      if (e < E) {
        int sb = 0, st = 0;
        for (int g = 0; g < G; ++g) {
          sb += pb[g * E + e];
          st += pt[g * E + e];
        }
        sbase[e] = sb;
        kept[u] = st < cap[e] ? st : cap[e];
        if (b == 0) {
          if (expert_load) expert_load[e] = st;
          expert_count[e] = kept[u];
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      kept[u] = e < E ? expert_count[e] : 0;
    }
  }
  {
    // exclusive scan of the kept counts over the experts
    int run = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) run += kept[u];
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int pre = incl - run;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      if (e < E) soff[e] = pre;
      pre += kept[u];
    }
    if (tid == kSlotThreads - 1) soff[E] = pre;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = tid; i <= E; i += kSlotThreads) expert_offset_out[i] = soff[i];
    for (int r = tid; r <= D; r += kSlotThreads) rank_offset[r] = soff[r * (E / D)];
  }
  const int32_t* expert_offset = soff;

  const int S = tile / 4;  // contiguous share of each wavefront (multiple of 64)
  const unsigned long long lt = lanemask_lt(lane);
  int* mycnt = wb + wave * E;
  for (int c = 0; c < S; c += 64) {
    const int e = ebuf[wave * S + c + lane];
    const unsigned long long m = match_expert(e, nbits);
    if (e >= 0 && (m & lt) == 0) mycnt[e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSlotThreads) {
    int b = FUSED ? sbase[e] : base[(int64_t)e * n_tiles + blockIdx.x];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int cnt = wb[w * E + e];
      wb[w * E + e] = b;
      b += cnt;
    }
  }
  __syncthreads();
  for (int c = 0; c < S; c += 64) {
    const int i = wave * S + c + lane;
    const int e = ebuf[i];
    const unsigned long long m = match_expert(e, nbits);
    const int rank = __popcll(m & lt);
    int p = -1;
    if (e >= 0) p = mycnt[e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && rank == 0) mycnt[e] = p + __popcll(m);
    __builtin_amdgcn_wave_barrier();
    if (i < n) {
      const int64_t q = q0 + i;
      const int64_t j = q / B;
      const int64_t t = q - j * B;
      const int64_t o = t * k + j;
      const bool kp = e >= 0 && p < cap[e];
      const int dr = kp ? expert_offset[e] + p : -1;
      pos[o] = p;
      keep[o] = kp ? 1 : 0;
      dest[o] = dr;
      if (kp) pack_src[dr] = (int32_t)t;
    }
  }
}

// One wavefront per token row, one lane per 16-byte chunk (block: 4 tokens x
// 64 chunks): the row is read once and written to each of its kept packed
// rows (non-temporal stores: each packed row is written once and read back
// by the expert GEMM long after any cache could hold it); the token index is
// wavefront-uniform, so dest comes through scalar loads.  The column piece
// is the grid's x (fastest in dispatch order): consecutive workgroups cover
// consecutive pieces of the same rows, not the same piece of consecutive
// rows.
template <bool XBF16>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ x,
                                                   const int32_t* __restrict__ dest, int64_t B,
                                                   int k, int d, uint16_t* __restrict__ packed,
                                                   const int32_t* __restrict__ skip_eo, int skip_b,
                                                   int skip_e) {
  const int cpr = d / 8;
  // rows [lo, hi) are not written (an empty range when there is no skip)
  const int lo = skip_eo ? skip_eo[skip_b] : 0, hi = skip_eo ? skip_eo[skip_e] : 0;
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t ntb = (B + 3) / 4;
  for (int64_t tb = blockIdx.y; tb < ntb; tb += gridDim.y) {
    const int64_t t = tb * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= B || c >= cpr) continue;
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
    for (int j = 0; j < k; ++j) {
      const int r = dest[t * k + j];
      if (r >= 0 && (r < lo || r >= hi))
        __builtin_nontemporal_store(v, (u32x4*)(packed + (int64_t)r * d + c * 8));
    }
  }
}

}  // namespace

// Claim-order tiles of 256 .. 2048 assignments: small enough that the
// histogram and rank passes run on many workgroups, large enough that the
// count table stays small (<= ~256 tiles).
SlotPlan slot_plan(int64_t B, int k) {
  SlotPlan p;
  p.BK = B * k;
  p.tile = 256;
  while (p.tile < 2048 && p.BK > (int64_t)p.tile * 256) p.tile <<= 1;
  p.n_tiles = (int)((p.BK + p.tile - 1) / p.tile);
  return p;
}

size_t slot_ws_bytes(int64_t B, int k, int E) {
  const SlotPlan p = slot_plan(B, k);
  return (size_t)(p.n_tiles > 0 ? p.n_tiles : 1) * E * sizeof(int32_t);
}

hipError_t launch_slots(const int32_t* idx, int64_t B, int k, int E, int C,
                        const uint8_t* unavail, int D, int32_t* pos,
                        uint8_t* keep, int32_t* dest, int32_t* expert_load, int32_t* expert_count,
                        int32_t* expert_offset, int32_t* rank_offset, int32_t* pack_src,
                        int32_t* ws_hist, hipStream_t s, const int32_t* cap_in) {
  const SlotPlan p = slot_plan(B, k);
  int Epad = 1;
  while (Epad < E) Epad <<= 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  // small count tables: the rank blocks scan them themselves (no scan
  // launch); larger ones are scanned by one block per expert over a
  // transposed table; an empty batch only needs the single-block scan's zeros
  const bool fused = p.n_tiles > 0 && E % 4 == 0 && (int64_t)p.n_tiles * E <= 16384 &&
                     (reinterpret_cast<uintptr_t>(ws_hist) & 15u) == 0;
  const bool rows = p.n_tiles > 0 && !fused;
  if (p.n_tiles > 0) {
    hipLaunchKernelGGL(slot_hist_kernel, dim3(p.n_tiles), dim3(kSlotThreads), E * sizeof(int), s,
                       idx, B, k, E, p.BK, p.tile, rows ? 1 : 0, ws_hist);
  }
  if (rows)
    hipLaunchKernelGGL(slot_scan_rows_kernel, dim3(E), dim3(kSlotThreads), 0, s, ws_hist,
                       p.n_tiles, C, unavail, cap_in, expert_load, expert_count);
  else if (!fused)
    hipLaunchKernelGGL(slot_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, ws_hist, p.n_tiles, E,
                       Epad, C, unavail, cap_in, D, expert_load, expert_count, expert_offset,
                       rank_offset);
  if (p.n_tiles > 0) {
    // ebuf, per-wavefront counts, capacities, bases, offsets, 4 wave sums;
    // fused: + 2 x 1024 partials
    const size_t lds =
        (size_t)(p.tile + 7 * E + 5 + (fused ? 2 * 4 * kSlotThreads : 0)) * sizeof(int);
    if (fused)
      hipLaunchKernelGGL(slot_rank_kernel<true>, dim3(p.n_tiles), dim3(kSlotThreads), lds, s, idx,
                         B, k, E, nbits, C, unavail, cap_in, p.BK, p.tile, ws_hist, pos, keep,
                         dest, pack_src, p.n_tiles, D, expert_load, expert_count, expert_offset,
                         rank_offset);
    else
      hipLaunchKernelGGL(slot_rank_kernel<false>, dim3(p.n_tiles), dim3(kSlotThreads), lds, s,
                         idx, B, k, E, nbits, C, unavail, cap_in, p.BK, p.tile, ws_hist, pos,
                         keep, dest, pack_src, p.n_tiles, D, nullptr, expert_count,
                         expert_offset, rank_offset);
  }
  return hipGetLastError();
}

hipError_t launch_pack(const void* x, bool x_bf16, const int32_t* dest, int64_t B, int k, int d,
                       uint16_t* packed, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                       const int32_t* skip_eo, int skip_b, int skip_e) {
  if (B == 0) return hipSuccess;
  // x: 512-column piece of the rows (fastest in dispatch order, so
  // consecutive workgroups cover consecutive pieces of the same rows);
  // y: groups of 4 rows, at most 65535 (the kernel loops over the rest)
  const int64_t ntb = (B + 3) / 4;
  const dim3 g((unsigned)((d / 8 + 63) / 64), (unsigned)(ntb < 65535 ? ntb : 65535));
  if (x_bf16)
    launch_timed(pack_kernel<true>, dim3(g), dim3(256), 0, s, e0, e1, x, dest, B, k, d,
                 packed, skip_eo, skip_b, skip_e);
  else
    launch_timed(pack_kernel<false>, dim3(g), dim3(256), 0, s, e0, e1, x, dest, B, k, d,
                 packed, skip_eo, skip_b, skip_e);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Overflow redirected to the next-best expert ("Expert Parallelism",
// narrativegoldmine.com, "Components and Architecture": tokens routed to a
// full expert are dropped or redirected to a secondary expert).  One
// fallback round: round 1 is the slot assignment of the top-k choices; the
// m-th dropped choice of a token then goes to its (k + m)-th ranked expert
// and the redirected assignments claim the capacity left, in the original
// claim order (the slot kernels again, with per-expert capacities); the
// merge numbers round-2 rows after the expert's round-1 rows.
namespace {

__global__ __launch_bounds__(256) void split_ranked_kernel(const int32_t* __restrict__ ranked,
                                                           int64_t n, int K2, int k,
                                                           int32_t* __restrict__ idx) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / k;
    const int j = (int)(i - t * k);
    idx[i] = ranked[t * K2 + j];
  }
}

__global__ __launch_bounds__(256) void fallback_kernel(
    const int32_t* __restrict__ ranked, const uint8_t* __restrict__ keep1,
    const int32_t* __restrict__ count1, int64_t B, int K2, int k, int E, int C,
    const uint8_t* __restrict__ unavail, int32_t* __restrict__ fb, int32_t* __restrict__ rk,
    int32_t* __restrict__ rem) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < E) {
    const int cap = (unavail && unavail[t]) ? 0 : C;
    rem[t] = cap - count1[t];
  }
  if (t >= B) return;
  int m = 0;
  for (int j = 0; j < k; ++j) {
    int f = -1, r = j;
    if (!keep1[t * k + j]) {
      r = k + m;
      if (r < K2) f = ranked[t * K2 + r];
      ++m;
    }
    fb[t * k + j] = f;
    rk[t * k + j] = r;
  }
}

__global__ __launch_bounds__(1024) void merge_offsets_kernel(
    const int32_t* __restrict__ count1, const int32_t* __restrict__ count2, int E, int D,
    int32_t* __restrict__ count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ rank_offset) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;  // E <= 1024: one expert per thread
  const int c = tid < E ? count1[tid] + count2[tid] : 0;
  if (tid < E) count[tid] = c;
  sc[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  // sc[i]: inclusive prefix over experts 0..i.  E + 1 and D + 1 entries:
  // with E (or D) = 1024 the last one is past the block's 1024 threads.
  for (int i = tid; i <= E; i += 1024) expert_offset[i] = i == 0 ? 0 : sc[i - 1];
  for (int r = tid; r <= D; r += 1024) {
    const int i = r * (E / D);
    rank_offset[r] = i == 0 ? 0 : sc[i - 1];
  }
}

__global__ __launch_bounds__(256) void merge_kernel(
    const float* __restrict__ ranked_w, int64_t B, int K2, int k,
    const uint8_t* __restrict__ keep1, const int32_t* __restrict__ pos1,
    const int32_t* __restrict__ fb, const int32_t* __restrict__ rk,
    const uint8_t* __restrict__ keep2, const int32_t* __restrict__ pos2,
    const int32_t* __restrict__ count1, const int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ pos,
    uint8_t* __restrict__ keep, int32_t* __restrict__ dest, int32_t* __restrict__ pack_src) {
  const int64_t n = B * k;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / k;
    int e = idx[i];
    int slot = -1;
    float wt = ranked_w[t * K2 + (i - t * k)];
    bool kp = false;
    if (keep1[i]) {
      slot = pos1[i];
      kp = true;
    } else if (fb[i] >= 0 && keep2[i]) {
      e = fb[i];
      slot = count1[e] + pos2[i];
      wt = ranked_w[t * K2 + rk[i]];
      kp = true;
    }
    idx[i] = e;
    w[i] = wt;
    pos[i] = slot;
    keep[i] = kp ? 1 : 0;
    const int r = kp ? expert_offset[e] + slot : -1;
    dest[i] = r;
    if (kp) pack_src[r] = (int32_t)t;
  }
}

unsigned flat_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65535) g = 65535;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_split_ranked(const int32_t* ranked, int64_t B, int K2, int k, int32_t* idx,
                               hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(split_ranked_kernel, dim3(flat_grid(B * k)), dim3(256), 0, s, ranked, B * k,
                     K2, k, idx);
  return hipGetLastError();
}

hipError_t launch_fallback(const int32_t* ranked, const uint8_t* keep1, const int32_t* count1,
                           int64_t B, int K2, int k, int E, int C, const uint8_t* unavail,
                           int32_t* fb, int32_t* rk, int32_t* rem, hipStream_t s) {
  const int64_t n = B > E ? B : E;
  hipLaunchKernelGGL(fallback_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ranked,
                     keep1, count1, B, K2, k, E, C, unavail, fb, rk, rem);
  return hipGetLastError();
}

hipError_t launch_merge_offsets(const int32_t* count1, const int32_t* count2, int E, int D,
                                int32_t* count, int32_t* expert_offset, int32_t* rank_offset,
                                hipStream_t s) {
  hipLaunchKernelGGL(merge_offsets_kernel, dim3(1), dim3(1024), 0, s, count1, count2, E, D, count,
                     expert_offset, rank_offset);
  return hipGetLastError();
}

hipError_t launch_merge(const float* ranked_w, int64_t B, int K2, int k, const uint8_t* keep1,
                        const int32_t* pos1, const int32_t* fb, const int32_t* rk,
                        const uint8_t* keep2, const int32_t* pos2, const int32_t* count1,
                        const int32_t* expert_offset, int32_t* idx, float* w, int32_t* pos,
                        uint8_t* keep, int32_t* dest, int32_t* pack_src, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(flat_grid(B * k)), dim3(256), 0, s, ranked_w, B, K2, k,
                     keep1, pos1, fb, rk, keep2, pos2, count1, expert_offset, idx, w, pos, keep,
                     dest, pack_src);
  return hipGetLastError();
}

}  // namespace moek
