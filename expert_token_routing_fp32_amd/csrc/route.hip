// Softmax over E and top-k selection, one token per group of L lanes.
//
// "Expert Parallelism" (narrativegoldmine.com), "Formal Algorithm":
// p_t = softmax(g_t / tau), e(t) = argmax p_t and w_t = p_{t,e(t)};
// "Components and Architecture": the top-k experts of that distribution are
// selected.  Experts are ranked by (logit descending, index ascending): the
// order of the exact probabilities, since softmax is strictly increasing, with
// ties to the lower index.  Ranking on the logits rather than on rounded fp32
// probabilities keeps the choice exact.  The weights are the raw
// probabilities of the chosen experts.
//
// A token's E logits are spread over L lanes, V per lane: L = pow2 >= E up to
// 16 experts, 16 lanes up to 512 experts, 64 beyond.
// Max, sum and each of the k arg-max rounds are butterfly reductions inside
// the L-lane segment of the 64-wide wavefront.
#include "launch.h"
#include "moe_kernels.h"

namespace moek {
namespace {

constexpr int kRouteThreads = 256;

template <int L, int V>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ logits, int64_t B, int E, int k, float inv_tau,
    int32_t* __restrict__ idx, float* __restrict__ w) {
  const int tid = threadIdx.x;
  const int64_t t = ((int64_t)blockIdx.x * kRouteThreads + tid) / L;
  const int li = tid % L;
  const bool tok = t < B;
  route_token<L, V>(logits + (tok ? t : 0) * E, E, k, inv_tau, li, tok, idx + t * k, w + t * k);
}

template <int L, int V>
hipError_t go(const float* logits, int64_t B, int E, int k, float tau, int32_t* idx, float* w,
              hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t threads = B * L;
  dim3 grid((unsigned)((threads + kRouteThreads - 1) / kRouteThreads));
  launch_timed((route_kernel<L, V>), grid, dim3(kRouteThreads), 0, s, e0, e1, logits,
               B, E, k, 1.0f / tau, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t B, int E, int k, float tau, int32_t* idx,
                        float* w, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (B == 0) return hipSuccess;
  if (E <= 1) return go<1, 1>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 2) return go<2, 1>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 4) return go<4, 1>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 8) return go<8, 1>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 16) return go<16, 1>(logits, B, E, k, tau, idx, w, s, e0, e1);
  // 16 lanes per token from 32 experts up: each lane walks E / 16 logits
  // itself and the butterflies take 4 steps instead of 6 (measured: 128
  // experts 9.9 -> 5.9 us, 256 experts x 32768 tokens 56 -> 35 us); past
  // 512 experts the per-lane walk costs more than it saves
  if (E <= 32) return go<16, 2>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 64) return go<16, 4>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 128) return go<16, 8>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 256) return go<16, 16>(logits, B, E, k, tau, idx, w, s, e0, e1);
  if (E <= 512) return go<16, 32>(logits, B, E, k, tau, idx, w, s, e0, e1);
  return go<64, 16>(logits, B, E, k, tau, idx, w, s, e0, e1);
}

}  // namespace moek
