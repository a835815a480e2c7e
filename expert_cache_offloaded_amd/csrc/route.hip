// moe_route: top-k routing with softmax gates, one wavefront per token.
//
// [jjl357] "1.1 Dense LLM 与 MoE LLM 的区别": the router selects the top-k experts of
// each token; the layer output is the gate-weighted sum of their outputs.
// Selection order: logit descending, equal logits to the lower expert id; the
// per-token routine (64-bit keys, DPP wavefront max) is in route_dev.h.
#include "route_dev.h"

namespace mc {

constexpr int kRouteWaves = 4;         // tokens per 256-thread workgroup

__global__ void __launch_bounds__(64 * kRouteWaves)
route_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
             int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;                  // wave-uniform
  int id;
  float gate;
  route_token_any(logits + (size_t)t * E, E, k, renorm, &id, &gate);
  if (lane < k) {
    topk_ids[(size_t)t * k + lane] = id;
    topk_w[(size_t)t * k + lane] = gate;
  }
}

}  // namespace mc

using namespace mc;

extern "C" int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                         int32_t* topk_ids, float* topk_w, hipStream_t s) {
  clear_error();
  MC_REQUIRE(T >= 0, "moe_route: T=%d must be >= 0", T);
  MC_REQUIRE(E >= 1 && E <= kRouteMaxE, "moe_route: E=%d must be in [1, %d]", E, kRouteMaxE);
  MC_REQUIRE(k >= 1 && k <= E && k <= 32, "moe_route: k=%d must be in [1, min(E, 32)]", k);
  MC_REQUIRE(renorm == 0 || renorm == 1, "moe_route: renorm=%d must be 0 or 1", renorm);
  if (T == 0) return MC_OK;
  MC_REQUIRE(logits && topk_ids && topk_w, "moe_route: NULL pointer");
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(route_kernel, grid, dim3(64 * kRouteWaves), 0, s, logits, T, E, k, renorm,
                     topk_ids, topk_w);
  MC_LAUNCH_CHECK();
  return MC_OK;
}
