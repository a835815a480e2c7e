// moe_route: top-k routing with softmax gates, one wavefront per token.
//
// [jjl357] "1.1 Dense LLM 与 MoE LLM 的区别": the router selects the top-k experts of
// each token; the layer output is the gate-weighted sum of their outputs.
// Selection order: logit descending, equal logits to the lower expert id.  Each of
// the 64 lanes keeps up to 16 logits in registers; k rounds of a wave-wide
// (value, id) arg-max pick the experts.
#include <math.h>

#include "mc_common.h"

namespace mc {

constexpr int kRouteMaxPerLane = 16;   // E <= 64 * 16
constexpr int kRouteWaves = 4;         // tokens per 256-thread workgroup

// a beats b: larger value, or equal value and smaller id
__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__global__ void __launch_bounds__(64 * kRouteWaves)
route_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
             int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  float v[kRouteMaxPerLane];
  float rmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    int e = lane + 64 * i;
    float x = e < E ? row[e] : -INFINITY;
    if (x != x) x = -INFINITY;              // NaN ranks with -inf
    v[i] = x;
    rmax = fmaxf(rmax, x);
  }
  uint32_t taken = 0;                       // bit i: v[i] already selected

  float sel_v = -INFINITY;                  // lane j < k keeps the j-th pick
  int sel_id = 0;
  for (int j = 0; j < k; ++j) {
    // lane-local best among untaken
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && beats(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    // wave arg-max
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      sel_v = bv;
      sel_id = bi;
    }
  }

  // gates
  float top = __shfl(sel_v, 0, 64);         // largest selected logit
  float z;
  float denom;
  if (renorm) {
    z = lane < k ? __expf(sel_v - top) : 0.0f;
    denom = wave_sum(z);
  } else {
    float wmax = rmax;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, o, 64));
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i)
      if (lane + 64 * i < E) part += __expf(v[i] - wmax);
    denom = wave_sum(part);
    z = lane < k ? __expf(sel_v - wmax) : 0.0f;
  }
  if (lane < k) {
    topk_ids[(size_t)t * k + lane] = sel_id;
    topk_w[(size_t)t * k + lane] = z / denom;
  }
}

}  // namespace mc

using namespace mc;

extern "C" int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                         int32_t* topk_ids, float* topk_w, hipStream_t s) {
  clear_error();
  MC_REQUIRE(T >= 0, "moe_route: T=%d must be >= 0", T);
  MC_REQUIRE(E >= 1 && E <= 64 * kRouteMaxPerLane, "moe_route: E=%d must be in [1, %d]", E,
             64 * kRouteMaxPerLane);
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
