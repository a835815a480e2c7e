// Device routine of top-k routing for one token on one wavefront, shared by
// moe_route and moe_route_lookup.
//
// [jjl357] "1.1 Dense LLM 与 MoE LLM 的区别": the router keeps the k experts with the
// largest logits; the layer output is their gate-weighted sum.  Order: logit
// descending, equal logits to the lower expert id; NaN ranks with -inf.
//
// Each (logit, id) pair becomes one 64-bit key whose unsigned order is that
// selection order: high word = the logit's bits mapped to an order-preserving
// unsigned integer, low word = 0xFFFF - id.  A lane holds NPER keys (ids lane,
// lane + 64, ...); each of the k rounds takes the lane-local best untaken key and a
// wavefront max built from DPP lane moves (no LDS traffic), then the owner marks it
// taken.  Padding lanes (id >= E) hold key 0, below every real key.
#pragma once

#include <math.h>

#include "mc_common.h"

namespace mc {

constexpr int kRouteMaxE = 1024;

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  if (v != v) v = -INFINITY;
  if (v == 0.0f) v = 0.0f;           // -0 and +0 compare equal: the lower id wins
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xFFFFu - (uint32_t)(key & 0xFFFFu)); }

// max(v, DPP-moved v) on a 64-bit key; lanes outside row_mask keep v
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t mlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t mhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  const uint64_t m = ((uint64_t)mhi << 32) | mlo;
  return m > v ? m : v;
}

// Maximum over the 64 lanes, returned to every lane (wave-uniform).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]: pairs
  v = dpp_max_u64<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]: quads
  v = dpp_max_u64<0x141, 0xF>(v);   // row_half_mirror: 8 lanes
  v = dpp_max_u64<0x140, 0xF>(v);   // row_mirror: rows of 16
  v = dpp_max_u64<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_u64<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3: lane 63 holds the max
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Top-k of one logits row on the calling wavefront.  Lane j < k returns the j-th
// pick in *id and its gate in *gate (softmax over the k picks when renorm, else the
// full-softmax probability); other lanes return id -1.  Needs E <= 64 * NPER, k <= 64.
template <int NPER>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int renorm,
                                            int* id, float* gate) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NPER];
  float val[NPER];                   // logits, NaN as -inf (padding -inf)
  float rmax = -INFINITY;
  // every logit read is issued before the first is used (a read under e < E would be a
  // branch holding its own wait, one round trip per read); padding lanes read logit E - 1
  float raw[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) raw[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    float x = e < E ? raw[i] : -INFINITY;
    if (x != x) x = -INFINITY;
    val[i] = x;
    key[i] = e < E ? route_key(x, e) : 0ull;
    rmax = fmaxf(rmax, x);
  }
  uint64_t mine = 0;                 // lane j keeps pick j
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t w = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (key[i] == w) key[i] = 0;   // taken (keys are unique)
    if (lane == j) mine = w;
  }
  const float v = key_value(mine);
  const float top = __shfl(v, 0, 64);                     // the largest pick
  float z, denom;
  if (renorm) {
    z = lane < k ? __expf(v - top) : 0.0f;
    denom = wave_sum(z);
  } else {
    float wmax = rmax;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, o, 64));
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + 64 * i < E) part += __expf(val[i] - wmax);
    denom = wave_sum(part);
    z = lane < k ? __expf(v - wmax) : 0.0f;
  }
  *id = lane < k ? key_id(mine) : -1;
  *gate = z / denom;
}

// Dispatch on the number of logits per lane.
__device__ __forceinline__ void route_token_any(const float* __restrict__ row, int E, int k, int renorm,
                                                int* id, float* gate) {
  if (E <= 64) route_token<1>(row, E, k, renorm, id, gate);
  else if (E <= 128) route_token<2>(row, E, k, renorm, id, gate);
  else if (E <= 256) route_token<4>(row, E, k, renorm, id, gate);
  else if (E <= 512) route_token<8>(row, E, k, renorm, id, gate);
  else route_token<16>(row, E, k, renorm, id, gate);
}

}  // namespace mc
