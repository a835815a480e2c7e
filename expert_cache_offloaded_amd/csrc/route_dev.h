// Device routine of top-k routing for one token on one wavefront, shared by
// moe_route and moe_route_lookup.
//
// [jjl357] "1.1 Dense LLM 与 MoE LLM 的区别": the router keeps the k experts with the
// largest logits; the layer output is their gate-weighted sum.  Order: logit
// descending, equal logits to the lower expert id; NaN ranks with -inf.
//
// Each logit becomes a 32-bit value whose unsigned order is the logit order (NaN as -inf,
// -0 as +0).  A lane holds NPER of them (ids lane, lane + 64, ...); each of the k rounds
// takes the lane-local best untaken entry and a wavefront max built from DPP lane moves
// (no LDS traffic); equal logits in several lanes go to the lowest id, found with ballots.
// The 64-bit wavefront max below serves the lookup's stamp minimum.
#pragma once

#include <math.h>

#include "mc_common.h"

namespace mc {

constexpr int kRouteMaxE = 1024;

// max(v, DPP-moved v) on a 64-bit value; lanes outside row_mask keep v
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

// Order-preserving 32-bit image of a logit (NaN as -inf, -0 as +0).  Every logit maps above
// 0, so 0 marks a taken or padding entry.
__device__ __forceinline__ uint32_t logit_order(float v) {
  if (v != v) v = -INFINITY;
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_value(uint32_t ord) {
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

// max(v, DPP-moved v); lanes outside ROW_MASK keep v
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
  return m > v ? m : v;
}

// Maximum over the 64 lanes, returned to every lane (wave-uniform).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1, 0xF>(v);
  v = dpp_max_u32<0x4E, 0xF>(v);
  v = dpp_max_u32<0x141, 0xF>(v);
  v = dpp_max_u32<0x140, 0xF>(v);
  v = dpp_max_u32<0x142, 0xA>(v);
  v = dpp_max_u32<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one logits row on the calling wavefront.  Lane j < k returns the j-th
// pick in *id and its gate in *gate (softmax over the k picks when renorm, else the
// full-softmax probability); other lanes return id -1.  Needs E <= 64 * NPER, k <= 64.
// A lane holds the ordered logits of ids lane, lane + 64, ...; each of the k rounds takes
// every lane's best untaken entry (the lowest id of its equal ones), a 32-bit DPP wave
// maximum of those, and, when several lanes hold that value, the lowest id among them
// (the lowest entry index first, then the lowest lane); the winner marks its entry taken.
template <int NPER>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int renorm,
                                            int* id, float* gate) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NPER];
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
    key[i] = e < E ? logit_order(x) : 0u;
    rmax = fmaxf(rmax, x);
  }
  uint32_t mine = 0;                 // lane j keeps pick j
  int mine_id = -1;
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (key[i] > best) {           // strict: the lowest index wins among equal entries
        best = key[i];
        bi = i;
      }
    const uint32_t m = wave_max_u32(best);
    const uint64_t cand = __ballot(best == m);
    uint64_t c = cand;
    if (__popcll(cand) > 1) {        // equal logits in several lanes: the lowest entry index
      c = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (c == 0) c = __ballot(best == m && bi == i);
    }
    const int w = (int)__builtin_ctzll(c);
    const int wi = __builtin_amdgcn_readlane(bi, w);
    if (lane == w) {
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i == wi) key[i] = 0u;
    }
    if (lane == j) {
      mine = m;
      mine_id = w + 64 * wi;
    }
  }
  const float v = order_value(mine);
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
  *id = lane < k ? mine_id : -1;
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
