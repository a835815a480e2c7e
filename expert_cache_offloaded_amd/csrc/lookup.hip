// slot_cache_lookup_evict: one layer call of the cross-layer LRU slot cache.
//
// [jjl357] "6.1 全局 LRU 专家缓存", "6.7 系统如何选择哪 q 个专家进入缓存" and
// "8.2 把控制流表示成数据": a single GPU kernel dedups the routed experts, checks
// residency, derives q, picks LRU victims and rewrites logical ids to a slot or a
// host flag, so the whole step stays on the device (capturable, no host round trip).
// [wanger] "3. ensure_experts_hybrid 内核": the integer (Q16) split rule.
// [juhe] "生成阶段": slot_for_id / id_of_slot / usage tables.
//
// One workgroup of 1024 threads.  Unique experts of the call come from a presence
// table over the layer's E experts (so they are already in ascending flat-id order);
// ranks of hits/misses come from one workgroup prefix sum.  The layer's slot_of
// entries (and, for pools of up to 4096 slots, every slot's stamp and id_of) are read
// into registers when the kernel starts, so those reads overlap the routing and the
// victim search runs on registers.  Victims are taken in rounds:
// each round finds the smallest stamp among the evictable slots not yet taken and
// takes the slots carrying it in ascending slot order, which yields the victims in
// (stamp, slot) order without sorting.  Every round takes at least one slot, so the
// loop ends after at most q rounds.
//
// moe_route_lookup runs the router and this lookup as one launch: the workgroup's
// 16 wavefronts first route the call's tokens (one wavefront per token, the
// routine of moe_route) into LDS, and the lookup reads the ids from there.
#include "route_dev.h"

namespace mc {

constexpr int kLkThreads = 1024;
constexpr int kLkMaxE = 4096;
constexpr int kLkMaxRoutes = 2048;
constexpr int kLkPerE = kLkMaxE / kLkThreads;     // experts of the layer per thread, at most
constexpr int kLkFastS = 4096;                    // pools up to this size: slot table in registers
constexpr int kLkPerS = kLkFastS / kLkThreads;    // slots per thread then

// x plus the value a DPP move brings; lanes outside ROW_MASK, and lanes whose source
// lies outside their row, add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_i32(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes: shifts inside each row of 16, then row 0's
// last lane into row 1, row 2's into row 3, and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = dpp_add_i32<0x111, 0xF>(x);   // row_shr:1
  x = dpp_add_i32<0x112, 0xF>(x);   // row_shr:2
  x = dpp_add_i32<0x114, 0xF>(x);   // row_shr:4
  x = dpp_add_i32<0x118, 0xF>(x);   // row_shr:8
  x = dpp_add_i32<0x142, 0xA>(x);   // row_bcast:15
  x = dpp_add_i32<0x143, 0xC>(x);   // row_bcast:31
  return x;
}

// Exclusive prefix sum of one int per thread over the workgroup; returns the
// thread's offset and writes the total to *total (all threads).  Each wave scans its
// lanes, publishes its total, and then scans the 16 wave totals itself.  With TRAIL the
// scan ends with a barrier, so sh_wave may be written again at once; without it, the
// caller passes another barrier before the next write.
template <bool TRAIL = true>
__device__ int block_excl_scan(int v, int* sh_wave, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) sh_wave[wid] = x;
  __syncthreads();
  const int w = lane < kLkThreads / 64 ? sh_wave[lane] : 0;
  const int wi = wave_incl_scan(w);
  const int before = __builtin_amdgcn_readlane(wi - w, wid);   // waves ahead of this one
  *total = __builtin_amdgcn_readlane(wi, kLkThreads / 64 - 1);
  if (TRAIL) __syncthreads();              // sh_wave is written again by the next scan
  return before + x - v;
}

// Minimum over the workgroup of a non-negative int64 (stamps, INT64_MAX for none):
// a DPP wave minimum (the route's 64-bit max on the complemented value), one LDS
// slot per wave, and every wave reduces the 16 slots itself.  The slots are written
// again only after the caller's next barrier.
__device__ __forceinline__ int64_t wave_min_nonneg(int64_t v) {
  return (int64_t)~wave_max_u64(~(uint64_t)v);
}

// Maximum over the workgroup of an unsigned 32-bit value: a DPP wave maximum, one LDS
// slot per wave, and every wave reduces the 16 slots itself.  The slots are written
// again only after the caller's next barrier.
__device__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_max_u32(v);
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  return wave_max_u32(lane < kLkThreads / 64 ? sh[lane] : 0u);
}

__device__ int64_t block_min_nonneg(int64_t v, int64_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_min_nonneg(v);
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  return wave_min_nonneg(lane < kLkThreads / 64 ? sh[lane] : INT64_MAX);
}

template <bool ROUTE, bool FAST>
__global__ void __launch_bounds__(kLkThreads)
lookup_kernel(const float* __restrict__ logits, int32_t renorm, int32_t* __restrict__ topk_ids,
              float* __restrict__ topk_w,
              int32_t L, int32_t E, int32_t S, int32_t* __restrict__ slot_of,
              int32_t* __restrict__ id_of, int64_t* __restrict__ stamp, int64_t* __restrict__ clock_p,
              int64_t* __restrict__ stats, int32_t layer, const int32_t* ids, int32_t T,
              int32_t k, const int32_t* __restrict__ n_tok, uint32_t frac_q16, int32_t fixed_cap,
              int32_t min_fill, int32_t* __restrict__ slots, int32_t* __restrict__ fill_flat,
              int32_t* __restrict__ fill_slot, int32_t* __restrict__ n_fill,
              int32_t* __restrict__ host_flat, int32_t* __restrict__ n_host, int32_t kcap) {
  __shared__ uint8_t s_present[kLkMaxE];     // 1 if expert e is routed in this call
  __shared__ int32_t s_slot_e[kLkMaxE];      // slot of expert e after the call, -1 = none
  __shared__ int32_t s_victim[kLkMaxRoutes]; // victims in (stamp, slot) order
  __shared__ int32_t s_vold[FAST ? kLkMaxRoutes : 1];   // the flat id each victim held
  __shared__ int32_t s_miss[kLkMaxRoutes];   // misses, ascending flat id
  __shared__ uint8_t s_hit_slot[FAST ? kLkFastS : 1];   // 1 if the slot is a hit of this call
  __shared__ int32_t s_so[kLkMaxE];                     // slot_of of the layer's experts
  __shared__ int64_t s_st[FAST ? kLkFastS : 1];         // stamp of every slot (FAST)
  __shared__ int32_t s_id[FAST ? kLkFastS : 1];         // id_of of every slot (FAST)
  __shared__ int s_scan[kLkThreads / 64 + 1];
  __shared__ int64_t s_min[kLkThreads / 64];
  __shared__ uint32_t s_max32[kLkThreads / 64];
  __shared__ int s_err, s_evict;
  __shared__ int32_t s_ids[ROUTE ? kLkMaxRoutes : 1];

  const int tid = threadIdx.x, wid = tid >> 6;
  // the scalars the call reads and later updates, read before anything else so their
  // round trips overlap the routing (nothing in the call writes them before the end)
  const int64_t clock0 = *clock_p;
  const int n_tok_in = n_tok ? *n_tok : T;
  int64_t stats0[MC_STAT_ERR + 1];
  if (tid == 0)
#pragma unroll
    for (int i = 0; i <= MC_STAT_ERR; ++i) stats0[i] = stats[i];
  // each thread owns a contiguous run of the layer's experts (so ranks follow e order)
  // and of the slots
  const int per = (E + kLkThreads - 1) / kLkThreads;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  const int sper = (S + kLkThreads - 1) / kLkThreads;
  const int s0 = tid * sper, s1 = min(S, s0 + sper);
  for (int e = tid; e < E; e += kLkThreads) {
    s_present[e] = 0;
    s_slot_e[e] = -1;
  }
  if (FAST)
    for (int sl = tid; sl < S; sl += kLkThreads) s_hit_slot[sl] = 0;
  if (tid == 0) {
    s_err = 0;
    s_evict = 0;
  }
  // the tables the lookup reads (the layer's slot_of; with FAST every slot's stamp and
  // id_of) go to LDS, loaded by the waves that do not route while the others route,
  // so neither the routing nor the later phases wait on these reads
  constexpr int kWaves = kLkThreads / 64;
  const int route_waves = ROUTE ? min(T, kWaves) : 0;
  auto load_tables = [&](int w_first) {
    const int nthr = (kWaves - w_first) * 64, i0 = tid - w_first * 64;
    for (int e = i0; e < E; e += nthr) s_so[e] = slot_of[(int64_t)layer * E + e];
    if (FAST)
      for (int sl = i0; sl < S; sl += nthr) {
        s_st[sl] = stamp[sl];
        s_id[sl] = id_of[sl];
      }
  };
  if (route_waves < kWaves && wid >= route_waves) load_tables(route_waves);
  // 0. (fused form) route every token of the call: ids go to LDS and to topk_ids
  if (ROUTE) {
    const int lane = tid & 63;
    for (int t = tid >> 6; t < T; t += kLkThreads / 64) {   // wave-uniform
      int id;
      float gate;
      route_token_any(logits + (size_t)t * E, E, k, renorm, &id, &gate);
      if (lane < k) {
        s_ids[t * k + lane] = id;
        topk_ids[(size_t)t * k + lane] = id;
        topk_w[(size_t)t * k + lane] = gate;
      }
    }
    ids = s_ids;
  }
  if (route_waves == kWaves) load_tables(0);     // every wave routed
  const int nt = min(max(n_tok_in, 0), T);
  const int nroutes = nt * k;
  const int64_t clock = clock0 + 1;
  __syncthreads();

  // 1. presence of the valid routes
  int my_err = 0;
  for (int r = tid; r < nroutes; r += kLkThreads) {
    int e = ids[r];
    if (e == -1) continue;
    if (e < 0 || e >= E) {
      ++my_err;
      continue;
    }
    s_present[e] = 1;
  }
  if (my_err) atomicAdd(&s_err, my_err);
  __syncthreads();

  // 2. hits are stamped; misses ranked in ascending expert order (one scan of both
  //    counts, hits in the high half)
  int my_hits = 0, my_miss = 0;
#pragma unroll
  for (int j = 0; j < kLkPerE; ++j) {
    const int e = e0 + j;
    if (e >= e1 || !s_present[e]) continue;
    const int sl = s_so[e];
    if (sl >= 0 && sl < S) {
      stamp[sl] = clock;
      s_slot_e[e] = sl;
      if (FAST) s_hit_slot[sl] = 1;
      ++my_hits;
    } else {
      ++my_miss;
    }
  }
  int both;
  const int both_off = block_excl_scan((my_hits << 16) | my_miss, s_scan, &both);
  const int m = both & 0xFFFF, n_hits = both >> 16;
  {
    int i = both_off & 0xFFFF;
#pragma unroll
    for (int j = 0; j < kLkPerE; ++j) {
      const int e = e0 + j;
      if (e < e1 && s_present[e] && s_slot_e[e] < 0) s_miss[i++] = layer * E + e;
    }
  }
  __syncthreads();

  // 3. split count (integer rule), capped by evictable slots and list capacity
  int q;
  if (m == 0) {
    q = 0;
  } else if (frac_q16 == 0) {
    q = min(m, fixed_cap);
  } else {
    // The slower branch, max(F (1 - f), (m - F) f), falls while the host share
    // dominates (F < m f) and rises after; of the two integers around m f the upper
    // one wins exactly when f (m + 1) > floor(m f) + 1, so the minimiser (ties to the
    // smaller F) is ceil(f (m + 1)) - 1, which is at most m.  In Q16 integers:
    q = (int)(((int64_t)frac_q16 * (m + 1) - 1) >> 16);
  }
  if (min_fill && m >= 1) q = max(q, 1);
  q = min(q, S - n_hits);
  q = min(q, kcap);

  // 4. victims in (stamp, slot) order, in rounds of equal stamp (FAST: on the stamps
  //    read at the start, a hit of this call counting as stamped now)
  int taken = 0;
  int64_t floor_stamp = -1;   // stamps <= floor_stamp were exhausted by earlier rounds
  int64_t st_e[kLkPerS];
  bool exact64 = !FAST;       // the 64-bit rounds: large pools, or a stamp 2^32 calls old
  if (FAST) {
#pragma unroll
    for (int j = 0; j < kLkPerS; ++j)
      st_e[j] = s0 + j < s1 ? (s_hit_slot[s0 + j] ? clock : s_st[s0 + j]) : INT64_MAX;
    // FAST rounds on ages clock - stamp of the evictable slots (0 for the rest), saturated
    // to 32 bits: a round takes the largest age not yet taken (the smallest stamp) with one
    // 32-bit block maximum and one scan, two barriers
    uint32_t age[kLkPerS];
#pragma unroll
    for (int j = 0; j < kLkPerS; ++j)
      age[j] = (s0 + j < s1 && st_e[j] < clock) ? (uint32_t)min(clock - st_e[j], (int64_t)0xFFFFFFFF) : 0u;
    uint32_t lim = 0xFFFFFFFFu;   // ages above lim were taken by earlier rounds
    while (taken < q) {
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < kLkPerS; ++j)
        if (age[j] <= lim && age[j] > mine) mine = age[j];
      const uint32_t amax = block_max_u32(mine, s_max32);
      if (amax == 0u) break;                  // no evictable slot left (inconsistent tables)
      if (amax == 0xFFFFFFFFu) {              // saturated (first round only): exact rounds
        exact64 = true;
        break;
      }
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kLkPerS; ++j) cnt += age[j] == amax;
      int tot;
      int off = block_excl_scan<false>(cnt, s_scan, &tot);
      const int need = q - taken;
#pragma unroll
      for (int j = 0; j < kLkPerS; ++j)
        if (age[j] == amax && off < need) {
          s_victim[taken + off] = s0 + j;
          s_vold[taken + off] = s_id[s0 + j];
          ++off;
        }
      taken += min(tot, need);
      lim = amax - 1u;
    }
    __syncthreads();                          // the victims are read by other threads
  }
  while (exact64 && taken < q) {
    int64_t mine = INT64_MAX;
    if (FAST) {
#pragma unroll
      for (int j = 0; j < kLkPerS; ++j)
        if (st_e[j] > floor_stamp && st_e[j] < clock && st_e[j] < mine) mine = st_e[j];
    } else {
      for (int sl = s0; sl < s1; ++sl) {
        const int64_t st = stamp[sl];
        if (st > floor_stamp && st < clock && st < mine) mine = st;
      }
    }
    const int64_t smin = block_min_nonneg(mine, s_min);
    int cnt = 0;
    if (FAST) {
#pragma unroll
      for (int j = 0; j < kLkPerS; ++j) cnt += s0 + j < s1 && st_e[j] == smin;
    } else {
      for (int sl = s0; sl < s1; ++sl) cnt += stamp[sl] == smin;
    }
    int tot;
    int off = block_excl_scan(cnt, s_scan, &tot);
    const int need = q - taken;
    if (FAST) {
#pragma unroll
      for (int j = 0; j < kLkPerS; ++j)
        if (s0 + j < s1 && st_e[j] == smin && off < need) {
          s_victim[taken + off] = s0 + j;
          s_vold[taken + off] = s_id[s0 + j];
          ++off;
        }
    } else {
      for (int sl = s0; sl < s1 && off < need; ++sl)
        if (stamp[sl] == smin) s_victim[taken + off++] = sl;
    }
    taken += min(tot, need);
    floor_stamp = smin;
    __syncthreads();
    if (tot == 0) break;   // no evictable slot left (only with inconsistent tables)
  }
  q = taken;

  // 5. install the first q misses into the victims
  int my_evict = 0;
  for (int i = tid; i < q; i += kLkThreads) {
    const int sl = s_victim[i];
    const int f = s_miss[i];
    const int old = FAST ? s_vold[i] : id_of[sl];
    if (old >= 0 && old < L * E) {
      slot_of[old] = -1;
      ++my_evict;
    }
    slot_of[f] = sl;
    id_of[sl] = f;
    stamp[sl] = clock;
    s_slot_e[f - layer * E] = sl;
    fill_flat[i] = f;
    fill_slot[i] = sl;
  }
  for (int i = q + tid; i < m; i += kLkThreads) host_flat[i - q] = s_miss[i];
  if (my_evict) atomicAdd(&s_evict, my_evict);
  __syncthreads();
  const int n_evict = s_evict;

  // 6. rewrite routes to slots (-1 = host-computed, masked, invalid, beyond n_tok)
  for (int r = tid; r < T * k; r += kLkThreads) {
    int v = -1;
    if (r < nroutes) {
      int e = ids[r];
      if (e >= 0 && e < E) v = s_slot_e[e];
    }
    slots[r] = v;
  }

  if (tid == 0) {
    *clock_p = clock;
    *n_fill = q;
    *n_host = m - q;
    stats[MC_STAT_HITS] = stats0[MC_STAT_HITS] + n_hits;
    stats[MC_STAT_MISSES] = stats0[MC_STAT_MISSES] + m;
    stats[MC_STAT_FILLS] = stats0[MC_STAT_FILLS] + q;
    stats[MC_STAT_HOST] = stats0[MC_STAT_HOST] + m - q;
    stats[MC_STAT_EVICT] = stats0[MC_STAT_EVICT] + n_evict;
    stats[MC_STAT_CALLS] = stats0[MC_STAT_CALLS] + 1;
    stats[MC_STAT_ERR] = stats0[MC_STAT_ERR] + s_err;
  }
}

}  // namespace mc

using namespace mc;

// argument checks shared by both entry points
static int check_lookup(const mc_cache* c, int32_t layer, int32_t T, int32_t k, uint32_t frac_q16,
                        int32_t fixed_cap, int32_t kcap, const char* fn) {
  MC_REQUIRE(c != nullptr, "%s: cache is NULL", fn);
  MC_REQUIRE(c->L > 0 && c->E > 0 && c->S > 0, "%s: L=%d E=%d S=%d", fn, c->L, c->E, c->S);
  MC_REQUIRE(c->E <= kLkMaxE, "%s: E=%d exceeds %d", fn, c->E, kLkMaxE);
  MC_REQUIRE((int64_t)c->L * c->E < (1ll << 31), "%s: L*E too large", fn);
  MC_REQUIRE(c->slot_of && c->id_of && c->stamp && c->clock && c->stats, "%s: NULL table pointer", fn);
  MC_REQUIRE(layer >= 0 && layer < c->L, "%s: layer=%d not in [0, %d)", fn, layer, c->L);
  MC_REQUIRE(T >= 0 && k >= 1, "%s: T=%d k=%d", fn, T, k);
  MC_REQUIRE((int64_t)T * k <= kLkMaxRoutes, "%s: T*k=%lld exceeds %d", fn, (long long)T * k,
             kLkMaxRoutes);
  MC_REQUIRE(frac_q16 <= 65536u, "%s: frac_q16=%u exceeds 65536", fn, frac_q16);
  MC_REQUIRE(fixed_cap >= 0, "%s: fixed_cap=%d must be >= 0", fn, fixed_cap);
  MC_REQUIRE(kcap >= T * k, "%s: kcap=%d < T*k=%d", fn, kcap, T * k);
  return MC_OK;
}

extern "C" int slot_cache_lookup_evict(const mc_cache* c, int32_t layer, const int32_t* ids,
                                       int32_t T, int32_t k, const int32_t* n_tok,
                                       uint32_t frac_q16, int32_t fixed_cap, int32_t min_fill,
                                       int32_t* slots, int32_t* fill_flat, int32_t* fill_slot,
                                       int32_t* n_fill, int32_t* host_flat, int32_t* n_host,
                                       int32_t kcap, hipStream_t s) {
  clear_error();
  int rc;
  if ((rc = check_lookup(c, layer, T, k, frac_q16, fixed_cap, kcap, "slot_cache_lookup_evict")) != MC_OK)
    return rc;
  MC_REQUIRE(ids && slots && fill_flat && fill_slot && n_fill && host_flat && n_host,
             "slot_cache_lookup_evict: NULL pointer");
  auto kern = c->S <= kLkFastS ? lookup_kernel<false, true> : lookup_kernel<false, false>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kLkThreads), 0, s, nullptr, 0, nullptr,
                     nullptr, c->L, c->E, c->S, c->slot_of, c->id_of, c->stamp, c->clock, c->stats,
                     layer, ids, T, k, n_tok, frac_q16, fixed_cap, min_fill, slots, fill_flat,
                     fill_slot, n_fill, host_flat, n_host, kcap);
  MC_LAUNCH_CHECK();
  return MC_OK;
}

extern "C" int moe_route_lookup(const float* logits, int32_t renorm, int32_t* topk_ids,
                                float* topk_w, const mc_cache* c, int32_t layer, int32_t T,
                                int32_t k, const int32_t* n_tok, uint32_t frac_q16,
                                int32_t fixed_cap, int32_t min_fill, int32_t* slots,
                                int32_t* fill_flat, int32_t* fill_slot, int32_t* n_fill,
                                int32_t* host_flat, int32_t* n_host, int32_t kcap, hipStream_t s) {
  clear_error();
  int rc;
  if ((rc = check_lookup(c, layer, T, k, frac_q16, fixed_cap, kcap, "moe_route_lookup")) != MC_OK)
    return rc;
  MC_REQUIRE(c->E <= kRouteMaxE, "moe_route_lookup: E=%d exceeds %d", c->E, kRouteMaxE);
  MC_REQUIRE(k <= c->E && k <= 32, "moe_route_lookup: k=%d must be in [1, min(E, 32)]", k);
  MC_REQUIRE(renorm == 0 || renorm == 1, "moe_route_lookup: renorm=%d must be 0 or 1", renorm);
  MC_REQUIRE(logits && topk_ids && topk_w && slots && fill_flat && fill_slot && n_fill && host_flat &&
                 n_host,
             "moe_route_lookup: NULL pointer");
  auto kern = c->S <= kLkFastS ? lookup_kernel<true, true> : lookup_kernel<true, false>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kLkThreads), 0, s, logits, renorm, topk_ids,
                     topk_w, c->L, c->E, c->S, c->slot_of, c->id_of, c->stamp, c->clock, c->stats,
                     layer, topk_ids, T, k, n_tok, frac_q16, fixed_cap, min_fill, slots, fill_flat,
                     fill_slot, n_fill, host_flat, n_host, kcap);
  MC_LAUNCH_CHECK();
  return MC_OK;
}

namespace mc {

// ---------------------------------------------------------------- install

// flat[i] -> slot i on a cache that holds no expert: slot_of / id_of set, stamp = a
// new clock tick (so the installed experts are more recent than the empty slots and
// less recent than anything the next call touches).  Id -1 leaves slot i empty.  Another
// id outside [0, L*E), one already placed (a duplicate in the list) or an occupied slot
// is skipped and counted in stats[err].  One workgroup: every lane reads the clock
// before the barrier, lane 0 advances it after.
__global__ void __launch_bounds__(256)
install_kernel(int32_t LE, int32_t S, int32_t* __restrict__ slot_of, int32_t* __restrict__ id_of,
               int64_t* __restrict__ stamp, int64_t* __restrict__ clock_p,
               int64_t* __restrict__ stats, const int32_t* __restrict__ flat, int32_t n) {
  const int64_t tick = *clock_p + 1;
  int errs = 0;
  for (int i = threadIdx.x; i < n && i < S; i += blockDim.x) {
    const int f = flat[i];
    if (f == -1) continue;
    if (id_of[i] != -1 || f < 0 || f >= LE || atomicCAS(&slot_of[f], -1, i) != -1) {
      ++errs;
      continue;
    }
    id_of[i] = f;
    stamp[i] = tick;
  }
  if (errs) atomicAdd(reinterpret_cast<unsigned long long*>(&stats[MC_STAT_ERR]), (unsigned long long)errs);
  __syncthreads();
  if (threadIdx.x == 0) *clock_p = tick;
}

}  // namespace mc

extern "C" int mc_cache_install(const mc_cache* c, const int32_t* flat, int32_t n, hipStream_t s) {
  clear_error();
  MC_REQUIRE(c != nullptr && c->L > 0 && c->E > 0 && c->S > 0, "mc_cache_install: bad cache");
  MC_REQUIRE(c->slot_of && c->id_of && c->stamp && c->clock && c->stats,
             "mc_cache_install: NULL table pointer");
  MC_REQUIRE(n >= 0 && n <= c->S, "mc_cache_install: n=%d not in [0, S=%d]", n, c->S);
  if (n == 0) return MC_OK;
  MC_REQUIRE(flat != nullptr, "mc_cache_install: NULL list");
  hipLaunchKernelGGL(install_kernel, dim3(1), dim3(256), 0, s, c->L * c->E, c->S,
                     c->slot_of, c->id_of, c->stamp, c->clock, c->stats, flat, n);
  MC_LAUNCH_CHECK();
  return MC_OK;
}
