// moe_experts_decode: slot-indirected SwiGLU experts + gated combine for decode.
//
// [jjl357] "1.1": h_t = sum_e p_{t,e} Expert_{l,e}(x_t).  [jjl357] "6.1": an expert
// routed by several tokens of the call is read and run once.  [jjl357] "6.7" step 5
// and [wanger] "代码全链路": the GPU runs hits + fills; host-computed routes arrive
// with slot -1 (or gate 0) and are skipped.
//
// Decode is a GEMV that streams ~0.53 B of MXFP4 weight per multiply-add, so it is
// bound by HBM bandwidth; at batch 1 a layer moves only ~15 MB, so what matters is
// having every weight load of a wave in flight at once (no branch or conversion
// between a load and the next one).  Two kernels, no cross-workgroup waiting:
//   gate_up: workgroup = (unit, 4 WR intermediate rows); a unit is one distinct slot of
//      the call, run by the grid column of the first route that holds it, or the
//      shared expert.  Each wave owns WR gate rows and the WR matching up rows; lane
//      l reads the 16-byte chunks l, l+64, ... of every row (one coalesced 1 KiB
//      row slice per load instruction), keeps them in registers and reuses them for
//      every token that routes to the unit.  Dot
//      products run on packed bf16 (MXFP4 -> bf16 is exact) with fp32 accumulation;
//      h = silu(g) * u is written in fp32 per route.
//   down: workgroup = (ROWS hidden rows, one token), over every route of the token.
//      The token's h vectors are staged in LDS; each wave takes every fourth route, loads all of
//      its rows first, then computes; the waves' partial sums meet in LDS and are
//      added in a fixed order, so every output element is written once (no atomics,
//      run-to-run identical).  The same pass writes the bf16 output when asked.
// Fill-through: when the call carries the lookup's fill list, a unit whose slot is
// being filled reads its rows from the pinned host entry instead (over the host
// link) and stores them into the slot from the registers that hold them, so the
// fill and the expert pass are one stream of loads.  gate_up records each route's
// host source in the workspace; down reads it there.
#include "mc_common.h"

namespace mc {

constexpr int kThreads = 256;
// gate_up: WR intermediate rows per wave (WR gate + WR up rows), 4 WR per workgroup;
// down: ROWS hidden rows per workgroup.  Chosen per call: single-token calls take the
// smaller gate_up tile (more workgroups for few units), batched calls the larger down
// tile (a token's h staged once for more rows).
constexpr int kB_RoutesPerWave = 3;          // down: routes a wave holds in registers at once
constexpr int kMaxRoutes = 1024;
constexpr int kMaxTok = 64;
constexpr int kB_LdsBytes = 64 * 1024;

// ---------------------------------------------------------------- chunk dots

// 16-byte weight load marked non-temporal: every weight byte of a call is used once,
// and the same form serves HBM slots and pinned host entries (fill-through).
__device__ __forceinline__ uint4 stream_load16(const uint4* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// x pairs: packed bf16 pairs of the chunk's activations.
// MXFP4 chunk: 32 elements, 16 B codes, one e8m0 scale; x: 16 dwords.
__device__ __forceinline__ float dot_chunk_mx(const uint4& w, float scale, const uint32_t* xp,
                                              float acc) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(d[q], scale), xp[4 * q + 0], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(d[q], scale), xp[4 * q + 1], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(d[q], scale), xp[4 * q + 2], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(d[q], scale), xp[4 * q + 3], acc);
  }
  return acc;
}

// bf16 chunk: 8 elements; x: 4 dwords.
__device__ __forceinline__ float dot_chunk_bf(const uint4& w, const uint32_t* xp, float acc) {
  acc = dot2_bf16(w.x, xp[0], acc);
  acc = dot2_bf16(w.y, xp[1], acc);
  acc = dot2_bf16(w.z, xp[2], acc);
  acc = dot2_bf16(w.w, xp[3], acc);
  return acc;
}

// fp32 activations (h): MXFP4 chunk of 32 weights against 32 floats.
__device__ __forceinline__ float dot_chunk_mx_f32(const uint4& w, float scale, const float* h,
                                                  float acc) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x2_t a = fp4x2_to_f32x2<0>(d[q], scale);
    f32x2_t b = fp4x2_to_f32x2<1>(d[q], scale);
    f32x2_t c = fp4x2_to_f32x2<2>(d[q], scale);
    f32x2_t e = fp4x2_to_f32x2<3>(d[q], scale);
    acc = fmaf(a.x, h[8 * q + 0], acc);
    acc = fmaf(a.y, h[8 * q + 1], acc);
    acc = fmaf(b.x, h[8 * q + 2], acc);
    acc = fmaf(b.y, h[8 * q + 3], acc);
    acc = fmaf(c.x, h[8 * q + 4], acc);
    acc = fmaf(c.y, h[8 * q + 5], acc);
    acc = fmaf(e.x, h[8 * q + 6], acc);
    acc = fmaf(e.y, h[8 * q + 7], acc);
  }
  return acc;
}

__device__ __forceinline__ float dot_chunk_bf_f32(const uint4& w, const float* h, float acc) {
  acc = fmaf(bf16_lo(w.x), h[0], acc);
  acc = fmaf(bf16_hi(w.x), h[1], acc);
  acc = fmaf(bf16_lo(w.y), h[2], acc);
  acc = fmaf(bf16_hi(w.y), h[3], acc);
  acc = fmaf(bf16_lo(w.z), h[4], acc);
  acc = fmaf(bf16_hi(w.z), h[5], acc);
  acc = fmaf(bf16_lo(w.w), h[6], acc);
  acc = fmaf(bf16_hi(w.w), h[7], acc);
  return acc;
}

struct DecodeArgs {
  const uint16_t* x;          // [T][H] bf16
  const int32_t* slots;       // [T][k]
  const float* w;             // [T][k]
  const int32_t* n_tok;
  int32_t T, k, H, I;
  int64_t n_pool;
  const uint8_t* gu;          // pool banks
  const uint8_t* gus;
  const uint8_t* dn;
  const uint8_t* dns;
  const uint8_t* sh_gu;       // shared expert entry 0 (or null)
  const uint8_t* sh_gus;
  const uint8_t* sh_dn;
  const uint8_t* sh_dns;
  float* h_route;             // [T*k][I]
  float* h_shared;            // [T][I]
  float* y;                   // [T][H]
  uint16_t* y_bf16;           // [T][H] or null
  int32_t accumulate;
  int32_t has_shared;
  // fill-through (f_gu == nullptr: off): device views of the host banks, the list
  const uint8_t* f_gu;
  const uint8_t* f_gus;
  const uint8_t* f_dn;
  const uint8_t* f_dns;
  int64_t n_host;
  const int32_t* fill_flat;
  const int32_t* fill_slot;
  const int32_t* n_fill;
  int32_t kcap;
  int32_t* rsrc;              // [T*k] host flat id a route's weights come from, -1 = slot
};

// Host entry that fills `slot` in this call, or -1 (wave-uniform; lanes search the
// list 64 entries at a time).
__device__ int64_t fill_source(const DecodeArgs& a, int slot) {
  const int lane = threadIdx.x & 63;
  const int nf = min(max(*a.n_fill, 0), a.kcap);
  for (int base = 0; base < nf; base += 64) {
    const int i = base + lane;
    const bool hit = i < nf && a.fill_slot[i] == slot;
    const uint64_t m = __ballot(hit);
    if (m) {
      const int64_t f = a.fill_flat[base + __builtin_ctzll(m)];
      return (f >= 0 && f < a.n_host) ? f : -1;
    }
  }
  return -1;
}

__device__ __forceinline__ int valid_tokens(const DecodeArgs& a) {
  return a.n_tok ? min(max(*a.n_tok, 0), a.T) : a.T;
}

__device__ __forceinline__ int pool_slot(const DecodeArgs& a, int r) {
  const int s = a.slots[r];
  return (s >= 0 && s < a.n_pool) ? s : -1;
}

// 64 routes from `base` on: lanes whose route is below `end` and holds `slot`.
__device__ __forceinline__ uint64_t routes_with_slot(const DecodeArgs& a, int base, int end, int slot) {
  const int j = base + (int)(threadIdx.x & 63);
  return __ballot(j < end && pool_slot(a, j) == slot);
}

// ---------------------------------------------------------------- gate_up kernel

template <int FMT, int CPL, int WR>
__global__ void __launch_bounds__(kThreads)
gate_up_kernel(DecodeArgs a) {
  // column u < T*k: route u's slot, when no earlier route of the call holds it (the
  // first route of a unit); column T*k: the shared expert
  // The unit's slot, the slots of its window of 64 routes and the valid count are read
  // in one round trip (every route index below T*k is readable, valid or not), so the
  // weight loads wait behind a single dependent read.
  const int u = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_all = a.T * a.k;
  const bool shared_unit = a.has_shared && u == n_all;
  const int wbase = u & ~63;
  int slot_raw = -1, win_slot = -1;
  if (!shared_unit) {
    slot_raw = a.slots[u];
    if (wbase + lane < n_all) win_slot = a.slots[wbase + lane];
  }
  const int nt = valid_tokens(a);
  const int nr = nt * a.k;
  int slot = -1;
  if (shared_unit) {
    if (nt == 0) return;
  } else {
    if (u >= nr) return;
    slot = (slot_raw >= 0 && slot_raw < a.n_pool) ? slot_raw : -1;
    if (slot < 0) return;
    if (__ballot(wbase + lane < u && win_slot == slot)) return;
    for (int base = 0; base < wbase; base += 64)
      if (routes_with_slot(a, base, u, slot)) return;
  }

  const int H = a.H, I = a.I;
  const int i0 = blockIdx.y * (4 * WR) + wave * WR;   // first intermediate row
  constexpr int ELEMS = FMT == MC_MXFP4 ? 32 : 8;             // elements per 16-B chunk
  const int n_chunks = H / ELEMS;
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)H / 2 : (size_t)H * 2;

  const uint8_t* gu;
  const uint8_t* gus = nullptr;
  uint8_t* wb_gu = nullptr;        // fill-through: the slot entry the rows are stored to
  uint8_t* wb_gus = nullptr;
  int64_t src = -1;
  if (shared_unit) {
    gu = a.sh_gu;
    gus = a.sh_gus;
  } else {
    const size_t per_gu = 2 * (size_t)I * row_bytes, per_gus = (size_t)2 * I * H / 32;
    gu = a.gu + (size_t)slot * per_gu;
    if (FMT == MC_MXFP4) gus = a.gus + (size_t)slot * per_gus;
    if (a.f_gu) src = fill_source(a, slot);
    if (src >= 0) {
      wb_gu = const_cast<uint8_t*>(gu);
      wb_gus = const_cast<uint8_t*>(gus);
      gu = a.f_gu + (size_t)src * per_gu;
      if (FMT == MC_MXFP4) gus = a.f_gus + (size_t)src * per_gus;
    }
  }

  // all loads of the wave's 8 rows first (chunk index clamped; out-of-row lanes are
  // zeroed after the loads), scale bytes kept raw until every load is issued
  int cq[CPL];
  bool okq[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + 64 * q;
    okq[q] = c < n_chunks;
    cq[q] = okq[q] ? c : n_chunks - 1;
  }
  uint4 wv[2 * WR][CPL];
  uint32_t sb[2 * WR][CPL];
#pragma unroll
  for (int r = 0; r < 2 * WR; ++r) {
    const int row = r < WR ? i0 + r : I + i0 + (r - WR);
    const uint4* rp = reinterpret_cast<const uint4*>(gu + (size_t)row * row_bytes);
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      wv[r][q] = stream_load16(rp + cq[q]);
      if (FMT == MC_MXFP4) sb[r][q] = gus[(size_t)row * (H / 32) + cq[q]];
    }
  }

  // the unit's routes in route order: a mask per 64 routes, the next one fetched when
  // this one runs out (the shared expert takes every valid token in turn)
  int base = wbase, t_next = 0;
  uint64_t unit_routes =
      shared_unit ? 0 : __ballot(wbase + lane >= u && wbase + lane < nr && win_slot == slot);
  while (true) {
    int t, route;
    if (shared_unit) {
      if (t_next >= nt) break;
      t = t_next++;
      route = -1;
    } else {
      while (!unit_routes && base + 64 < nr) {
        base += 64;
        unit_routes = routes_with_slot(a, base, nr, slot);
      }
      if (!unit_routes) break;
      route = base + __builtin_ctzll(unit_routes);
      unit_routes &= unit_routes - 1;
      t = route / a.k;
      if (blockIdx.y == 0 && threadIdx.x == 0) a.rsrc[route] = (int32_t)src;
    }
    const uint32_t* xrow = reinterpret_cast<const uint32_t*>(a.x + (size_t)t * H);
    uint32_t xp[CPL][ELEMS / 2];
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const uint4* xs = reinterpret_cast<const uint4*>(xrow + (size_t)cq[q] * (ELEMS / 2));
#pragma unroll
      for (int v = 0; v < ELEMS / 8; ++v) {
        const uint4 xx = xs[v];
        xp[q][4 * v + 0] = xx.x;
        xp[q][4 * v + 1] = xx.y;
        xp[q][4 * v + 2] = xx.z;
        xp[q][4 * v + 3] = xx.w;
      }
    }
    float acc[2 * WR];
#pragma unroll
    for (int r = 0; r < 2 * WR; ++r) {
      acc[r] = 0.0f;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const uint4 wq = okq[q] ? wv[r][q] : make_uint4(0, 0, 0, 0);
        if (FMT == MC_MXFP4)
          acc[r] = dot_chunk_mx(wq, e8m0_to_f32(sb[r][q]), xp[q], acc[r]);
        else
          acc[r] = dot_chunk_bf(wq, xp[q], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 2 * WR; ++r) acc[r] = wave_sum(acc[r]);
    if (lane < WR) {
      float g = acc[0], up = acc[WR];
#pragma unroll
      for (int r = 1; r < WR; ++r)
        if (lane == r) {
          g = acc[r];
          up = acc[WR + r];
        }
      float* dst = shared_unit ? a.h_shared + (size_t)t * I : a.h_route + (size_t)route * I;
      dst[i0 + lane] = silu(g) * up;
    }
  }
  // fill-through: the rows this wave read from the host go into the slot
  if (wb_gu) {
#pragma unroll
    for (int r = 0; r < 2 * WR; ++r) {
      const int row = r < WR ? i0 + r : I + i0 + (r - WR);
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        if (!okq[q]) continue;
        reinterpret_cast<uint4*>(wb_gu + (size_t)row * row_bytes)[cq[q]] = wv[r][q];
        if (FMT == MC_MXFP4) wb_gus[(size_t)row * (H / 32) + cq[q]] = (uint8_t)sb[r][q];
      }
    }
  }
}

// ---------------------------------------------------------------- down kernel

template <int FMT, int LPR, int CPLB, int ROWS>
__global__ void __launch_bounds__(kThreads)
down_kernel(DecodeArgs a) {
  extern __shared__ float s_h[];                 // [k + 1][I]: one token's route vectors (swizzled)
  __shared__ float s_part[4][ROWS];
  const int t = blockIdx.y;
  const int H = a.H, I = a.I, k = a.k;
  const int r0 = blockIdx.x * ROWS;
  // The valid count, the accumulated y and the token's h vectors are read before the
  // first wait; the wave's slots and gates and then its weight rows follow once the token
  // is known to be valid (with no count given, at once), so the rows wait behind one
  // dependent read.
  const int n_raw = a.n_tok ? *a.n_tok : a.T;
  float y_old = 0.0f;                            // the value accumulated into
  if (a.accumulate && threadIdx.x < ROWS && r0 + (int)threadIdx.x < H)
    y_old = a.y[(size_t)t * H + r0 + threadIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int ELEMS = FMT == MC_MXFP4 ? 32 : 8;
  constexpr int E4 = ELEMS / 4;                              // float4 of h per chunk
  constexpr int RPP = 64 / LPR;                              // rows per pass of a wave
  constexpr int PASSES = ROWS >= RPP ? ROWS / RPP : 1;
  const int n_chunks = I / ELEMS;
  const int row_sub = lane / LPR, c_lane = lane % LPR;
  const bool lane_rows = RPP <= ROWS || row_sub < ROWS;
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)I / 2 : (size_t)I * 2;
  const size_t per = (size_t)H * row_bytes;
  const size_t per_s = (size_t)H * I / 32;
  const int nvec = k + a.has_shared;                         // routes (+ shared) of a token

  int cq[CPLB];
  bool okq[CPLB];
#pragma unroll
  for (int q = 0; q < CPLB; ++q) {
    const int c = c_lane + LPR * q;
    okq[q] = c < n_chunks && lane_rows;
    cq[q] = c < n_chunks ? c : n_chunks - 1;
  }
  int rowp[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) rowp[p] = min(r0 + row_sub + RPP * p, H - 1);

  constexpr int kGroup = 4 * kB_RoutesPerWave;             // routes covered by one round
  const int n_groups = (nvec + kGroup - 1) / kGroup;

  uint4 wv[kB_RoutesPerWave][PASSES][CPLB];
  uint32_t sb[kB_RoutesPerWave][PASSES][CPLB];
  float gate[kB_RoutesPerWave];
  uint8_t* wb[kB_RoutesPerWave];           // fill-through: slot entry to store the rows to
  uint8_t* wbs[kB_RoutesPerWave];
  // the wave's routes v0, v0+4, v0+8: gates and all row loads
  auto load_group = [&](int v0) {
    // the routes' slots, gates and host sources first, all in flight together (route
    // index clamped into the token's routes), then the rows that depend on them
    int s_raw[kB_RoutesPerWave], src_raw[kB_RoutesPerWave];
    float g_raw[kB_RoutesPerWave];
    if (k > 0) {
#pragma unroll
      for (int j = 0; j < kB_RoutesPerWave; ++j) {
        const int r = t * k + min(v0 + 4 * j, k - 1);
        s_raw[j] = a.slots[r];
        g_raw[j] = a.w[r];
        src_raw[j] = a.f_dn ? a.rsrc[r] : -1;
      }
    }
#pragma unroll
    for (int j = 0; j < kB_RoutesPerWave; ++j) {
      const int v = v0 + 4 * j;
      const uint8_t* dn = a.dn;            // any readable address when there is nothing to read
      const uint8_t* dns = a.dns;
      gate[j] = 0.0f;
      wb[j] = nullptr;
      wbs[j] = nullptr;
      if (v < k) {
        const int s = (s_raw[j] >= 0 && s_raw[j] < a.n_pool) ? s_raw[j] : -1;
        if (s >= 0) {
          dn = a.dn + (size_t)s * per;
          if (FMT == MC_MXFP4) dns = a.dns + (size_t)s * per_s;
          gate[j] = g_raw[j];
          const int src = src_raw[j] < a.n_host ? src_raw[j] : -1;
          if (src >= 0) {
            wb[j] = const_cast<uint8_t*>(dn);
            wbs[j] = const_cast<uint8_t*>(dns);
            dn = a.f_dn + (size_t)src * per;
            if (FMT == MC_MXFP4) dns = a.f_dns + (size_t)src * per_s;
          }
        }
      } else if (v == k && a.has_shared) {
        dn = a.sh_dn;
        dns = a.sh_dns;
        gate[j] = 1.0f;
      }
#pragma unroll
      for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int q = 0; q < CPLB; ++q) {
          wv[j][p][q] = stream_load16(reinterpret_cast<const uint4*>(dn + (size_t)rowp[p] * row_bytes) + cq[q]);
          if (FMT == MC_MXFP4) sb[j][p][q] = dns[(size_t)rowp[p] * (I / 32) + cq[q]];
        }
    }
  };

  {
    // h of this token straight into LDS (global_load_lds, 1 KiB per wave instruction),
    // then the first route group's rows: both sets of loads are in flight together.
    // Float4 e of chunk c sits at LDS float4 c * E4 + (e ^ (c & (E4 - 1))): the lanes
    // of a row, which read the same e of consecutive chunks, hit different banks, and
    // each chunk still comes from one contiguous piece of global memory.
    const int n4 = nvec * I / 4, r4 = I / 4;
    for (int ch = wave; ch * 64 < n4; ch += 4) {
      int i4 = ch * 64 + lane;
      if (i4 >= n4) i4 = n4 - 1;                       // tail lanes re-read a valid vector
      const int v = i4 / r4, sl = i4 % r4, c = sl / E4;
      const int e = (c * E4 + ((sl % E4) ^ (c & (E4 - 1)))) * 4;
      const float* src = v < k ? a.h_route + ((size_t)t * k + v) * I : a.h_shared + (size_t)t * I;
      __builtin_amdgcn_global_load_lds(src + e, (__attribute__((address_space(3))) void*)(s_h + ch * 256),
                                       16, 0, 0);
    }
    const int nt = min(max(n_raw, 0), a.T);
    if (t >= nt) {                                     // a token beyond the valid count: its rows
      __builtin_amdgcn_s_waitcnt(0);
      if (threadIdx.x < ROWS && r0 + (int)threadIdx.x < H) {
        const size_t o = (size_t)t * H + r0 + threadIdx.x;
        if (!a.accumulate) a.y[o] = 0.0f;
        if (a.y_bf16) a.y_bf16[o] = 0;
      }
      return;
    }
    if (n_groups > 0) load_group(wave);
    __builtin_amdgcn_s_waitcnt(0);                     // the LDS copies have landed
    __syncthreads();

    float acc[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) acc[p] = 0.0f;
    for (int g = 0; g < n_groups; ++g) {
      const int v0 = wave + g * kGroup;
      if (g > 0) load_group(v0);
#pragma unroll
      for (int j = 0; j < kB_RoutesPerWave; ++j) {
        const int v = v0 + 4 * j;
        if (v >= nvec || gate[j] == 0.0f) continue;
#pragma unroll
        for (int q = 0; q < CPLB; ++q) {
          float hv[ELEMS];
          const float4* hs = reinterpret_cast<const float4*>(s_h + (size_t)v * I) + cq[q] * E4;
          const int sw = cq[q] & (E4 - 1);
#pragma unroll
          for (int e = 0; e < E4; ++e) {
            const float4 f = hs[e ^ sw];
            hv[4 * e + 0] = f.x;
            hv[4 * e + 1] = f.y;
            hv[4 * e + 2] = f.z;
            hv[4 * e + 3] = f.w;
          }
#pragma unroll
          for (int p = 0; p < PASSES; ++p) {
            const uint4 wq = okq[q] ? wv[j][p][q] : make_uint4(0, 0, 0, 0);
            const float part = FMT == MC_MXFP4
                                   ? dot_chunk_mx_f32(wq, e8m0_to_f32(sb[j][p][q]), hv, 0.0f)
                                   : dot_chunk_bf_f32(wq, hv, 0.0f);
            acc[p] = fmaf(gate[j], part, acc[p]);
          }
        }
      }
      // fill-through: rows read from the host go into the slot (rows of this block)
#pragma unroll
      for (int j = 0; j < kB_RoutesPerWave; ++j) {
        if (!wb[j]) continue;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          const int rl = row_sub + RPP * p, row = r0 + rl;
          if (rl >= ROWS || row >= H) continue;
#pragma unroll
          for (int q = 0; q < CPLB; ++q) {
            if (!okq[q]) continue;
            reinterpret_cast<uint4*>(wb[j] + (size_t)row * row_bytes)[cq[q]] = wv[j][p][q];
            if (FMT == MC_MXFP4) wbs[j][(size_t)row * (I / 32) + cq[q]] = (uint8_t)sb[j][p][q];
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float sum = group_sum(acc[p], LPR);
      const int rl = row_sub + RPP * p;
      if (c_lane == 0 && lane_rows && rl < ROWS) s_part[wave][rl] = sum;
    }
    __syncthreads();
    if (threadIdx.x < ROWS) {
      const int row = r0 + threadIdx.x;
      float v = ((s_part[0][threadIdx.x] + s_part[1][threadIdx.x]) + s_part[2][threadIdx.x]) +
                s_part[3][threadIdx.x];
      float* yp = a.y + (size_t)t * H + row;
      if (a.accumulate) v += y_old;
      *yp = v;
      if (a.y_bf16) a.y_bf16[(size_t)t * H + row] = f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------- dispatch

template <int FMT, int WR>
static void launch_gate_up_w(const DecodeArgs& a, int cpl, dim3 grid, hipStream_t s) {
  switch (cpl) {
    case 1: hipLaunchKernelGGL((gate_up_kernel<FMT, 1, WR>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gate_up_kernel<FMT, 2, WR>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((gate_up_kernel<FMT, 4, WR>), grid, dim3(kThreads), 0, s, a); break;
  }
}

template <int FMT>
static void launch_gate_up(const DecodeArgs& a, int cpl, int wr, dim3 grid, hipStream_t s) {
  if (wr == 2) launch_gate_up_w<FMT, 2>(a, cpl, grid, s);
  else launch_gate_up_w<FMT, 4>(a, cpl, grid, s);
}

template <int FMT, int LPR, int ROWS>
static void launch_down_l(const DecodeArgs& a, int cplb, dim3 grid, size_t lds, hipStream_t s) {
  if (cplb == 1)
    hipLaunchKernelGGL((down_kernel<FMT, LPR, 1, ROWS>), grid, dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL((down_kernel<FMT, LPR, 2, ROWS>), grid, dim3(kThreads), lds, s, a);
}

// rows = 16 only with lpr 4 or 16 (the 64-lane row form keeps 8)
template <int FMT>
static void launch_down(const DecodeArgs& a, int lpr, int cplb, int rows, dim3 grid, size_t lds,
                        hipStream_t s) {
  switch (lpr) {
    case 4:
      if (rows == 16) launch_down_l<FMT, 4, 16>(a, cplb, grid, lds, s);
      else launch_down_l<FMT, 4, 8>(a, cplb, grid, lds, s);
      break;
    case 16:
      if (rows == 16) launch_down_l<FMT, 16, 16>(a, cplb, grid, lds, s);
      else launch_down_l<FMT, 16, 8>(a, cplb, grid, lds, s);
      break;
    default: launch_down_l<FMT, 64, 8>(a, cplb, grid, lds, s); break;
  }
}

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace mc

using namespace mc;

// workspace: h of every route [T*k][I] and of the shared expert [T][I] (fp32), then
// the routes' fill-through sources [T*k] (int32)
static size_t ws_h_bytes(int32_t T, int32_t k, int32_t I) {
  return ((size_t)T * k + (size_t)T) * (size_t)I * sizeof(float);
}

extern "C" size_t moe_experts_decode_ws_bytes(int32_t T, int32_t k, int32_t I) {
  if (T < 0 || k < 0 || I < 0) return 0;
  return ws_h_bytes(T, k, I) + (size_t)T * k * sizeof(int32_t);
}

extern "C" int moe_experts_decode(const void* x_bf16, const int32_t* slots, const float* w,
                                  int32_t T, int32_t k, const int32_t* n_tok,
                                  const mc_banks* pool, const mc_banks* shared, void* ws,
                                  size_t ws_bytes, float* y_acc, int32_t accumulate, void* y_bf16,
                                  hipStream_t s, const mc_fill_list* fill) {
  clear_error();
  int rc;
  if ((rc = check_banks(pool, "moe_experts_decode pool")) != MC_OK) return rc;
  if (shared) {
    if ((rc = check_banks(shared, "moe_experts_decode shared")) != MC_OK) return rc;
    MC_REQUIRE(shared->fmt == pool->fmt && shared->H == pool->H && shared->I == pool->I,
               "moe_experts_decode: shared expert differs from the pool in format or shape");
  }
  MC_REQUIRE(T >= 0 && k >= 1, "moe_experts_decode: T=%d k=%d", T, k);
  MC_REQUIRE(T <= kMaxTok, "moe_experts_decode: T=%d exceeds %d", T, kMaxTok);
  MC_REQUIRE((int64_t)T * k <= kMaxRoutes, "moe_experts_decode: T*k=%lld exceeds %d",
             (long long)T * k, kMaxRoutes);
  MC_REQUIRE(accumulate == 0 || accumulate == 1, "moe_experts_decode: accumulate=%d", accumulate);
  if (T == 0) return MC_OK;
  MC_REQUIRE(x_bf16 && slots && w && y_acc && ws, "moe_experts_decode: NULL pointer");
  MC_REQUIRE(ws_bytes >= moe_experts_decode_ws_bytes(T, k, pool->I),
             "moe_experts_decode: workspace %zu < %zu bytes", ws_bytes,
             moe_experts_decode_ws_bytes(T, k, pool->I));
  MC_REQUIRE((uintptr_t)x_bf16 % 16 == 0 && (uintptr_t)ws % 16 == 0,
             "moe_experts_decode: x and ws must be 16-byte aligned");
  const int H = pool->H, I = pool->I, fmt = pool->fmt;
  const int elems = fmt == MC_MXFP4 ? 32 : 8;
  const int cpl = pow2_at_least((H / elems + 63) / 64);
  if (cpl > 4) {
    set_error("moe_experts_decode: H=%d too large", H);
    return MC_EUNSUPPORTED;
  }
  const int chunks_b = I / elems;
  const int lpr = chunks_b <= 4 ? 4 : (chunks_b <= 16 ? 16 : 64);
  const int cplb = pow2_at_least((chunks_b + lpr - 1) / lpr);
  if (cplb > 2) {
    set_error("moe_experts_decode: I=%d too large", I);
    return MC_EUNSUPPORTED;
  }
  const int has_shared = shared ? 1 : 0;
  const size_t lds = ((size_t)(k + has_shared) * I * sizeof(float) + 1023) & ~(size_t)1023;
  if (lds > (size_t)kB_LdsBytes) {
    set_error("moe_experts_decode: (k+1)*I*4 = %zu bytes of staged activations exceed %d", lds,
              kB_LdsBytes);
    return MC_EUNSUPPORTED;
  }

  DecodeArgs a{};
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.slots = slots;
  a.w = w;
  a.n_tok = n_tok;
  a.T = T;
  a.k = k;
  a.H = H;
  a.I = I;
  a.n_pool = pool->n;
  a.gu = static_cast<const uint8_t*>(pool->gate_up);
  a.gus = static_cast<const uint8_t*>(pool->gate_up_scale);
  a.dn = static_cast<const uint8_t*>(pool->down);
  a.dns = static_cast<const uint8_t*>(pool->down_scale);
  if (shared) {
    a.sh_gu = static_cast<const uint8_t*>(shared->gate_up);
    a.sh_gus = static_cast<const uint8_t*>(shared->gate_up_scale);
    a.sh_dn = static_cast<const uint8_t*>(shared->down);
    a.sh_dns = static_cast<const uint8_t*>(shared->down_scale);
  }
  a.h_route = static_cast<float*>(ws);
  a.h_shared = a.h_route + (size_t)T * k * I;
  a.y = y_acc;
  a.y_bf16 = static_cast<uint16_t*>(y_bf16);
  a.accumulate = accumulate;
  a.has_shared = has_shared;
  a.rsrc = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + ws_h_bytes(T, k, I));
  if (fill) {
    if ((rc = check_banks(fill->host, "moe_experts_decode fill host")) != MC_OK) return rc;
    MC_REQUIRE(fill->host->fmt == fmt && fill->host->H == H && fill->host->I == I,
               "moe_experts_decode: fill host banks differ from the pool in format or shape");
    MC_REQUIRE(fill->kcap >= 0 && fill->fill_flat && fill->fill_slot && fill->n_fill,
               "moe_experts_decode: bad fill list");
    if ((rc = host_device_view(fill->host->gate_up, &a.f_gu, "moe_experts_decode: fill host bank", s)) ||
        (rc = host_device_view(fill->host->gate_up_scale, &a.f_gus, "moe_experts_decode: fill host bank", s)) ||
        (rc = host_device_view(fill->host->down, &a.f_dn, "moe_experts_decode: fill host bank", s)) ||
        (rc = host_device_view(fill->host->down_scale, &a.f_dns, "moe_experts_decode: fill host bank", s)))
      return rc;
    a.n_host = fill->host->n;
    a.fill_flat = fill->fill_flat;
    a.fill_slot = fill->fill_slot;
    a.n_fill = fill->n_fill;
    a.kcap = fill->kcap;
    MC_REQUIRE(fill->gate_up_only == 0 || fill->gate_up_only == 1,
               "moe_experts_decode: fill gate_up_only=%d", fill->gate_up_only);
    if (fill->gate_up_only) a.f_dn = a.f_dns = nullptr;   // down reads the slots
    if (a.kcap == 0) a.f_gu = a.f_dn = nullptr;
  }

  const int wr = T == 1 ? 2 : 4;
  const int rows = (T >= 4 && lpr != 64) ? 16 : 8;
  dim3 grid_a(T * k + has_shared, I / (4 * wr));
  if (fmt == MC_MXFP4)
    launch_gate_up<MC_MXFP4>(a, cpl, wr, grid_a, s);
  else
    launch_gate_up<MC_BF16>(a, cpl, wr, grid_a, s);
  MC_LAUNCH_CHECK();
  if (fill && fill->down_after) MC_HIP(hipStreamWaitEvent(s, fill->down_after, 0));
  dim3 grid_b((H + rows - 1) / rows, T);
  if (fmt == MC_MXFP4)
    launch_down<MC_MXFP4>(a, lpr, cplb, rows, grid_b, lds, s);
  else
    launch_down<MC_BF16>(a, lpr, cplb, rows, grid_b, lds, s);
  MC_LAUNCH_CHECK();
  return MC_OK;
}
