// moe_experts_decode: slot-indirected SwiGLU experts + gated combine for decode.
//
// [jjl357] "1.1": h_t = sum_e p_{t,e} Expert_{l,e}(x_t).  [jjl357] "6.1": an expert
// routed by several tokens of the call is read and run once.  [jjl357] "6.7" step 5
// and [wanger] "代码全链路": the GPU runs hits + fills; host-computed routes arrive
// with slot -1 (or gate 0) and are skipped.
//
// Decode streams ~0.53 B of MXFP4 weight per multiply-add, so it is bound by HBM
// bandwidth, and every weight must be dequantised exactly once whatever the batch.
// One token (the common decode call):
//   gate_up: workgroup = (route, 8 intermediate rows); each wave owns 2 gate rows and
//      the 2 matching up rows and reads each row whole with 16-B loads (bf16 dot2
//      against the bf16 activation), so a wave's loads are contiguous row runs; the
//      fp32 h = silu(g) * u goes to the workspace.
//   down: workgroup = a block of hidden rows over every route of the token, the
//      token's h vectors copied into LDS by DMA.  Rows of 64 lanes (I >= 2048 MXFP4):
//      each wave owns its own rows over all routes (even work whatever the route
//      count) and its row loads go out right behind the h copies, so it computes the
//      first routes while the later routes' rows still stream in.  Shorter rows: the
//      waves split the routes and meet in LDS.  Each output row is one fixed-order sum.
// Several tokens: both passes run on the matrix cores.  The expert's weight rows are
// the MFMA's N side (16 rows per tile, MXFP4 -> bf16 dequantised exactly), the tokens
// its M side, and K runs in steps of 128 in which each lane owns one whole 32-element
// MX block (16 B of codes + 1 scale byte) of its row; the activation operand is read in
// the same permuted K order.  A unit is one distinct slot of the call (run by the grid
// column of the first route that holds it) or the shared expert.
//   gate_up: workgroup = (unit, 16 intermediate rows); the four waves split H, each
//      loading its gate and up fragments for all of its K steps at once, and the four
//      products meet in LDS in a fixed order.  The unit's tokens, 16 at a time, are the
//      MFMA rows.  h = silu(g) * u is stored as two bf16 halves (hi = bf16(h), lo =
//      bf16(h - hi): 16 significant bits, the fp32 value to within 2^-17).
//   down: workgroup = (unit, 64 hidden rows); each wave owns a 16-row tile over all
//      of I, loaded once; the unit's routes (hi and lo rows, 8 routes per product) are
//      staged in LDS a batch at a time.  Each route's gated partial is stored, and the
//      last workgroup of a row block to arrive (one arrival counter per row block) adds
//      the partials of every token in route order (j = 0 .. k-1, then the shared
//      expert), so each output element is one fixed-order sum (no float atomics,
//      run-to-run identical).
// Fill-through: when the call carries the lookup's fill list, a unit whose slot is
// being filled reads its fragments from the pinned host entry instead (over the host
// link) and stores them into the slot from the registers that hold them, so the fill
// and the expert pass are one stream of loads.
#include <algorithm>
#include <mutex>

#include "fill_dev.h"

namespace mc {

constexpr int kThreads = 256;
static_assert(kThreads == kFillThreads, "the fused copy workgroups run the fill's chunk loop");
constexpr int kMaxRoutes = 1024;
constexpr int kMaxTok = 64;
constexpr int kKS = 128;                     // K elements per step (4 MFMAs of 32)
constexpr int kHLdsBytes = 16 * 1024;        // down (several tokens): LDS for a batch of h
constexpr int kRouteTile = 8;                // routes per down product (hi + lo rows)
constexpr int kUnitRows = 64;                // down (several tokens): rows per workgroup
constexpr int kCntStride = 16;               // uint32 words between arrival counters (64 B)
constexpr int kTok1LdsBytes = 64 * 1024;    // down (one token): LDS for all of the token's h

// 16-byte weight load marked non-temporal: every weight byte of a call is used once,
// and the same form serves HBM slots and pinned host entries (fill-through).
__device__ __forceinline__ u32x4_t stream_load16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
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
  // vector v: route v (v < T*k) or the shared expert of token v - T*k
  float* h32;                 // [T*k + T][I] fp32 h (one-token path)
  uint16_t* h_hi;             // [T*k + T][I] bf16(h)
  uint16_t* h_lo;             // [T*k + T][I] bf16(h - hi)
  float* part;                // [T*k + T][H] gated partial outputs (several-token down)
  int32_t* rsrc;              // [T*k] host entry a route's unit reads (fill-through), -1 = slot
  uint32_t* cnt;              // [n_cnt * kCntStride] arrival counters of the down row blocks
  int32_t n_cnt;
  int32_t tb;                 // several-token down: routes per LDS batch
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
};

// ---------------------------------------------------------------- units

// Store visible to the other XCDs once this wave's stores have completed (coherent
// write, no L2 write-back needed); read of such a value.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Host entry that fills `slot` in this call, or -1 (wave-uniform; lanes search the
// list 64 entries at a time).  The count and the first 64 entries are read in one round
// trip (entries below kcap are always readable).
__device__ int64_t fill_source(const DecodeArgs& a, int slot) {
  const int lane = threadIdx.x & 63;
  const int nf_raw = *a.n_fill;
  int fs = -1, ff = -1;
  if (lane < a.kcap) {
    fs = a.fill_slot[lane];
    ff = a.fill_flat[lane];
  }
  const int nf = min(max(nf_raw, 0), a.kcap);
  for (int base = 0; base < nf; base += 64) {
    const int i = base + lane;
    if (base > 0 && i < nf) {
      fs = a.fill_slot[i];
      ff = a.fill_flat[i];
    }
    const uint64_t m = __ballot(i < nf && fs == slot);
    if (m) {
      const int64_t f = __builtin_amdgcn_readlane(ff, __builtin_ctzll(m));
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

// Whether grid column u runs a unit, and its slot.  Column u < T*k runs route u's slot
// when no earlier route of the call holds it; column T*k is the shared expert (runs
// when any token is valid).  The column's slot, the slots of its window of 64 routes
// and the valid count are read in one round trip (every route index below T*k is
// readable, valid or not), so the weight loads wait behind a single dependent read.
// Wave-uniform; every wave of the workgroup gets the same answer.
__device__ __forceinline__ bool column_unit(const DecodeArgs& a, int u, int& slot, int& win_slot,
                                            int& nt, int& nr) {
  const int lane = threadIdx.x & 63;
  const int n_all = a.T * a.k;
  const bool shared_unit = a.has_shared && u == n_all;
  const int wbase = u & ~63;
  int slot_raw = -1;
  win_slot = -1;
  if (!shared_unit) {
    slot_raw = a.slots[u];
    if (wbase + lane < n_all) win_slot = a.slots[wbase + lane];
  }
  nt = valid_tokens(a);
  nr = nt * a.k;
  slot = -1;
  if (shared_unit) return nt > 0;
  if (u >= nr) return false;
  slot = (slot_raw >= 0 && slot_raw < a.n_pool) ? slot_raw : -1;
  if (slot < 0) return false;
  if (__ballot(wbase + lane < u && win_slot == slot)) return false;
  for (int base = 0; base < wbase; base += 64)
    if (routes_with_slot(a, base, u, slot)) return false;
  return true;
}

// The unit's vectors in route order into LDS (the shared expert: every valid token);
// run by one wave, returns the count on every lane of it.
__device__ __forceinline__ int unit_vectors(const DecodeArgs& a, int u, int slot, int win_slot, int nt,
                                            int nr, int32_t* s_vec) {
  const int lane = threadIdx.x & 63;
  const int n_all = a.T * a.k;
  if (a.has_shared && u == n_all) {
    for (int t = lane; t < nt; t += 64) s_vec[t] = n_all + t;
    return nt;
  }
  int n = 0, base = u & ~63;
  uint64_t m = __ballot(base + lane >= u && base + lane < nr && win_slot == slot);
  while (true) {
    while (!m && base + 64 < nr) {
      base += 64;
      m = routes_with_slot(a, base, nr, slot);
    }
    if (!m) break;
    if ((m >> lane) & 1)
      s_vec[n + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0))] =
          base + lane;
    n += __builtin_popcountll(m);
    m = 0;
  }
  return n;
}

// ---------------------------------------------------------------- MFMA fragments
//
// Weight fragment of one 16-row tile and one K step: lane l owns row (l & 15) and the
// 32-element block 4 * step + (l >> 4) of it: 16 B of MXFP4 codes + its scale byte, or
// 64 B of bf16.  The four MFMAs of the step consume elements 8 ks .. 8 ks + 7 of every
// lane's block (ks = 0..3), so the activation operand of lane l holds, for its token
// row (l & 15), elements 128 step + 32 (l >> 4) + 8 ks .. + 7.

template <int FMT>
struct WFrag {
  u32x4_t v[FMT == MC_MXFP4 ? 1 : 4];
  uint32_t s;
};

template <int FMT>
__device__ __forceinline__ void wfrag_load(WFrag<FMT>& f, const uint8_t* row, const uint8_t* srow, int blk,
                                           bool ok) {
  const int b = ok ? blk : 0;
  if (FMT == MC_MXFP4) {
    f.v[0] = stream_load16(row + (size_t)b * 16);
    f.s = srow[b];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) f.v[q] = stream_load16(row + (size_t)b * 64 + q * 16);
    f.s = 0;
  }
}

template <int FMT>
__device__ __forceinline__ void wfrag_store(const WFrag<FMT>& f, uint8_t* row, uint8_t* srow, int blk) {
  if (FMT == MC_MXFP4) {
    *reinterpret_cast<u32x4_t*>(row + (size_t)blk * 16) = f.v[0];
    srow[blk] = (uint8_t)f.s;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4_t*>(row + (size_t)blk * 64 + q * 16) = f.v[q];
  }
}

// MXFP4 codes loaded four consecutive lanes per row (lane l: row (l >> 2) & 15 of the tile,
// 16-byte chunk l & 3 of the row's 64-byte run of four blocks), which the vector memory path
// serves faster than the operand layout, and moved into the operand layout (lane l: row
// l & 15, chunk l >> 4) with four cross-lane reads once the data is in.  The scale byte is
// loaded in the operand layout directly.  bf16 fragments load in the operand layout.
template <int FMT>
__device__ __forceinline__ void wfrag_load_rows(WFrag<FMT>& f, const uint8_t* base, size_t row_bytes, int row0,
                                                int row_last, const uint8_t* srow, int blk0, int n_blk) {
  const int lane = threadIdx.x & 63;
  if (FMT == MC_MXFP4) {
    const int bl = blk0 + (lane & 3), b = blk0 + (lane >> 4);
    const int r = min(row0 + ((lane >> 2) & 15), row_last);
    f.v[0] = stream_load16(base + (size_t)r * row_bytes + (size_t)(bl < n_blk ? bl : 0) * 16);
    f.s = srow[b < n_blk ? b : 0];
  } else {
    const int b = blk0 + (lane >> 4);
    wfrag_load<FMT>(f, base + (size_t)min(row0 + (lane & 15), row_last) * row_bytes, srow, b, b < n_blk);
  }
}

template <int FMT>
__device__ __forceinline__ void wfrag_to_operand(WFrag<FMT>& f) {
  if (FMT == MC_MXFP4) {
    const int lane = threadIdx.x & 63;
    const int src = (4 * (lane & 15) + (lane >> 4)) << 2;
#pragma unroll
    for (int d = 0; d < 4; ++d) f.v[0][d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f.v[0][d]);
  }
}

// B operand of MFMA ks (an invalid block contributes zeros)
template <int FMT>
__device__ __forceinline__ bf16x8_t wfrag_op(const WFrag<FMT>& f, int ks, bool ok) {
  if (!ok) return bf16x8_t{};
  if (FMT == MC_MXFP4) return fp4x8_bf16(f.v[0][ks], e8m0_to_f32(f.s));
  return __builtin_bit_cast(bf16x8_t, f.v[ks]);
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ---------------------------------------------------------------- gate_up kernel

// Four waves per SIMD for MXFP4 rows of up to four K steps per wave (the compiler then keeps
// the kernel within 128 registers, against 140 on its own); longer rows and bf16 weights keep
// the registers they need.
template <int FMT, int SPW>   // SPW: K steps per wave
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(FMT == MC_MXFP4 && SPW <= 4 ? 4 : 1)))
gate_up_kernel(DecodeArgs a) {
  __shared__ f32x4_t s_red[4][2][64];            // per-wave gate / up products
  __shared__ int32_t s_vec[kMaxRoutes];
  __shared__ int32_t s_n;
  // the several-token down pass's arrival counters start at zero in every call
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.n_cnt; i += kThreads) a.cnt[i * kCntStride] = 0u;
  const int u = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I, n_all = a.T * a.k;
  const bool shared_unit = a.has_shared && u == n_all;
  int slot, win_slot, nt, nr;
  if (!column_unit(a, u, slot, win_slot, nt, nr)) return;

  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)H / 2 : (size_t)H * 2;
  const size_t per_gu = 2 * (size_t)I * row_bytes, per_gus = (size_t)2 * I * H / 32;
  const uint8_t* gu;
  const uint8_t* gus = nullptr;
  uint8_t* wb = nullptr;                         // fill-through: slot entry the fragments go to
  uint8_t* wbs = nullptr;
  int64_t src = -1;
  if (shared_unit) {
    gu = a.sh_gu;
    gus = a.sh_gus;
  } else {
    gu = a.gu + (size_t)slot * per_gu;
    if (FMT == MC_MXFP4) gus = a.gus + (size_t)slot * per_gus;
    if (a.f_gu) src = fill_source(a, slot);
    if (src >= 0) {
      wb = const_cast<uint8_t*>(gu);
      wbs = const_cast<uint8_t*>(gus);
      gu = a.f_gu + (size_t)src * per_gu;
      if (FMT == MC_MXFP4) gus = a.f_gus + (size_t)src * per_gus;
    }
  }
  const int i0 = blockIdx.x * 16;                // first intermediate row of the tile
  const int rl = lane & 15, g4 = lane >> 4;
  const int n_blk = H / 32;
  const uint8_t* gsrow = FMT == MC_MXFP4 ? gus + (size_t)(i0 + rl) * (H / 32) : nullptr;
  const uint8_t* usrow = FMT == MC_MXFP4 ? gus + (size_t)(I + i0 + rl) * (H / 32) : nullptr;

  // every weight load of the wave first
  WFrag<FMT> fg[SPW], fu[SPW];
  bool okb[SPW];
  int blk[SPW];
#pragma unroll
  for (int q = 0; q < SPW; ++q) {
    blk[q] = 4 * (wave * SPW + q) + g4;
    okb[q] = blk[q] < n_blk;
    wfrag_load_rows<FMT>(fg[q], gu, row_bytes, i0, i0 + 15, gsrow, 4 * (wave * SPW + q), n_blk);
    wfrag_load_rows<FMT>(fu[q], gu, row_bytes, I + i0, I + i0 + 15, usrow, 4 * (wave * SPW + q), n_blk);
  }
  if (wave == 0) {
    const int n = unit_vectors(a, u, slot, win_slot, nt, nr, s_vec);
    if (lane == 0) s_n = n;
  }
  __syncthreads();
  const int n_vec = s_n;
  if (!shared_unit && blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_vec; i += kThreads) a.rsrc[s_vec[i]] = (int32_t)src;

  for (int b0 = 0; b0 < n_vec; b0 += 16) {
    const int nb = min(16, n_vec - b0);
    // activation rows: the token of vector b0 + rl
    const bool row_ok = rl < nb;
    const int vec = row_ok ? s_vec[b0 + rl] : 0;
    const int tok = vec < n_all ? vec / a.k : vec - n_all;
    const uint16_t* xrow = a.x + (size_t)tok * H;
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < SPW; ++q) {
      u32x4_t xa[4];
      const bool ok = okb[q] && row_ok;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        xa[ks] = ok ? *reinterpret_cast<const u32x4_t*>(xrow + (size_t)blk[q] * 32 + 8 * ks) : u32x4_t{0, 0, 0, 0};
      if (b0 == 0) {                               // the weights into the operand layout, once
        wfrag_to_operand<FMT>(fg[q]);
        wfrag_to_operand<FMT>(fu[q]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[ks]);
        accg = mfma(av, wfrag_op<FMT>(fg[q], ks, okb[q]), accg);
        accu = mfma(av, wfrag_op<FMT>(fu[q], ks, okb[q]), accu);
      }
    }
    s_red[wave][0][lane] = accg;
    s_red[wave][1][lane] = accu;
    __syncthreads();
    if (wave == 0) {
      const f32x4_t g = ((s_red[0][0][lane] + s_red[1][0][lane]) + s_red[2][0][lane]) + s_red[3][0][lane];
      const f32x4_t up = ((s_red[0][1][lane] + s_red[1][1][lane]) + s_red[2][1][lane]) + s_red[3][1][lane];
      // D[token row 4 g4 + j][weight row rl]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 4 * g4 + j;
        if (m < nb) {
          const float h = silu(g[j]) * up[j];
          const uint16_t hi = f32_to_bf16_rne(h);
          const size_t o = (size_t)s_vec[b0 + m] * I + i0 + rl;
          a.h_hi[o] = hi;
          a.h_lo[o] = f32_to_bf16_rne(h - bf16_val(hi));
        }
      }
    }
    __syncthreads();
  }
  // fill-through: the fragments read from the host go into the slot
  if (wb) {
#pragma unroll
    for (int q = 0; q < SPW; ++q) {
      if (!okb[q]) continue;
      wfrag_store<FMT>(fg[q], wb + (size_t)(i0 + rl) * row_bytes,
                       FMT == MC_MXFP4 ? wbs + (size_t)(i0 + rl) * (H / 32) : nullptr, blk[q]);
      wfrag_store<FMT>(fu[q], wb + (size_t)(I + i0 + rl) * row_bytes,
                       FMT == MC_MXFP4 ? wbs + (size_t)(I + i0 + rl) * (H / 32) : nullptr, blk[q]);
    }
  }
}

// ---------------------------------------------------------------- h staging

// XOR applied to the 16-byte chunks of an LDS row of h (rows of I bf16).
__device__ __forceinline__ int h_cmask(int I) { return (I / 8) % 16 == 0 ? 15 : 7; }

// LDS rows of h: row R = 2 b + half (half 0 = hi, 1 = lo) of the b-th staged vector,
// I bf16 each; 16-byte chunk c of row R sits at chunk c ^ (R & cmask), so the 16 rows
// an operand read touches fall in different banks.  Copied by DMA (global_load_lds,
// 1 KiB per wave instruction, the LDS area rounded up to whole KiB): LDS position is
// fixed per lane, so each lane fetches the global chunk that belongs there.
__device__ __forceinline__ void stage_h(const DecodeArgs& a, const int32_t* vecs, int nvec, uint16_t* s_hv,
                                        int wave, int lane) {
  const int I = a.I;
  const int cpr = I / 8, cmask = h_cmask(I);
  const int total = 2 * nvec * cpr;
  for (int ch = wave; ch * 64 < total; ch += 4) {
    int p = ch * 64 + lane;
    if (p >= total) p = total - 1;               // tail lanes re-read a valid chunk
    const int R = p / cpr, c = (p % cpr) ^ (R & cmask);
    const uint16_t* src = (R & 1 ? a.h_lo : a.h_hi) + (size_t)vecs[R >> 1] * I + c * 8;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(s_hv + ch * 512), 16, 0,
                                     0);
  }
}

// Activation operand of MFMA ks in block `blk`: row R of the staged h.
__device__ __forceinline__ bf16x8_t h_op(const uint16_t* s_hv, int R, int blk, int ks, int I) {
  const int c = (blk * 4 + ks) ^ (R & h_cmask(I));
  return *reinterpret_cast<const bf16x8_t*>(s_hv + (size_t)R * I + c * 8);
}

// ---------------------------------------------------------------- one token
//
// At batch 1 a layer's weights are streamed once and each lane's work per 16-byte
// chunk is a handful of instructions, so what decides the time is that every load of
// the grid is in flight in a single round of resident workgroups.  Both one-token
// kernels read whole row slices (lane l takes 16-byte chunks l, l + 64, ... of a row:
// one coalesced 1 KiB piece per load instruction) straight into registers and keep
// their register count low enough for the whole grid to be resident at once.

// x pairs: packed bf16 pairs of the chunk's activations.
// MXFP4 chunk: 32 elements, 16 B codes, one e8m0 scale; x: 16 dwords.
__device__ __forceinline__ float dot_chunk_mx(const u32x4_t& w, float scale, const uint32_t* xp, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(w[q], scale), xp[4 * q + 0], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(w[q], scale), xp[4 * q + 1], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(w[q], scale), xp[4 * q + 2], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(w[q], scale), xp[4 * q + 3], acc);
  }
  return acc;
}

// bf16 chunk: 8 elements; x: 4 dwords.
__device__ __forceinline__ float dot_chunk_bf(const u32x4_t& w, const uint32_t* xp, float acc) {
  acc = dot2_bf16(w[0], xp[0], acc);
  acc = dot2_bf16(w[1], xp[1], acc);
  acc = dot2_bf16(w[2], xp[2], acc);
  acc = dot2_bf16(w[3], xp[3], acc);
  return acc;
}

// fp32 activations (h): MXFP4 chunk of 32 weights against 32 floats.
__device__ __forceinline__ float dot_chunk_mx_f32(const u32x4_t& w, float scale, const float* h, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x2_t p0 = fp4x2_to_f32x2<0>(w[q], scale);
    f32x2_t p1 = fp4x2_to_f32x2<1>(w[q], scale);
    f32x2_t p2 = fp4x2_to_f32x2<2>(w[q], scale);
    f32x2_t p3 = fp4x2_to_f32x2<3>(w[q], scale);
    acc = fmaf(p0.x, h[8 * q + 0], acc);
    acc = fmaf(p0.y, h[8 * q + 1], acc);
    acc = fmaf(p1.x, h[8 * q + 2], acc);
    acc = fmaf(p1.y, h[8 * q + 3], acc);
    acc = fmaf(p2.x, h[8 * q + 4], acc);
    acc = fmaf(p2.y, h[8 * q + 5], acc);
    acc = fmaf(p3.x, h[8 * q + 6], acc);
    acc = fmaf(p3.y, h[8 * q + 7], acc);
  }
  return acc;
}

__device__ __forceinline__ float dot_chunk_bf_f32(const u32x4_t& w, const float* h, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(bf16_lo(w[q]), h[2 * q], acc);
    acc = fmaf(bf16_hi(w[q]), h[2 * q + 1], acc);
  }
  return acc;
}

// gate_up for one token: group of 256 threads = (route column, 4 * NP intermediate rows);
// each wave owns NP gate rows and the NP matching up rows of the route's slot (or of the
// shared expert).  Every route with a valid slot runs (a slot named twice by the token is
// read twice, which only a malformed id list can cause).  NP, measured on one box (A/B in
// one run): the pass alone (HBM) is fastest with NP = 1 (Qwen shape 9.9 against 10.3 µs,
// DeepSeek-V4-Flash shape 21.7 against 23.3 with NP = 2), the launch that also carries
// the fills with NP = 4 for rows of one 16-B chunk per lane (58 against 54.5 GB/s over the
// host link, 2.61 against 2.65-2.68 ms per decode token); wider rows keep NP = 2 there,
// within the registers of four waves per SIMD.
constexpr int kTok1NP = 1;                                     // the pass alone
template <int CPL> constexpr int tok1_fill_np() { return CPL == 1 ? 4 : 2; }   // with the fills (no spills)
template <int FMT, int CPL, int NP>
__device__ __forceinline__ void gate_up_tok1_role(const DecodeArgs& a, int u, int ib) {
  const int k = a.k;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;   // wave of its 256-thread group
  const bool shared_unit = a.has_shared && u == k;
  const int slot_raw = shared_unit ? -1 : a.slots[u];
  if (valid_tokens(a) == 0) return;
  const int slot = (slot_raw >= 0 && slot_raw < a.n_pool) ? slot_raw : -1;
  if (!shared_unit && slot < 0) return;
  const int H = a.H, I = a.I;
  constexpr int ELEMS = FMT == MC_MXFP4 ? 32 : 8;              // elements per 16-B chunk
  const int n_chunks = H / ELEMS;
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)H / 2 : (size_t)H * 2;
  const size_t per_gu = 2 * (size_t)I * row_bytes, per_gus = (size_t)2 * I * H / 32;
  const uint8_t* gu;
  const uint8_t* gus = nullptr;
  uint8_t* wb = nullptr;
  uint8_t* wbs = nullptr;
  int64_t src = -1;
  if (shared_unit) {
    gu = a.sh_gu;
    gus = a.sh_gus;
  } else {
    gu = a.gu + (size_t)slot * per_gu;
    if (FMT == MC_MXFP4) gus = a.gus + (size_t)slot * per_gus;
    if (a.f_gu) src = fill_source(a, slot);
    if (src >= 0) {
      wb = const_cast<uint8_t*>(gu);
      wbs = const_cast<uint8_t*>(gus);
      gu = a.f_gu + (size_t)src * per_gu;
      if (FMT == MC_MXFP4) gus = a.f_gus + (size_t)src * per_gus;
    }
    if (ib == 0 && (threadIdx.x & (kThreads - 1)) == 0) a.rsrc[u] = (int32_t)src;
  }
  const int i0 = ib * (4 * NP) + wave * NP;
  int cq[CPL];
  bool okq[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + 64 * q;
    okq[q] = c < n_chunks;
    cq[q] = okq[q] ? c : n_chunks - 1;
  }
  // all loads of the wave's 4 rows first, the scale bytes kept raw until every load is issued
  u32x4_t wv[2 * NP][CPL];
  uint32_t sb[2 * NP][CPL];
#pragma unroll
  for (int r = 0; r < 2 * NP; ++r) {
    const int row = r < NP ? i0 + r : I + i0 + r - NP;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      wv[r][q] = stream_load16(gu + (size_t)row * row_bytes + (size_t)cq[q] * 16);
      if (FMT == MC_MXFP4) sb[r][q] = gus[(size_t)row * (H / 32) + cq[q]];
    }
  }
  const uint16_t* xrow = a.x;                                  // the one token
  float acc[2 * NP];
#pragma unroll
  for (int r = 0; r < 2 * NP; ++r) acc[r] = 0.f;
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    uint32_t xp[ELEMS / 2];
    const u32x4_t* xs = reinterpret_cast<const u32x4_t*>(xrow + (size_t)cq[q] * ELEMS);
#pragma unroll
    for (int v = 0; v < ELEMS / 8; ++v) {
      const u32x4_t xx = xs[v];
      xp[4 * v + 0] = xx[0];
      xp[4 * v + 1] = xx[1];
      xp[4 * v + 2] = xx[2];
      xp[4 * v + 3] = xx[3];
    }
#pragma unroll
    for (int r = 0; r < 2 * NP; ++r) {
      const u32x4_t wq = okq[q] ? wv[r][q] : u32x4_t{0, 0, 0, 0};
      acc[r] = FMT == MC_MXFP4 ? dot_chunk_mx(wq, e8m0_to_f32(sb[r][q]), xp, acc[r]) : dot_chunk_bf(wq, xp, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 2 * NP; ++r) acc[r] = wave_sum(acc[r]);
#pragma unroll
  for (int r = 0; r < NP; ++r)
    if (lane == r) a.h32[(size_t)u * I + i0 + r] = silu(acc[r]) * acc[NP + r];
  if (wb) {
#pragma unroll
    for (int r = 0; r < 2 * NP; ++r) {
      const int row = r < NP ? i0 + r : I + i0 + r - NP;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        if (!okq[q]) continue;
        *reinterpret_cast<u32x4_t*>(wb + (size_t)row * row_bytes + (size_t)cq[q] * 16) = wv[r][q];
        if (FMT == MC_MXFP4) wbs[(size_t)row * (H / 32) + cq[q]] = (uint8_t)sb[r][q];
      }
    }
  }
}

template <int FMT, int CPL>
__global__ void __launch_bounds__(kThreads)
gate_up_tok1_kernel(DecodeArgs a) {
  gate_up_tok1_role<FMT, CPL, kTok1NP>(a, blockIdx.y, blockIdx.x);
}

// The same pass with the fill's down-bank copy in the launch.  A workgroup of NT threads
// runs NT / 256 groups: group v < n_gu is gate_up group (route v mod nu, row block v / nu,
// 4 * tok1_fill_np rows), which fills through its gate_up banks, and the
// groups after n_gu copy chunk (j mod chunks) of fill entry (j / chunks) into its slot's
// down banks (the fill kernel's loop, entries beyond *n_fill skipped).  The copies and
// the filled routes' gate_up rows share the host link while the hits' rows stream from
// HBM.  Measured on the Qwen-shaped decode step (one box, A/B in one run each): the
// copies after the gate_up groups 2.66 against 2.74 ms with them first; 1024-thread
// workgroups 2.64-2.66 against 2.67-2.68 ms with 256-thread ones.  NT: threads per
// workgroup (256 for CPL 4, whose registers do not fit four waves per SIMD).
template <int FMT, int CPL, int NT>
__global__ void __launch_bounds__(NT)
gate_up_fill_tok1_kernel(DecodeArgs a, FillSegs g, int n_gu) {
  const int v = (int)blockIdx.x * (NT / kThreads) + (int)(threadIdx.x / kThreads);
  if (v >= n_gu) {
    const int chunks = g.chunk0[4];
    const int i = (v - n_gu) / chunks;
    if (i >= min(*a.n_fill, a.kcap)) return;
    fill_chunk<kFusedCopyUnroll>(g, a.fill_flat[i], a.fill_slot[i], v - n_gu - i * chunks);
    return;
  }
  const int nu = a.k + a.has_shared;
  gate_up_tok1_role<FMT, CPL, tok1_fill_np<CPL>()>(a, v % nu, v / nu);
}

// down for one token: workgroup = ROWS hidden rows over every route of the token.  The
// token's h vectors are staged in LDS; each wave takes every fourth route, loads all of
// its rows first, then computes; the waves' partial sums meet in LDS and are added in
// a fixed order, so every output element is written once (no atomics, run-to-run
// identical), together with the bf16 output when asked.
constexpr int kRoutesPerWave = 3;          // routes a wave holds in registers at once

template <int FMT, int LPR, int CPLB, int ROWS>
__global__ void __launch_bounds__(kThreads)
down_tok1_kernel(DecodeArgs a) {
  extern __shared__ float s_h[];                 // [k + 1][I]: the token's h vectors (swizzled)
  __shared__ float s_part[4][ROWS];
  const int H = a.H, I = a.I, k = a.k;
  const int r0 = blockIdx.x * ROWS;
  const int n_raw = a.n_tok ? *a.n_tok : a.T;
  float y_old = 0.0f;                            // the value accumulated into
  if (a.accumulate && threadIdx.x < ROWS && r0 + (int)threadIdx.x < H) y_old = a.y[r0 + threadIdx.x];
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
  const int nvec = k + a.has_shared;

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

  constexpr int kGroup = 4 * kRoutesPerWave;
  const int n_groups = (nvec + kGroup - 1) / kGroup;
  u32x4_t wv[kRoutesPerWave][PASSES][CPLB];
  uint32_t sb[kRoutesPerWave][PASSES][CPLB];
  float gate[kRoutesPerWave];
  int wsl[kRoutesPerWave];                   // fill-through: slot the rows are stored to, or -1
  // the wave's routes v0, v0+4, v0+8: slots, gates and host sources in one round trip
  // (route index clamped into the token's routes), then the rows that depend on them
  auto load_group = [&](int v0) {
    int s_raw[kRoutesPerWave], src_raw[kRoutesPerWave];
    float g_raw[kRoutesPerWave];
#pragma unroll
    for (int j = 0; j < kRoutesPerWave; ++j) {
      const int r = min(v0 + 4 * j, k - 1);
      s_raw[j] = a.slots[r];
      g_raw[j] = a.w[r];
      src_raw[j] = a.f_dn ? a.rsrc[r] : -1;
    }
#pragma unroll
    for (int j = 0; j < kRoutesPerWave; ++j) {
      const int v = v0 + 4 * j;
      const uint8_t* dn = a.dn;            // any readable address when there is nothing to read
      const uint8_t* dns = a.dns;
      gate[j] = 0.0f;
      wsl[j] = -1;
      if (v < k) {
        const int s = (s_raw[j] >= 0 && s_raw[j] < a.n_pool) ? s_raw[j] : -1;
        if (s >= 0) {
          dn = a.dn + (size_t)s * per;
          if (FMT == MC_MXFP4) dns = a.dns + (size_t)s * per_s;
          gate[j] = g_raw[j];
          if (src_raw[j] >= 0 && src_raw[j] < a.n_host) {
            wsl[j] = s;
            dn = a.f_dn + (size_t)src_raw[j] * per;
            if (FMT == MC_MXFP4) dns = a.f_dns + (size_t)src_raw[j] * per_s;
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
          wv[j][p][q] = stream_load16(dn + (size_t)rowp[p] * row_bytes + (size_t)cq[q] * 16);
          if (FMT == MC_MXFP4) sb[j][p][q] = dns[(size_t)rowp[p] * (I / 32) + cq[q]];
        }
    }
  };

  // h of this token straight into LDS (global_load_lds, 1 KiB per wave instruction),
  // then the first route group's rows: both sets of loads are in flight together.
  // Float4 e of chunk c sits at LDS float4 c * E4 + (e ^ (c & (E4 - 1))): the lanes of a
  // row, which read the same e of consecutive chunks, hit different banks, and each
  // chunk still comes from one contiguous piece of global memory.
  const int n4 = nvec * I / 4, r4 = I / 4;
  for (int ch = wave; ch * 64 < n4; ch += 4) {
    int i4 = ch * 64 + lane;
    if (i4 >= n4) i4 = n4 - 1;                       // tail lanes re-read a valid vector
    const int v = i4 / r4, sl = i4 % r4, c = sl / E4;
    const int e = (c * E4 + ((sl % E4) ^ (c & (E4 - 1)))) * 4;
    __builtin_amdgcn_global_load_lds(a.h32 + (size_t)v * I + e,
                                     (__attribute__((address_space(3))) void*)(s_h + ch * 256), 16, 0, 0);
  }
  const int nt = min(max(n_raw, 0), a.T);
  if (nt == 0) {                                     // no valid token: the rows are zero
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x < ROWS && r0 + (int)threadIdx.x < H) {
      if (!a.accumulate) a.y[r0 + threadIdx.x] = 0.0f;
      if (a.y_bf16) a.y_bf16[r0 + threadIdx.x] = 0;
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
    for (int j = 0; j < kRoutesPerWave; ++j) {
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
          const u32x4_t wq = okq[q] ? wv[j][p][q] : u32x4_t{0, 0, 0, 0};
          const float part = FMT == MC_MXFP4 ? dot_chunk_mx_f32(wq, e8m0_to_f32(sb[j][p][q]), hv, 0.0f)
                                             : dot_chunk_bf_f32(wq, hv, 0.0f);
          acc[p] = fmaf(gate[j], part, acc[p]);
        }
      }
    }
    // fill-through: rows read from the host go into the slot (rows of this block)
#pragma unroll
    for (int j = 0; j < kRoutesPerWave; ++j) {
      if (wsl[j] < 0) continue;
      uint8_t* wb = const_cast<uint8_t*>(a.dn) + (size_t)wsl[j] * per;
      uint8_t* wbs = FMT == MC_MXFP4 ? const_cast<uint8_t*>(a.dns) + (size_t)wsl[j] * per_s : nullptr;
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int rl = row_sub + RPP * p, row = r0 + rl;
        if (rl >= ROWS || row >= H) continue;
#pragma unroll
        for (int q = 0; q < CPLB; ++q) {
          if (!okq[q]) continue;
          *reinterpret_cast<u32x4_t*>(wb + (size_t)row * row_bytes + (size_t)cq[q] * 16) = wv[j][p][q];
          if (FMT == MC_MXFP4) wbs[(size_t)row * (I / 32) + cq[q]] = (uint8_t)sb[j][p][q];
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
    if (row < H) {
      float v = ((s_part[0][threadIdx.x] + s_part[1][threadIdx.x]) + s_part[2][threadIdx.x]) +
                s_part[3][threadIdx.x];
      if (a.accumulate) v += y_old;
      a.y[row] = v;
      if (a.y_bf16) a.y_bf16[row] = f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------- down, one token, wide rows
//
// For rows of 64 lanes (I / 32 >= 64 MXFP4 blocks): workgroup = ROWS hidden rows over
// every route of the token, each wave its own rows (all routes), so the work is even
// whatever the route count.  The rows go out right behind the copies of h into LDS and
// the waves start computing as soon as h has landed, the later routes' rows still
// streaming in.  A row's sum is formed in one wave in a fixed order (routes 0..k-1, then
// the shared expert, lanes by a fixed butterfly).

template <int FMT, int LPR, int CPLB, int NV>
__device__ __forceinline__ void tok1_down_role(const DecodeArgs& a, int d, float* s_h) {
  const int H = a.H, I = a.I, k = a.k;
  constexpr int ELEMS = FMT == MC_MXFP4 ? 32 : 8;
  constexpr int E4 = ELEMS / 4;                              // float4 of h per chunk
  constexpr int RPP = 64 / LPR;                              // rows per pass of a wave
  constexpr int NPASS = LPR == 64 ? 2 : 1;
  constexpr int ROWS = 4 * NPASS * RPP;                      // rows of the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_sub = lane / LPR, c_lane = lane % LPR;
  const int n_chunks = I / ELEMS;
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)I / 2 : (size_t)I * 2;
  const size_t per = (size_t)H * row_bytes;
  const size_t per_s = (size_t)H * I / 32;
  const int nvec = k + a.has_shared;
  const int nt = valid_tokens(a);
  const int rw0 = d * ROWS + wave * NPASS * RPP;             // first row of the wave

  int rowc[NPASS];
  bool rowok[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int row = rw0 + RPP * p + row_sub;
    rowok[p] = row < H;
    rowc[p] = min(row, H - 1);
  }
  int cq[CPLB];
  bool okq[CPLB];
#pragma unroll
  for (int q = 0; q < CPLB; ++q) {
    const int c = c_lane + LPR * q;
    okq[q] = c < n_chunks;
    cq[q] = okq[q] ? c : n_chunks - 1;
  }

  u32x4_t wv[NV][NPASS][CPLB];
  uint32_t sb[NV][NPASS][CPLB];
  float gate[NV];
  int wsl[NV];                                 // fill-through: slot the rows go to, or -1
  // units v0 .. v0 + NV - 1: slot, gate and host source
  const uint8_t* dnp[NV];
  const uint8_t* dnsp[NV];
  auto meta_group = [&](int v0) {
    // the slots, gates and host sources of all NV units in one round trip (indices
    // clamped into the token's routes), then the pointers that depend on them
    int s_raw[NV], src_raw[NV];
    float g_raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int r = min(v0 + j, k - 1);
      s_raw[j] = a.slots[r];
      g_raw[j] = a.w[r];
      src_raw[j] = a.f_dn ? a.rsrc[r] : -1;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = v0 + j;
      dnp[j] = nullptr;
      dnsp[j] = nullptr;
      gate[j] = 0.0f;
      wsl[j] = -1;
      if (v < nvec && nt > 0) {
        if (v < k) {
          const int sl = (s_raw[j] >= 0 && s_raw[j] < a.n_pool) ? s_raw[j] : -1;
          if (sl >= 0) {
            dnp[j] = a.dn + (size_t)sl * per;
            if (FMT == MC_MXFP4) dnsp[j] = a.dns + (size_t)sl * per_s;
            gate[j] = g_raw[j];
            const int64_t src = src_raw[j];              // the host source gate_up found
            if (src >= 0 && src < a.n_host) {
              wsl[j] = sl;
              dnp[j] = a.f_dn + (size_t)src * per;
              if (FMT == MC_MXFP4) dnsp[j] = a.f_dns + (size_t)src * per_s;
            }
          }
        } else {
          dnp[j] = a.sh_dn;
          dnsp[j] = a.sh_dns;
          gate[j] = 1.0f;
        }
      }
    }
  };
  // every row the group's units need (a unit with nothing to read loads one row of
  // slot 0, the same for every lane group, and is then skipped)
  auto rows_group = [&]() {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool any = dnp[j] != nullptr;
      const uint8_t* dn = any ? dnp[j] : a.dn;
      const uint8_t* dns = any ? dnsp[j] : a.dns;
#pragma unroll
      for (int p = 0; p < NPASS; ++p)
#pragma unroll
        for (int q = 0; q < CPLB; ++q) {
          const size_t r = any ? (size_t)rowc[p] : 0;
          wv[j][p][q] = stream_load16(dn + r * row_bytes + (size_t)cq[q] * 16);
          if (FMT == MC_MXFP4) sb[j][p][q] = dns[r * (I / 32) + cq[q]];
        }
    }
  };
  auto load_group = [&](int v0) {
    meta_group(v0);
    rows_group();
  };
  auto compute_group = [&](int v0, float* acc) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = v0 + j;
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
        for (int p = 0; p < NPASS; ++p) {
          const u32x4_t wq = okq[q] ? wv[j][p][q] : u32x4_t{0, 0, 0, 0};
          const float part = FMT == MC_MXFP4 ? dot_chunk_mx_f32(wq, e8m0_to_f32(sb[j][p][q]), hv, 0.0f)
                                             : dot_chunk_bf_f32(wq, hv, 0.0f);
          acc[p] = fmaf(gate[j], part, acc[p]);
        }
      }
    }
    // fill-through: the rows read from the host go into their slot
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (wsl[j] < 0) continue;
      uint8_t* wb = const_cast<uint8_t*>(a.dn) + (size_t)wsl[j] * per;
      uint8_t* wbs = FMT == MC_MXFP4 ? const_cast<uint8_t*>(a.dns) + (size_t)wsl[j] * per_s : nullptr;
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        if (!rowok[p]) continue;
#pragma unroll
        for (int q = 0; q < CPLB; ++q) {
          if (!okq[q]) continue;
          *reinterpret_cast<u32x4_t*>(wb + (size_t)rowc[p] * row_bytes + (size_t)cq[q] * 16) = wv[j][p][q];
          if (FMT == MC_MXFP4) wbs[(size_t)rowc[p] * (I / 32) + cq[q]] = (uint8_t)sb[j][p][q];
        }
      }
    }
  };

  meta_group(0);
  // the token's h vectors into LDS; float4 e of chunk c at float4 c * E4 + (e ^ (c & (E4 - 1)))
  const int n4 = nvec * I / 4, r4 = I / 4;
  for (int ch = wave; ch * 64 < n4; ch += 4) {
    int i4 = ch * 64 + lane;
    if (i4 >= n4) i4 = n4 - 1;                       // tail lanes re-read a valid vector
    const int v = i4 / r4, sl = i4 % r4, c = sl / E4;
    const int e = (c * E4 + ((sl % E4) ^ (c & (E4 - 1)))) * 4;
    __builtin_amdgcn_global_load_lds(a.h32 + (size_t)v * I + e,
                                     (__attribute__((address_space(3))) void*)(s_h + ch * 256), 16, 0, 0);
  }
  // The rows go out behind the h copies (the empty asm keeps the compiler from moving
  // any load across), exactly kRowLoads vector loads per wave, all issued whatever the
  // units (a unit with nothing to read loads one row of slot 0).  Vector memory
  // operations complete in order, so waiting until at most kRowLoads are outstanding
  // waits for this wave's h copies only; the rows of later units keep streaming in
  // while the first ones are computed (the compiler waits for each register as it is
  // used).  The barrier is issued bare, so that it carries no wait for every load.
  asm volatile("" ::: "memory");
  rows_group();
  constexpr int kRowLoads = NV * NPASS * CPLB * (FMT == MC_MXFP4 ? 2 : 1);
  static_assert(kRowLoads <= 63, "vmcnt holds at most 63");
  __builtin_amdgcn_s_waitcnt((((kRowLoads >> 4) & 3) << 14) | (0xF << 8) | (0x7 << 4) | (kRowLoads & 0xF));
  asm volatile("s_barrier" ::: "memory");

  float acc[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) acc[p] = 0.0f;
  compute_group(0, acc);
  for (int v0 = NV; v0 < nvec; v0 += NV) {
    load_group(v0);
    compute_group(v0, acc);
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const float sum = group_sum(acc[p], LPR);
    if (c_lane == 0 && rowok[p]) {
      const int row = rowc[p];
      if (nt == 0) {
        if (!a.accumulate) a.y[row] = 0.0f;
        if (a.y_bf16) a.y_bf16[row] = 0;
      } else {
        const float v = a.accumulate ? a.y[row] + sum : sum;
        a.y[row] = v;
        if (a.y_bf16) a.y_bf16[row] = f32_to_bf16_rne(v);
      }
    }
  }
}

// down for one token after gate_up_tok1_kernel: workgroup = ROWS hidden rows over every
// route, each wave its own rows (balanced whatever the route count)
template <int FMT, int LPR, int CPLB, int NV>
__global__ void __launch_bounds__(kThreads)
down_tok1b_kernel(DecodeArgs a) {
  extern __shared__ float s_h2[];                 // [k + 1][I] (swizzled)
  tok1_down_role<FMT, LPR, CPLB, NV>(a, (int)blockIdx.x, s_h2);
}

// ---------------------------------------------------------------- down, several tokens


template <int FMT, int NSTEP>   // NSTEP: K steps covering all of I
__global__ void __launch_bounds__(kThreads)
down_unit_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_hv[];   // [2 tb][I]
  __shared__ int32_t s_vec[kMaxRoutes];
  __shared__ float s_gate[kMaxRoutes];
  __shared__ int32_t s_n;
  __shared__ uint32_t s_last;
  const int u = blockIdx.y, rb = blockIdx.x;
  const int H = a.H, I = a.I, k = a.k, n_all = a.T * k;
  const int r0 = rb * kUnitRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 15, g4 = lane >> 4;
  const bool shared_unit = a.has_shared && u == n_all;
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)I / 2 : (size_t)I * 2;
  const size_t per = (size_t)H * row_bytes, per_s = (size_t)H * I / 32;
  const int n_blk = I / 32;

  int slot, win_slot, nt, nr;
  if (column_unit(a, u, slot, win_slot, nt, nr)) {
    const uint8_t* dn;
    const uint8_t* dns = nullptr;
    uint8_t* wb = nullptr;
    uint8_t* wbs = nullptr;
    if (shared_unit) {
      dn = a.sh_dn;
      dns = a.sh_dns;
    } else {
      dn = a.dn + (size_t)slot * per;
      if (FMT == MC_MXFP4) dns = a.dns + (size_t)slot * per_s;
      const int64_t src = a.f_dn ? fill_source(a, slot) : -1;
      if (src >= 0) {
        wb = const_cast<uint8_t*>(dn);
        wbs = const_cast<uint8_t*>(dns);
        dn = a.f_dn + (size_t)src * per;
        if (FMT == MC_MXFP4) dns = a.f_dns + (size_t)src * per_s;
      }
    }
    // the wave's 16-row tile over all of I, loaded once
    const int prow = r0 + wave * 16 + rl;
    const int row = min(prow, H - 1);
    const int tile0 = r0 + wave * 16;                  // first row of the wave's tile
    const uint8_t* srow = FMT == MC_MXFP4 ? dns + (size_t)row * (I / 32) : nullptr;
    WFrag<FMT> f[NSTEP];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
      wfrag_load_rows<FMT>(f[s], dn, row_bytes, tile0, H - 1, srow, 4 * s, n_blk);
    if (wave == 0) {
      const int n = unit_vectors(a, u, slot, win_slot, nt, nr, s_vec);
      for (int i = lane; i < n; i += 64) s_gate[i] = s_vec[i] < n_all ? a.w[s_vec[i]] : 1.0f;
      if (lane == 0) s_n = n;
    }
    __syncthreads();
    const int n_vec = s_n;
    for (int b0 = 0; b0 < n_vec; b0 += a.tb) {
      const int nb = min(a.tb, n_vec - b0);
      stage_h(a, s_vec + b0, nb, s_hv, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);                   // the LDS copies (and the rows) have landed
      __syncthreads();
      if (b0 == 0) {                                   // the rows into the operand layout, once
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) wfrag_to_operand<FMT>(f[s]);
      }
      for (int t0 = 0; t0 < nb; t0 += kRouteTile) {
        // product row R = 2 i + half for route t0 + i of the batch
        const int R = 2 * t0 + rl;
        const bool ok_r = R < 2 * nb;
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
          const int blk = 4 * s + g4;
          const bool ok = blk < n_blk;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8_t av = (ok_r && ok) ? h_op(s_hv, R, blk, ks, I) : bf16x8_t{};
            d = mfma(av, wfrag_op<FMT>(f[s], ks, ok), d);
          }
        }
        // lane holds D[4 g4 + j][rl]: route t0 + 2 g4 (j = 0, 1) and t0 + 2 g4 + 1 (j = 2, 3)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = t0 + 2 * g4 + e;
          if (i < nb && prow < H)
            store_coherent(a.part + (size_t)s_vec[b0 + i] * H + prow,
                           s_gate[b0 + i] * (d[2 * e] + d[2 * e + 1]));
        }
      }
      __syncthreads();                                 // the batch's LDS is free again
    }
    if (wb && prow < H) {
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const int blk = 4 * s + g4;
        if (blk < n_blk)
          wfrag_store<FMT>(f[s], wb + (size_t)prow * row_bytes,
                           FMT == MC_MXFP4 ? wbs + (size_t)prow * (I / 32) : nullptr, blk);
      }
    }
  }

  // arrival: every column arrives once per row block; the last one sums the partials
  __builtin_amdgcn_s_waitcnt(0);                       // this wave's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(a.cnt + (size_t)rb * kCntStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == gridDim.y - 1;
  }
  __syncthreads();
  if (!s_last) return;
  nt = valid_tokens(a);
  for (int i = threadIdx.x; i < a.T * kUnitRows; i += kThreads) {
    const int t = i / kUnitRows, row = r0 + i % kUnitRows;
    if (row >= H) continue;
    const size_t o = (size_t)t * H + row;
    if (t >= nt) {                                   // a token beyond the valid count
      if (!a.accumulate) a.y[o] = 0.0f;
      if (a.y_bf16) a.y_bf16[o] = 0;
      continue;
    }
    // the token's partials (routes in order, then the shared expert), eight loads in
    // flight at a time: indices past the end re-read the last one, unused
    const int nv = k + (a.has_shared ? 1 : 0);
    float sum = 0.0f;
    for (int j0 = 0; j0 < nv; j0 += 8) {
      float pv[8];
      int sl[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = min(j0 + q, nv - 1);
        sl[q] = a.slots[t * k + min(j, k - 1)];
        pv[q] = load_coherent(a.part + (size_t)(j < k ? t * k + j : n_all + t) * H + row);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q;
        if (j < k) sum += (sl[q] >= 0 && sl[q] < a.n_pool) ? pv[q] : 0.0f;
        else if (j < nv) sum += pv[q];
      }
    }
    if (a.accumulate) sum = a.y[o] + sum;
    a.y[o] = sum;
    if (a.y_bf16) a.y_bf16[o] = f32_to_bf16_rne(sum);
  }
  if (threadIdx.x == 0) a.cnt[(size_t)rb * kCntStride] = 0u;
}

// ---------------------------------------------------------------- dispatch

template <int FMT>
static bool launch_gate_up(const DecodeArgs& a, int spw, dim3 grid, hipStream_t s) {
  switch (spw) {
    case 1: hipLaunchKernelGGL((gate_up_kernel<FMT, 1>), grid, dim3(kThreads), 0, s, a); return true;
    case 2: hipLaunchKernelGGL((gate_up_kernel<FMT, 2>), grid, dim3(kThreads), 0, s, a); return true;
    case 4: hipLaunchKernelGGL((gate_up_kernel<FMT, 4>), grid, dim3(kThreads), 0, s, a); return true;
    case 8: hipLaunchKernelGGL((gate_up_kernel<FMT, 8>), grid, dim3(kThreads), 0, s, a); return true;
    default: return false;
  }
}

template <int FMT>
static bool launch_gate_up_tok1(const DecodeArgs& a, int cpl, dim3 grid, hipStream_t s) {
  switch (cpl) {
    case 1: hipLaunchKernelGGL((gate_up_tok1_kernel<FMT, 1>), grid, dim3(kThreads), 0, s, a); return true;
    case 2: hipLaunchKernelGGL((gate_up_tok1_kernel<FMT, 2>), grid, dim3(kThreads), 0, s, a); return true;
    case 4: hipLaunchKernelGGL((gate_up_tok1_kernel<FMT, 4>), grid, dim3(kThreads), 0, s, a); return true;
    default: return false;
  }
}

template <int FMT>
static bool launch_gate_up_fill_tok1(const DecodeArgs& a, int cpl, const FillSegs& g, int n_copy, int n_gu,
                                     hipStream_t s) {
  const int n = n_copy + n_gu;
  switch (cpl) {
    case 1: hipLaunchKernelGGL((gate_up_fill_tok1_kernel<FMT, 1, 1024>), dim3((n + 3) / 4), dim3(1024), 0, s, a, g,
                               n_gu);
            return true;
    case 2: hipLaunchKernelGGL((gate_up_fill_tok1_kernel<FMT, 2, 1024>), dim3((n + 3) / 4), dim3(1024), 0, s, a, g,
                               n_gu);
            return true;
    case 4: hipLaunchKernelGGL((gate_up_fill_tok1_kernel<FMT, 4, kThreads>), dim3(n), dim3(kThreads), 0, s, a, g,
                               n_gu);
            return true;
    default: return false;
  }
}

template <int FMT, int LPR>
static bool launch_down_tok1_l(const DecodeArgs& a, int cplb, dim3 grid, size_t lds, hipStream_t s) {
  if (cplb == 1) hipLaunchKernelGGL((down_tok1_kernel<FMT, LPR, 1, 8>), grid, dim3(kThreads), lds, s, a);
  else if (cplb == 2) hipLaunchKernelGGL((down_tok1_kernel<FMT, LPR, 2, 8>), grid, dim3(kThreads), lds, s, a);
  else return false;
  return true;
}

template <int FMT>
static bool launch_down_tok1(const DecodeArgs& a, int lpr, int cplb, dim3 grid, size_t lds, hipStream_t s) {
  switch (lpr) {
    case 4: return launch_down_tok1_l<FMT, 4>(a, cplb, grid, lds, s);
    case 16: return launch_down_tok1_l<FMT, 16>(a, cplb, grid, lds, s);
    default: return launch_down_tok1_l<FMT, 64>(a, cplb, grid, lds, s);
  }
}

template <int FMT, int CPLB>
static bool launch_down_tok1b_nv(const DecodeArgs& a, int nv, uint32_t n_dn, size_t lds, hipStream_t s) {
  switch (nv) {
    case 3: hipLaunchKernelGGL((down_tok1b_kernel<FMT, 64, CPLB, 3>), dim3(n_dn), dim3(kThreads), lds, s, a);
            return true;
    case 6: hipLaunchKernelGGL((down_tok1b_kernel<FMT, 64, CPLB, 6>), dim3(n_dn), dim3(kThreads), lds, s, a);
            return true;
    case 9: hipLaunchKernelGGL((down_tok1b_kernel<FMT, 64, CPLB, 9>), dim3(n_dn), dim3(kThreads), lds, s, a);
            return true;
  }
  return false;
}

// one-token down for rows of 64 lanes (two 16-B chunks per lane: three routes at once)
template <int FMT>
static bool launch_down_tok1b(const DecodeArgs& a, int cplb, int nv, uint32_t n_dn, size_t lds, hipStream_t s) {
  if (cplb == 1) return launch_down_tok1b_nv<FMT, 1>(a, nv, n_dn, lds, s);
  if (cplb == 2 && nv == 3) {
    hipLaunchKernelGGL((down_tok1b_kernel<FMT, 64, 2, 3>), dim3(n_dn), dim3(kThreads), lds, s, a);
    return true;
  }
  return false;
}

template <int FMT>
static bool launch_down_unit(const DecodeArgs& a, int nstep, dim3 grid, size_t lds, hipStream_t s) {
  switch (nstep) {
    case 1: hipLaunchKernelGGL((down_unit_kernel<FMT, 1>), grid, dim3(kThreads), lds, s, a); return true;
    case 2: hipLaunchKernelGGL((down_unit_kernel<FMT, 2>), grid, dim3(kThreads), lds, s, a); return true;
    case 4: hipLaunchKernelGGL((down_unit_kernel<FMT, 4>), grid, dim3(kThreads), lds, s, a); return true;
    case 8: hipLaunchKernelGGL((down_unit_kernel<FMT, 8>), grid, dim3(kThreads), lds, s, a); return true;
    case 16: hipLaunchKernelGGL((down_unit_kernel<FMT, 16>), grid, dim3(kThreads), lds, s, a); return true;
    default: return false;
  }
}

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

static size_t round_kib(size_t b) { return (b + 1023) & ~(size_t)1023; }

}  // namespace mc

using namespace mc;

// workspace: h as bf16 hi and lo halves of every vector [T*k + T][I] each (the
// one-token path keeps fp32 h [T*k + T][I] in the same bytes), the gated partial
// outputs [T*k + T][H] (fp32), the routes' fill-through sources [T*k] (int32), then the
// several-token down pass's arrival counters
static size_t ws_vec(int32_t T, int32_t k) { return (size_t)T * k + (size_t)T; }
static size_t ws_h_bytes(int32_t T, int32_t k, int32_t I) { return ws_vec(T, k) * (size_t)I * 2; }
static size_t ws_part_bytes(int32_t T, int32_t k, int32_t H) { return ws_vec(T, k) * (size_t)H * 4; }
static size_t ws_rsrc_bytes(int32_t T, int32_t k) { return (((size_t)T * k * 4) + 15) & ~(size_t)15; }
static size_t ws_cnt_bytes(int32_t H) {
  return (size_t)((H + kUnitRows - 1) / kUnitRows) * kCntStride * sizeof(uint32_t);
}

extern "C" size_t moe_experts_decode_ws_bytes(int32_t T, int32_t k, int32_t H, int32_t I) {
  if (T < 0 || k < 0 || H < 0 || I < 0) return 0;
  return 2 * ws_h_bytes(T, k, I) + ws_part_bytes(T, k, H) + ws_rsrc_bytes(T, k) + ws_cnt_bytes(H);
}

static int decode_impl(const void* x_bf16, const int32_t* slots, const float* w, int32_t T, int32_t k,
                       const int32_t* n_tok, const mc_banks* pool, const mc_banks* shared, void* ws,
                       size_t ws_bytes, float* y_acc, int32_t accumulate, void* y_bf16, hipStream_t s,
                       const mc_fill_list* fill) {
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
  MC_REQUIRE(ws_bytes >= moe_experts_decode_ws_bytes(T, k, pool->H, pool->I),
             "moe_experts_decode: workspace %zu < %zu bytes", ws_bytes,
             moe_experts_decode_ws_bytes(T, k, pool->H, pool->I));
  MC_REQUIRE((uintptr_t)x_bf16 % 16 == 0 && (uintptr_t)ws % 16 == 0,
             "moe_experts_decode: x and ws must be 16-byte aligned");
  const int H = pool->H, I = pool->I, fmt = pool->fmt;
  const int has_shared = shared ? 1 : 0;
  // one token: dot-product kernels over whole row slices; several: MFMA kernels
  const int elems = fmt == MC_MXFP4 ? 32 : 8;
  const int cpl1 = pow2_at_least((H / elems + 63) / 64);
  const int chunks_b = I / elems;
  const int lpr1 = chunks_b <= 4 ? 4 : (chunks_b <= 16 ? 16 : 64);
  const int cplb1 = pow2_at_least((chunks_b + lpr1 - 1) / lpr1);
  const size_t lds1 = ((size_t)(k + has_shared) * I * sizeof(float) + 1023) & ~(size_t)1023;
  // K steps of 128: the several-token gate_up splits H's steps over its 4 waves
  const int nstep_gu = (H + kKS - 1) / kKS, nstep_dn = (I + kKS - 1) / kKS;
  const int spw_gu = pow2_at_least((nstep_gu + 3) / 4);
  const int tb = (int)std::min<size_t>(std::min<size_t>(64, (size_t)T * k + 1), kHLdsBytes / ((size_t)I * 4));
  const size_t ldsn = round_kib((size_t)2 * tb * I * 2);
  const bool tile_ok = T == 1 ? (cpl1 <= 4 && cplb1 <= 2 && lds1 <= (size_t)kTok1LdsBytes)
                              : (spw_gu <= 8 && tb >= 1 && pow2_at_least(nstep_dn) <= 16);
  if (!tile_ok) {
    set_error("moe_experts_decode: H=%d I=%d k=%d T=%d is beyond the library's tiles", H, I, k, T);
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
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  a.h32 = reinterpret_cast<float*>(wsb);
  a.h_hi = reinterpret_cast<uint16_t*>(wsb);
  a.h_lo = reinterpret_cast<uint16_t*>(wsb + ws_h_bytes(T, k, I));
  a.part = reinterpret_cast<float*>(wsb + 2 * ws_h_bytes(T, k, I));
  a.rsrc = reinterpret_cast<int32_t*>(wsb + 2 * ws_h_bytes(T, k, I) + ws_part_bytes(T, k, H));
  a.cnt = reinterpret_cast<uint32_t*>(wsb + 2 * ws_h_bytes(T, k, I) + ws_part_bytes(T, k, H) +
                                      ws_rsrc_bytes(T, k));
  a.n_cnt = T == 1 ? 0 : (H + kUnitRows - 1) / kUnitRows;
  a.tb = tb;
  a.y = y_acc;
  a.y_bf16 = static_cast<uint16_t*>(y_bf16);
  a.accumulate = accumulate;
  a.has_shared = has_shared;
  if (fill) {
    if ((rc = check_banks(fill->host, "moe_experts_decode fill host")) != MC_OK) return rc;
    MC_REQUIRE(fill->host->fmt == fmt && fill->host->H == H && fill->host->I == I,
               "moe_experts_decode: fill host banks differ from the pool in format or shape");
    MC_REQUIRE(fill->kcap >= 0 && fill->fill_flat && fill->fill_slot && fill->n_fill,
               "moe_experts_decode: bad fill list");
    MC_REQUIRE(fill->mode == MC_FILL_THROUGH || fill->mode == MC_FILL_GATE_UP ||
                   fill->mode == MC_FILL_WITH_GATE_UP,
               "moe_experts_decode: fill mode=%d", fill->mode);
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
    if (fill->mode != MC_FILL_THROUGH) a.f_dn = a.f_dns = nullptr;   // down reads the slots
    if (a.kcap == 0) a.f_gu = a.f_dn = nullptr;
  }
  // the fill's down-bank copy carried by this call (MC_FILL_WITH_GATE_UP)
  const bool copy_down = fill && fill->mode == MC_FILL_WITH_GATE_UP && a.kcap > 0;
  FillSegs gd{};
  int chunks_dn = 0;
  if (copy_down) {
    MC_REQUIRE(fill->down_after == nullptr,
               "moe_experts_decode: fill mode MC_FILL_WITH_GATE_UP copies the down banks itself (down_after must be NULL)");
    MC_REQUIRE(a.kcap <= 65535, "moe_experts_decode: fill kcap=%d (0..65535)", a.kcap);
    // one token: copy groups in the gate_up launch; several: the fill kernel between the passes
    const int64_t chunk = T == 1 ? (int64_t)kFillThreads * kFusedCopyUnroll * 16
                                 : (int64_t)kFillBlock * kFillUnroll * 16;
    if ((rc = fill_segs(fill->host, pool, MC_BANK_DOWN | (fmt == MC_MXFP4 ? MC_BANK_DOWN_SCALE : 0), chunk,
                        "moe_experts_decode fill", s, &gd, &chunks_dn)) != MC_OK)
      return rc;
  }

  bool ok_a, ok_b;
  // one-token down: rows of 64 lanes take the wide-row kernel (8 rows per workgroup,
  // nv1 routes held at once), shorter rows the route-split one
  const int nvec1 = k + has_shared;
  const int nv1 = (nvec1 <= 3 || cplb1 > 1) ? 3 : (nvec1 <= 6 ? 6 : 9);
  if (T == 1 && copy_down) {
    const int np = cpl1 == 1 ? tok1_fill_np<1>() : tok1_fill_np<2>();
    const int n_copy = chunks_dn * a.kcap, n_gu = (k + has_shared) * (I / (4 * np));
    ok_a = fmt == MC_MXFP4 ? launch_gate_up_fill_tok1<MC_MXFP4>(a, cpl1, gd, n_copy, n_gu, s)
                           : launch_gate_up_fill_tok1<MC_BF16>(a, cpl1, gd, n_copy, n_gu, s);
  } else if (T == 1) {
    // a unit's row blocks are launched one after another (x), the units along y
    const dim3 grid_a(I / (4 * kTok1NP), k + has_shared);
    ok_a = fmt == MC_MXFP4 ? launch_gate_up_tok1<MC_MXFP4>(a, cpl1, grid_a, s)
                           : launch_gate_up_tok1<MC_BF16>(a, cpl1, grid_a, s);
  } else {
    // a unit's row blocks are launched one after another (x), the units along y
    const dim3 grid_a(I / 16, T * k + has_shared);
    ok_a = fmt == MC_MXFP4 ? launch_gate_up<MC_MXFP4>(a, spw_gu, grid_a, s)
                           : launch_gate_up<MC_BF16>(a, spw_gu, grid_a, s);
  }
  if (!ok_a) {
    set_error("moe_experts_decode: no gate_up tile for H=%d", H);
    return MC_EUNSUPPORTED;
  }
  MC_LAUNCH_CHECK();
  if (fill && fill->down_after) MC_HIP(hipStreamWaitEvent(s, fill->down_after, 0));
  if (T > 1 && copy_down) {          // several tokens: the down-bank copy between the passes
    if ((rc = launch_fill(gd, a.fill_flat, a.fill_slot, a.n_fill, a.kcap, s)) != MC_OK) return rc;
  }
  if (T == 1 && lpr1 == 64) {
    const uint32_t n_dn = (uint32_t)((H + 7) / 8);
    ok_b = fmt == MC_MXFP4 ? launch_down_tok1b<MC_MXFP4>(a, cplb1, nv1, n_dn, lds1, s)
                           : launch_down_tok1b<MC_BF16>(a, cplb1, nv1, n_dn, lds1, s);
  } else if (T == 1) {
    const dim3 grid_b((H + 7) / 8);
    ok_b = fmt == MC_MXFP4 ? launch_down_tok1<MC_MXFP4>(a, lpr1, cplb1, grid_b, lds1, s)
                           : launch_down_tok1<MC_BF16>(a, lpr1, cplb1, grid_b, lds1, s);
  } else {
    const dim3 grid_b((H + kUnitRows - 1) / kUnitRows, T * k + has_shared);
    ok_b = fmt == MC_MXFP4 ? launch_down_unit<MC_MXFP4>(a, pow2_at_least(nstep_dn), grid_b, ldsn, s)
                           : launch_down_unit<MC_BF16>(a, pow2_at_least(nstep_dn), grid_b, ldsn, s);
  }
  if (!ok_b) {
    set_error("moe_experts_decode: no down tile for I=%d", I);
    return MC_EUNSUPPORTED;
  }
  MC_LAUNCH_CHECK();
  return MC_OK;
}

extern "C" int moe_experts_decode(const void* x_bf16, const int32_t* slots, const float* w,
                                  int32_t T, int32_t k, const int32_t* n_tok,
                                  const mc_banks* pool, const mc_banks* shared, void* ws,
                                  size_t ws_bytes, float* y_acc, int32_t accumulate, void* y_bf16,
                                  hipStream_t s, const mc_fill_list* fill) {
  clear_error();
  return decode_impl(x_bf16, slots, w, T, k, n_tok, pool, shared, ws, ws_bytes, y_acc, accumulate, y_bf16, s,
                     fill);
}

// ---------------------------------------------------------------- no-allocation variant
//
// The workspace of moe_experts_decode_noalloc lives in this file-scope device array,
// one copy per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is only a stand-in for the symbol): the device
// address of each GPU's copy is looked up once, with that GPU current, and kept.
// Every call on a GPU shares that GPU's copy and leaves the last call's contents in it;
// no part of it needs to start at zero (the kernels write every word they later read,
// and the arrival counters are cleared by the first kernel of each call), and calls that
// overlap on one GPU race on it.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

// Device address of this GPU's scratch array (looked up on the first call per GPU).
static int scratch_for_current_device(void** out) {
  int dev = -1;
  MC_HIP(hipGetDevice(&dev));
  MC_REQUIRE(dev >= 0 && dev < kMaxDevices, "moe_experts_decode_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    MC_REQUIRE(p != nullptr, "moe_experts_decode_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MC_OK;
}

extern "C" size_t moe_experts_decode_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int moe_experts_decode_noalloc(const void* x_bf16, const int32_t* slots, const float* w,
                                          int32_t T, int32_t k, const int32_t* n_tok,
                                          const mc_banks* pool, const mc_banks* shared, float* y_acc,
                                          int32_t accumulate, void* y_bf16, hipStream_t s,
                                          const mc_fill_list* fill) {
  clear_error();
  int rc;
  if ((rc = check_banks(pool, "moe_experts_decode_noalloc pool")) != MC_OK) return rc;
  MC_REQUIRE(T >= 0 && k >= 1, "moe_experts_decode_noalloc: T=%d k=%d", T, k);
  const size_t need = moe_experts_decode_ws_bytes(T, k, pool->H, pool->I);
  if (need > kScratchBytes) {
    set_error("moe_experts_decode_noalloc: T=%d k=%d H=%d I=%d needs %zu bytes of workspace, beyond the "
              "%zu-byte scratch array (use moe_experts_decode with a workspace)",
              T, k, pool->H, pool->I, need, kScratchBytes);
    return MC_ENOMEM;
  }
  if (T == 0) return decode_impl(x_bf16, slots, w, T, k, n_tok, pool, shared, nullptr, 0, y_acc, accumulate,
                                 y_bf16, s, fill);
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws)) != MC_OK) return rc;
  return decode_impl(x_bf16, slots, w, T, k, n_tok, pool, shared, ws, kScratchBytes, y_acc, accumulate, y_bf16,
                     s, fill);
}
