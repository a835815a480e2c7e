// moe_experts_decode: slot-indirected SwiGLU experts + gated combine for decode.
//
// [jjl357] "1.1": h_t = sum_e p_{t,e} Expert_{l,e}(x_t).  [jjl357] "6.1": an expert
// routed by several tokens of the call is read and run once.  [jjl357] "6.7" step 5
// and [wanger] "代码全链路": the GPU runs hits + fills; host-computed routes arrive
// with slot -1 (or gate 0) and are skipped.
//
// Decode is a GEMV that streams ~0.53 B of MXFP4 weight per multiply-add, so it is
// bound by HBM bandwidth.  Two kernels:
//   A. gate_up + SwiGLU.  Workgroup = (unit, 16 intermediate rows); a unit is one
//      distinct slot of the call (first-occurrence order) or the shared expert.  Each
//      wave owns 4 gate rows and the 4 matching up rows; lane l reads the 16-byte
//      chunks l, l+64, ... of every row (one coalesced 1 KiB row slice per load
//      instruction), keeps them in registers and reuses them for every token that
//      routes to the unit.  Dot products run on packed bf16 (MXFP4 -> bf16 is exact)
//      with fp32 accumulation; h = silu(g) * u is written in fp32 per route.
//   B. down + combine.  Workgroup = 8 hidden rows for every route of every token, so
//      each output element is produced by exactly one lane group and written once
//      (deterministic, no atomics).  A token's route vectors h (fp32) are staged in
//      LDS; lanes split a row's contraction into 16-byte chunks and reduce across
//      the row's lanes at the end.
#include "mc_common.h"

namespace mc {

constexpr int kA_Threads = 256;
constexpr int kA_RowsI = 16;                 // intermediate rows per workgroup
constexpr int kA_WaveRows = kA_RowsI / 4;    // per wave: 4 gate + 4 up rows
constexpr int kB_Rows = 8;                   // hidden rows per workgroup (one wave)
constexpr int kMaxRoutes = 1024;
constexpr int kB_LdsBytes = 64 * 1024;

// ---------------------------------------------------------------- chunk dots

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
  float* y;                   // [T][H] accumulated
};

// ---------------------------------------------------------------- kernel A

// Unit table of the call, computed by every workgroup (at most kMaxRoutes routes):
// s_first[u] = first route of the u-th distinct valid slot.
__device__ int build_units(const DecodeArgs& a, int nr, int32_t* s_slot, int32_t* s_first,
                           int* s_cnt) {
  const int tid = threadIdx.x;
  for (int r = tid; r < nr; r += blockDim.x) {
    int s = a.slots[r];
    s_slot[r] = (s >= 0 && s < a.n_pool) ? s : -1;
  }
  if (tid == 0) *s_cnt = 0;
  __syncthreads();
  // first occurrences, ranked in route order by a serial pass of wave 0 with ballots
  if (tid < 64) {
    int count = 0;
    for (int base = 0; base < nr; base += 64) {
      int r = base + tid;
      bool first = false;
      if (r < nr && s_slot[r] >= 0) {
        first = true;
        for (int j = 0; j < r; ++j)
          if (s_slot[j] == s_slot[r]) {
            first = false;
            break;
          }
      }
      uint64_t m = __ballot(first);
      if (first) s_first[count + __popcll(m & ((1ull << tid) - 1ull))] = r;
      count += __popcll(m);
    }
    if (tid == 0) *s_cnt = count;
  }
  __syncthreads();
  return *s_cnt;
}

template <int FMT, int CPL>
__global__ void __launch_bounds__(kA_Threads)
gate_up_kernel(DecodeArgs a, int has_shared) {
  __shared__ int32_t s_slot[kMaxRoutes];
  __shared__ int32_t s_first[kMaxRoutes];
  __shared__ int s_cnt;
  const int nt = a.n_tok ? min(max(*a.n_tok, 0), a.T) : a.T;
  const int nr = nt * a.k;
  const int n_units = build_units(a, nr, s_slot, s_first, &s_cnt);
  const int u = blockIdx.x;
  const bool shared_unit = has_shared && u == n_units;
  if (u > n_units || (u == n_units && !shared_unit)) return;
  if (shared_unit && nt == 0) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int i0 = blockIdx.y * kA_RowsI + wave * kA_WaveRows;   // first intermediate row
  constexpr int ELEMS = FMT == MC_MXFP4 ? 32 : 8;              // elements per 16-B chunk
  const int n_chunks = H / ELEMS;                              // chunks per row

  const uint8_t* gu;
  const uint8_t* gus;
  int slot = -1;
  if (shared_unit) {
    gu = a.sh_gu;
    gus = a.sh_gus;
  } else {
    slot = s_slot[s_first[u]];
    const size_t per = FMT == MC_MXFP4 ? (size_t)2 * I * H / 2 : (size_t)2 * I * H * 2;
    gu = a.gu + (size_t)slot * per;
    gus = FMT == MC_MXFP4 ? a.gus + (size_t)slot * ((size_t)2 * I * H / 32) : nullptr;
  }
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)H / 2 : (size_t)H * 2;

  // weights of the wave's 8 rows: rows 0..3 gate i0.., rows 4..7 up I+i0..
  uint4 wv[2 * kA_WaveRows][CPL];
  float sc[2 * kA_WaveRows][CPL];
#pragma unroll
  for (int r = 0; r < 2 * kA_WaveRows; ++r) {
    const int row = r < kA_WaveRows ? i0 + r : I + i0 + (r - kA_WaveRows);
    const uint4* rp = reinterpret_cast<const uint4*>(gu + (size_t)row * row_bytes);
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = lane + 64 * q;
      if (c < n_chunks) {
        wv[r][q] = rp[c];
        if (FMT == MC_MXFP4) sc[r][q] = e8m0_to_f32(gus[(size_t)row * (H / 32) + c]);
      } else {
        wv[r][q] = make_uint4(0, 0, 0, 0);
        sc[r][q] = 0.0f;
      }
    }
  }

  // tokens of this unit
  int r_next = shared_unit ? 0 : s_first[u];
  while (true) {
    int t, route;
    if (shared_unit) {
      if (r_next >= nt) break;
      t = r_next;
      route = -1;
      ++r_next;
    } else {
      while (r_next < nr && s_slot[r_next] != slot) ++r_next;
      if (r_next >= nr) break;
      route = r_next;
      t = route / a.k;
      ++r_next;
    }
    const uint32_t* xrow = reinterpret_cast<const uint32_t*>(a.x + (size_t)t * H);
    float acc[2 * kA_WaveRows];
#pragma unroll
    for (int r = 0; r < 2 * kA_WaveRows; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = lane + 64 * q;
      if (c < n_chunks) {
        uint32_t xp[ELEMS / 2];
        const uint4* xs = reinterpret_cast<const uint4*>(xrow + (size_t)c * (ELEMS / 2));
#pragma unroll
        for (int v = 0; v < ELEMS / 8; ++v) {
          uint4 xx = xs[v];
          xp[4 * v + 0] = xx.x;
          xp[4 * v + 1] = xx.y;
          xp[4 * v + 2] = xx.z;
          xp[4 * v + 3] = xx.w;
        }
#pragma unroll
        for (int r = 0; r < 2 * kA_WaveRows; ++r) {
          if (FMT == MC_MXFP4)
            acc[r] = dot_chunk_mx(wv[r][q], sc[r][q], xp, acc[r]);
          else
            acc[r] = dot_chunk_bf(wv[r][q], xp, acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2 * kA_WaveRows; ++r) acc[r] = wave_sum(acc[r]);
    if (lane < kA_WaveRows) {
      float g = acc[0], up = acc[kA_WaveRows];
#pragma unroll
      for (int r = 1; r < kA_WaveRows; ++r)
        if (lane == r) {
          g = acc[r];
          up = acc[kA_WaveRows + r];
        }
      float* dst = shared_unit ? a.h_shared + (size_t)t * I : a.h_route + (size_t)route * I;
      dst[i0 + lane] = silu(g) * up;
    }
  }
}

// ---------------------------------------------------------------- kernel B

template <int FMT, int LPR, int CPLB>
__global__ void __launch_bounds__(64)
down_kernel(DecodeArgs a, int has_shared) {
  extern __shared__ float s_h[];      // [(k + 1)][I] route vectors of one token
  const int nt = a.n_tok ? min(max(*a.n_tok, 0), a.T) : a.T;
  const int lane = threadIdx.x;
  const int H = a.H, I = a.I, k = a.k;
  constexpr int ELEMS = FMT == MC_MXFP4 ? 32 : 8;
  constexpr int RPP = 64 / LPR;                      // rows per pass
  constexpr int PASSES = kB_Rows >= RPP ? kB_Rows / RPP : 1;
  const int n_chunks = I / ELEMS;
  const int row_sub = lane / LPR, c_lane = lane % LPR;
  const int r0 = blockIdx.x * kB_Rows;
  const size_t row_bytes = FMT == MC_MXFP4 ? (size_t)I / 2 : (size_t)I * 2;
  const size_t per = FMT == MC_MXFP4 ? (size_t)H * I / 2 : (size_t)H * I * 2;
  const size_t per_s = (size_t)H * I / 32;
  const int nvec = k + (has_shared ? 1 : 0);

  for (int t = 0; t < nt; ++t) {
    // stage h of this token's routes (and the shared expert) in LDS
    __syncthreads();
    for (int v = 0; v < nvec; ++v) {
      const float* src = v < k ? a.h_route + ((size_t)t * k + v) * I : a.h_shared + (size_t)t * I;
      bool valid = true;
      if (v < k) {
        int s = a.slots[(size_t)t * k + v];
        valid = s >= 0 && s < a.n_pool;
      }
      if (!valid) continue;
      for (int i = lane * 4; i < I; i += 64 * 4)
        *reinterpret_cast<float4*>(s_h + (size_t)v * I + i) =
            *reinterpret_cast<const float4*>(src + i);
    }
    __syncthreads();

    float acc[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) acc[p] = 0.0f;

    for (int v = 0; v < nvec; ++v) {
      const uint8_t* dn;
      const uint8_t* dns;
      float gate;
      if (v < k) {
        const int s = a.slots[(size_t)t * k + v];
        if (s < 0 || s >= a.n_pool) continue;
        gate = a.w[(size_t)t * k + v];
        dn = a.dn + (size_t)s * per;
        dns = FMT == MC_MXFP4 ? a.dns + (size_t)s * per_s : nullptr;
      } else {
        gate = 1.0f;
        dn = a.sh_dn;
        dns = a.sh_dns;
      }
      // issue all weight loads of this route first
      uint4 wv[PASSES][CPLB];
      float sc[PASSES][CPLB];
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = r0 + row_sub + RPP * p;
#pragma unroll
        for (int q = 0; q < CPLB; ++q) {
          const int c = c_lane + LPR * q;
          if (row < H && c < n_chunks && (RPP <= kB_Rows || row_sub < kB_Rows)) {
            wv[p][q] = reinterpret_cast<const uint4*>(dn + (size_t)row * row_bytes)[c];
            if (FMT == MC_MXFP4) sc[p][q] = e8m0_to_f32(dns[(size_t)row * (I / 32) + c]);
          } else {
            wv[p][q] = make_uint4(0, 0, 0, 0);
            sc[p][q] = 0.0f;
          }
        }
      }
#pragma unroll
      for (int q = 0; q < CPLB; ++q) {
        const int c = c_lane + LPR * q;
        if (c >= n_chunks) continue;
        float hv[ELEMS];
        const float4* hs = reinterpret_cast<const float4*>(s_h + (size_t)v * I + (size_t)c * ELEMS);
#pragma unroll
        for (int e = 0; e < ELEMS / 4; ++e) {
          float4 f = hs[e];
          hv[4 * e + 0] = f.x;
          hv[4 * e + 1] = f.y;
          hv[4 * e + 2] = f.z;
          hv[4 * e + 3] = f.w;
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          float part = FMT == MC_MXFP4 ? dot_chunk_mx_f32(wv[p][q], sc[p][q], hv, 0.0f)
                                       : dot_chunk_bf_f32(wv[p][q], hv, 0.0f);
          acc[p] = fmaf(gate, part, acc[p]);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float sum = group_sum(acc[p], LPR);
      const int row = r0 + row_sub + RPP * p;
      if (c_lane == 0 && row < H && (RPP <= kB_Rows || row_sub < kB_Rows))
        a.y[(size_t)t * H + row] += sum;
    }
  }
}

// ---------------------------------------------------------------- dispatch

template <int FMT>
static void launch_gate_up(const DecodeArgs& a, int has_shared, int cpl, dim3 grid, hipStream_t s) {
  switch (cpl) {
    case 1: hipLaunchKernelGGL((gate_up_kernel<FMT, 1>), grid, dim3(kA_Threads), 0, s, a, has_shared); break;
    case 2: hipLaunchKernelGGL((gate_up_kernel<FMT, 2>), grid, dim3(kA_Threads), 0, s, a, has_shared); break;
    case 4: hipLaunchKernelGGL((gate_up_kernel<FMT, 4>), grid, dim3(kA_Threads), 0, s, a, has_shared); break;
    default: hipLaunchKernelGGL((gate_up_kernel<FMT, 8>), grid, dim3(kA_Threads), 0, s, a, has_shared); break;
  }
}

template <int FMT, int LPR>
static void launch_down_l(const DecodeArgs& a, int has_shared, int cplb, dim3 grid, size_t lds,
                          hipStream_t s) {
  switch (cplb) {
    case 1: hipLaunchKernelGGL((down_kernel<FMT, LPR, 1>), grid, dim3(64), lds, s, a, has_shared); break;
    case 2: hipLaunchKernelGGL((down_kernel<FMT, LPR, 2>), grid, dim3(64), lds, s, a, has_shared); break;
    default: hipLaunchKernelGGL((down_kernel<FMT, LPR, 4>), grid, dim3(64), lds, s, a, has_shared); break;
  }
}

template <int FMT>
static void launch_down(const DecodeArgs& a, int has_shared, int lpr, int cplb, dim3 grid,
                        size_t lds, hipStream_t s) {
  switch (lpr) {
    case 2: launch_down_l<FMT, 2>(a, has_shared, cplb, grid, lds, s); break;
    case 4: launch_down_l<FMT, 4>(a, has_shared, cplb, grid, lds, s); break;
    case 8: launch_down_l<FMT, 8>(a, has_shared, cplb, grid, lds, s); break;
    case 16: launch_down_l<FMT, 16>(a, has_shared, cplb, grid, lds, s); break;
    case 32: launch_down_l<FMT, 32>(a, has_shared, cplb, grid, lds, s); break;
    default: launch_down_l<FMT, 64>(a, has_shared, cplb, grid, lds, s); break;
  }
}

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace mc

using namespace mc;

extern "C" size_t moe_experts_decode_ws_bytes(int32_t T, int32_t k, int32_t I) {
  if (T < 0 || k < 0 || I < 0) return 0;
  return ((size_t)T * k + (size_t)T) * (size_t)I * sizeof(float);
}

extern "C" int moe_experts_decode(const void* x_bf16, const int32_t* slots, const float* w,
                                  int32_t T, int32_t k, const int32_t* n_tok,
                                  const mc_banks* pool, const mc_banks* shared, void* ws,
                                  size_t ws_bytes, float* y_acc, hipStream_t s) {
  clear_error();
  int rc;
  if ((rc = check_banks(pool, "moe_experts_decode pool")) != MC_OK) return rc;
  if (shared) {
    if ((rc = check_banks(shared, "moe_experts_decode shared")) != MC_OK) return rc;
    MC_REQUIRE(shared->fmt == pool->fmt && shared->H == pool->H && shared->I == pool->I,
               "moe_experts_decode: shared expert differs from the pool in format or shape");
  }
  MC_REQUIRE(T >= 0 && k >= 1, "moe_experts_decode: T=%d k=%d", T, k);
  MC_REQUIRE((int64_t)T * k <= kMaxRoutes, "moe_experts_decode: T*k=%lld exceeds %d",
             (long long)T * k, kMaxRoutes);
  if (T == 0) return MC_OK;
  MC_REQUIRE(x_bf16 && slots && w && y_acc && ws, "moe_experts_decode: NULL pointer");
  MC_REQUIRE(ws_bytes >= moe_experts_decode_ws_bytes(T, k, pool->I),
             "moe_experts_decode: workspace %zu < %zu bytes", ws_bytes,
             moe_experts_decode_ws_bytes(T, k, pool->I));
  MC_REQUIRE((uintptr_t)x_bf16 % 16 == 0 && (uintptr_t)ws % 16 == 0,
             "moe_experts_decode: x and ws must be 16-byte aligned");
  const int H = pool->H, I = pool->I, fmt = pool->fmt;
  const int nvec = k + (shared ? 1 : 0);
  const size_t lds = (size_t)nvec * I * sizeof(float);
  if (lds > (size_t)kB_LdsBytes) {
    set_error("moe_experts_decode: (k+1)*I*4 = %zu bytes of staged activations exceed %d", lds,
              kB_LdsBytes);
    return MC_EUNSUPPORTED;
  }
  const int elems = fmt == MC_MXFP4 ? 32 : 8;
  const int cpl = pow2_at_least((H / elems + 63) / 64);
  if (cpl > 8) {
    set_error("moe_experts_decode: H=%d too large", H);
    return MC_EUNSUPPORTED;
  }
  const int chunks_b = I / elems;
  int lpr = chunks_b >= 64 ? 64 : pow2_at_least(chunks_b);
  if (lpr < 2) lpr = 2;
  const int cplb = pow2_at_least((chunks_b + lpr - 1) / lpr);
  if (cplb > 4) {
    set_error("moe_experts_decode: I=%d too large", I);
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
  const int has_shared = shared ? 1 : 0;

  dim3 grid_a(T * k + has_shared, I / kA_RowsI);
  if (fmt == MC_MXFP4)
    launch_gate_up<MC_MXFP4>(a, has_shared, cpl, grid_a, s);
  else
    launch_gate_up<MC_BF16>(a, has_shared, cpl, grid_a, s);
  MC_LAUNCH_CHECK();
  dim3 grid_b((H + kB_Rows - 1) / kB_Rows);
  if (fmt == MC_MXFP4)
    launch_down<MC_MXFP4>(a, has_shared, lpr, cplb, grid_b, lds, s);
  else
    launch_down<MC_BF16>(a, has_shared, lpr, cplb, grid_b, lds, s);
  MC_LAUNCH_CHECK();
  return MC_OK;
}
