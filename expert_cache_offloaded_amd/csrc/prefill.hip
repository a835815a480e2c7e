// moe_experts_prefill: token-sorted grouped expert GEMM over one layer's resident
// experts, plus the whole-layer prefetch of the next layer.
//
// [jjl357] "4.1"-"4.3": in prefill the routed experts of thousands of tokens cover
// almost the whole layer, so the next layer's complete expert pool is copied into a
// second layer-sized buffer while this layer computes (T_layer ~ max(T_compute,
// T_PCIe)); the two buffers come from the slot pool.  [jjl357] "6.8" / [wanger]
// "代码全链路": experts run as grouped GPU execution.
//
// Steps (all on the compute stream, fixed grids, no host synchronisation):
//   1. count:   one workgroup per expert counts its routes (ballots; 4 wave quarters).
//   2. plan:    one workgroup: row offsets per expert (exclusive scan), the M-tile
//               offsets (64-row tiles per expert) and the expert of every M tile.
//   3. scatter: one workgroup per expert writes its routes' indices r = t*k + j in
//               (t, j) order — a stable counting sort — into perm.
//   4. gate_up: grouped GEMM, tile = (expert, 64 sorted rows, 128 intermediate
//               columns).  Four waves share the gathered activation tile in LDS;
//               each wave owns 32 gate and the matching 32 up columns and reads its
//               MXFP4 weights straight from memory into MFMA operand registers,
//               dequantising to bf16 (exact).  K is visited in 128-element steps;
//               the MFMA's K order is permuted so a lane consumes one whole 32-element
//               MX block (16 B + 1 scale byte) per row per step.  bf16 MFMA 16x16x32,
//               fp32 accumulation; epilogue h = silu(g) * u, stored as fp16.
//   5. down:    grouped GEMM of h (fp16, rows contiguous per expert) against W_down
//               dequantised to fp16 (exact for block exponents in [-23, 13]), fp16
//               MFMA 16x16x32; epilogue writes w_r * Y into the route's own row of a
//               [T*k][H] fp32 buffer (no atomics).
//   6. combine: y[t] = bf16_rne(sum_j Yr[t*k + j]) in route order — one rounding.
// Tiles are enumerated expert-major, then column block, then row tile, and the
// block id is remapped so consecutive tiles run on the same XCD (its L2 holds the
// expert's weights and activation rows while they are reused).
#include "mc_common.h"

namespace mc {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kP_BM = 64;          // rows per tile
constexpr int kP_KS = 128;         // K per pipeline step
constexpr int kP_Threads = 256;
constexpr int kP_GU_Cols = 128;    // intermediate columns per gate_up tile (32 per wave)
constexpr int kP_DN_Cols = 256;    // output columns per down tile (64 per wave)
constexpr int kP_LdsRow = kP_KS + 8;   // padded LDS row (elements)
constexpr int kP_MaxE = 1024;
constexpr int kP_MaxK = 8192;      // largest H or I (sizes the generic kernel's scale table)

// Status bits of a prefill call (the workspace's first word, cleared by the call's first
// kernel): an h value beyond the fp16 range (it became +-inf in the down GEMM's input).
constexpr uint32_t kStatusHOverflow = 1u;

struct PrefillWs {
  uint32_t* status;     // [1] kStatus* bits of the last call
  int32_t* counts;      // [E]
  int32_t* counts4;     // [E][4] per-wave counts
  int32_t* offsets;     // [E+1]
  int32_t* mtile_off;   // [E+1]
  int32_t* tile_e;      // [T*k/BM + E]: expert of each M tile
  int32_t* perm;        // [T*k]
  _Float16* h;          // [T*k][I]
  float* yr;            // [T*k][H]
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// bound on the M tiles of a call: sum over experts of ceil(n_e / BM) <= T*k / BM + E
__host__ __device__ inline int max_mtiles(int T, int k, int E) { return (T * k) / kP_BM + E; }

static size_t ws_layout(int T, int k, int E, int H, int I, PrefillWs* w, uint8_t* base) {
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return base ? base + at : nullptr;
  };
  const size_t nr = (size_t)T * k;
  uint8_t* p;
  p = take(sizeof(uint32_t));
  if (w) w->status = (uint32_t*)p;
  p = take((size_t)E * 4);
  if (w) w->counts = (int32_t*)p;
  p = take((size_t)E * 16);
  if (w) w->counts4 = (int32_t*)p;
  p = take((size_t)(E + 1) * 4);
  if (w) w->offsets = (int32_t*)p;
  p = take((size_t)(E + 1) * 4);
  if (w) w->mtile_off = (int32_t*)p;
  p = take((size_t)max_mtiles(T, k, E) * 4);
  if (w) w->tile_e = (int32_t*)p;
  p = take(nr * 4);
  if (w) w->perm = (int32_t*)p;
  p = take(nr * (size_t)I * 2);
  if (w) w->h = (_Float16*)p;
  p = take(nr * (size_t)H * 4);
  if (w) w->yr = (float*)p;
  return o;
}

// ---------------------------------------------------------------- sort

__device__ __forceinline__ int route_count(const int32_t* n_tok, int T, int k) {
  const int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  return nt * k;
}

// Routes a wave reads per batch, in 64-route groups: every id load of a batch is issued
// before the first compare, so a wave waits once per batch instead of once per group.
constexpr int kSortBatch = 8;

// 1. per-expert route counts, per wave quarter (ballot + popcount, no atomics)
__global__ void __launch_bounds__(256)
sort_count_kernel(const int32_t* __restrict__ ids, int T, int k, const int32_t* __restrict__ n_tok,
                  int E, int32_t* __restrict__ counts, int32_t* __restrict__ counts4,
                  uint32_t* __restrict__ status) {
  if (status && blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;
  const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nr = route_count(n_tok, T, k);
  const int q = (nr + 3) / 4, r0 = wave * q, r1 = min(nr, r0 + q);
  int c = 0;
  for (int base = r0; base < r1; base += 64 * kSortBatch) {
    int v[kSortBatch];                       // a batch of ids in flight before the first compare
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) {
      const int r = base + 64 * u + lane;
      v[u] = r < r1 ? ids[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) c += __popcll(__ballot(v[u] == e));
  }
  __shared__ int s_c[4];
  if (lane == 0) {
    s_c[wave] = c;
    counts4[e * 4 + wave] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) counts[e] = s_c[0] + s_c[1] + s_c[2] + s_c[3];
}

// 2. offsets and the M-tile table (one workgroup, E <= 1024)
__global__ void __launch_bounds__(1024)
sort_plan_kernel(int E, const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ mtile_off, int32_t* __restrict__ tile_e) {
  __shared__ int s_a[kP_MaxE], s_b[kP_MaxE];
  const int tid = threadIdx.x;
  const int c = tid < E ? counts[tid] : 0;
  s_a[tid] = c;
  s_b[tid] = (c + kP_BM - 1) / kP_BM;
  __syncthreads();
  // Hillis-Steele inclusive scans
  for (int o = 1; o < kP_MaxE; o <<= 1) {
    int va = tid >= o ? s_a[tid - o] : 0;
    int vb = tid >= o ? s_b[tid - o] : 0;
    __syncthreads();
    s_a[tid] += va;
    s_b[tid] += vb;
    __syncthreads();
  }
  if (tid < E) {
    offsets[tid + 1] = s_a[tid];
    mtile_off[tid + 1] = s_b[tid];
  }
  if (tid == 0) {
    offsets[0] = 0;
    mtile_off[0] = 0;
  }
  // expert of every M tile (the first e whose inclusive tile count exceeds j), so a GEMM
  // workgroup finds its tile with one table read instead of a search over mtile_off
  if (tile_e) {
    const int n_mt = s_b[E - 1];
    for (int j = tid; j < n_mt; j += blockDim.x) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_b[mid] > j) hi = mid;
        else lo = mid + 1;
      }
      tile_e[j] = lo;
    }
  }
}

// 3. stable scatter: routes of expert e in (t, j) order
__global__ void __launch_bounds__(256)
sort_scatter_kernel(const int32_t* __restrict__ ids, int T, int k, const int32_t* __restrict__ n_tok,
                    int E, const int32_t* __restrict__ counts4, const int32_t* __restrict__ offsets,
                    int32_t* __restrict__ perm) {
  const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nr = route_count(n_tok, T, k);
  const int q = (nr + 3) / 4, r0 = wave * q, r1 = min(nr, r0 + q);
  int pos = offsets[e];
  for (int w = 0; w < wave; ++w) pos += counts4[e * 4 + w];
  for (int base = r0; base < r1; base += 64 * kSortBatch) {
    int v[kSortBatch];
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) {
      const int r = base + 64 * u + lane;
      v[u] = r < r1 ? ids[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) {              // groups in route order: stable
      const bool hit = v[u] == e;
      const uint64_t m = __ballot(hit);
      if (hit) perm[pos + __popcll(m & ((1ull << lane) - 1ull))] = base + 64 * u + lane;
      pos += __popcll(m);
    }
  }
}

// ---------------------------------------------------------------- GEMM helpers

struct PrefillArgs {
  const uint16_t* x;          // [T][H] bf16
  const float* w;             // [T*k]
  int32_t T, k, E, H, I;
  const uint8_t* gu;          // layer buffer banks (entry e = expert e)
  const uint8_t* gus;
  const uint8_t* dn;
  const uint8_t* dns;
  PrefillWs ws;
  int32_t n_nb;               // column blocks per expert
  const int32_t* entry_of;    // [E] buffer entry of expert e (-1: not in this part), or null = e
};

// Tile of logical id L: expert, row range, column block.  Returns false if L is past
// the last tile of this call.
__device__ __forceinline__ bool find_tile(const PrefillArgs& a, int L, int* e_out, int* row0,
                                          int* nrows, int* nb) {
  const int32_t* mo = a.ws.mtile_off;
  // tiles run expert-major, so tile L belongs to M tile L / n_nb's expert (mo[e] * n_nb <= L
  // < mo[e + 1] * n_nb exactly when mo[e] <= L / n_nb < mo[e + 1]); both reads are issued
  // together, the table index clamped into the table
  const int j = min(L / a.n_nb, max_mtiles(a.T, a.k, a.E) - 1);
  const int total = mo[a.E] * a.n_nb;
  const int e = a.ws.tile_e[j];
  if (L >= total) return false;
  const int m_e = mo[e + 1] - mo[e];
  const int Lp = L - mo[e] * a.n_nb;
  *nb = Lp / m_e;
  const int mt = Lp % m_e;
  const int start = a.ws.offsets[e] + mt * kP_BM;
  *row0 = start;
  *nrows = min(kP_BM, a.ws.offsets[e + 1] - start);
  *e_out = e;
  return true;
}

// Consecutive logical tiles on the same XCD: hardware block b runs on XCD b % 8.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int per = G >> 3;
  return (b & 7) * per + (b >> 3);
}

// 8 consecutive MXFP4 elements (one dword of codes) -> f16x8, scaled.
__device__ __forceinline__ f16x8_t fp4x8_f16(uint32_t v, float s) {
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, s, 0);
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, s, 1);
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, s, 2);
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, s, 3);
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}


// ---------------------------------------------------------------- grouped GEMM
//
// One kernel template for both GEMMs.  Block = 4 waves = 64 sorted rows x 4 x 64 weight
// rows; K in steps of 128.  Pipeline: the activation tile of step s+2 and the weight
// operands of step s+2 are loaded into registers while step s computes; the tile of
// step s+1 (loaded one step earlier) is then written to the other half of an LDS
// double buffer.  The LDS tile is XOR-swizzled (16-byte chunk c of row r lives at
// c ^ (r & 15)) so the 16 rows an MFMA operand read touches fall in different banks.
// For the real shapes the K loop is fully unrolled so every register ring index is
// static and the compiler's wait counts stay exact.

constexpr int kP_StageBytes = kP_BM * kP_KS * 2;     // 16 KiB per activation tile

struct GemmStage {
  u32x4_t b[4];       // one MX block (16 B) per column tile
  uint32_t s[4];      // its scale byte
};

// Block scale table in LDS: the 256 weight rows of a block x (K / 32) e8m0 bytes, one
// dword per K step (its 4 MX blocks).  Row stride kScaleRow(NSTEPS) bytes; the 16-byte
// chunk c of row r is stored at chunk c ^ (r % 16 * stride / 256), so the 16 rows one
// scale read touches land in distinct banks.
__host__ __device__ constexpr int scale_row_bytes(int nsteps_fixed) {
  return nsteps_fixed > 0 ? nsteps_fixed * 4 : kP_MaxK / 32;
}

// One tile of MT 16-row slices (MT = 4 for a full 64-row tile; a tile of fewer rows takes
// the smallest MT that covers them, so no product runs on 16 rows of padding).
template <int MODE, int NSTEPS, int MT>   // MODE 0: gate_up (bf16, SwiGLU), 1: down (fp16, gated rows)
__device__ __forceinline__ void gemm_tile(const PrefillArgs& a, int e, int eb, int row0, int nrows, int nb,
                                          uint8_t (*sA)[kP_StageBytes], uint8_t* sS, int* s_shift) {
  constexpr int SROW = scale_row_bytes(NSTEPS);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I;
  const int K = MODE == 0 ? H : I;
  const int nsteps = NSTEPS > 0 ? NSTEPS : K / kP_KS;

  // the activation chunks this thread moves per step: slot i of the tile holds row
  // i / 16, logical chunk (i % 16) ^ (row % 16); chunk q covers rows 16 q .. 16 q + 15,
  // so the MT slices need chunks q < MT
  // gate_up's activation rows come from perm: its reads go out first, and the row
  // addresses are formed after the first weight loads are issued (a wait for an earlier
  // load waits for everything issued before it)
  const uint16_t* aptr[MT];
  int aslot[MT];
  int prow[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    const int rr = min((tid + kP_Threads * q) >> 4, nrows - 1);
    prow[q] = MODE == 0 ? a.ws.perm[row0 + rr] : 0;
  }
  // weight rows of the lane's 4 column tiles; srow_g = scales of table row tid
  const uint8_t* brow[4];
  const uint8_t* srow_g;
  int c0;
  {
    const size_t row_b = (size_t)K / 2, row_s = (size_t)K / 32;
    const uint8_t* wbase;
    const uint8_t* sbase;
    if (MODE == 0) {
      wbase = a.gu + (size_t)eb * (2 * (size_t)I * row_b);
      sbase = a.gus + (size_t)eb * (2 * (size_t)I * row_s);
      c0 = nb * kP_GU_Cols + wave * 32;
    } else {
      wbase = a.dn + (size_t)eb * ((size_t)H * row_b);
      sbase = a.dns + (size_t)eb * ((size_t)H * row_s);
      c0 = nb * kP_DN_Cols + wave * 64;
    }
    // table row tid = wave * 64 + nt * 16 + r holds the scales of weight row wrow(nt, r)
    auto wrow = [&](int nt, int r) {
      return MODE == 0 ? (nt < 2 ? 0 : I) + c0 + (nt & 1) * 16 + r : c0 + nt * 16 + r;
    };
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) brow[nt] = wbase + (size_t)wrow(nt, lane & 15) * row_b;
    srow_g = sbase + (size_t)wrow((tid >> 4) & 3, tid & 15) * row_s;
  }
  const int kq = lane >> 4;                             // MX block of the step this lane owns

  f32x4_t acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // register rings: three weight stages (loaded two steps ahead) and three activation
  // tiles (loaded three steps ahead); named, so that every index is static and nothing
  // is placed in scratch memory
  GemmStage st0, st1, st2;
  u32x4_t ar0[MT], ar1[MT], ar2[MT];
  int shf[4] = {0, 0, 0, 0};                     // down: the shift of the lane's 4 weight rows
  auto issue_a = [&](int s, u32x4_t* ar) {
    const int k0 = s * kP_KS;
#pragma unroll
    for (int q = 0; q < MT; ++q) ar[q] = *reinterpret_cast<const u32x4_t*>(aptr[q] + k0);
  };
  auto issue_w = [&](int s, GemmStage& g) {
    const int kb = ((s * kP_KS) >> 5) + kq;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) g.b[nt] = *reinterpret_cast<const u32x4_t*>(brow[nt] + (size_t)kb * 16);
  };
  // scale byte of step s for the lane's 4 column tiles, from the LDS table
  const int sw = ((lane & 15) * SROW) >> 8;
  auto scales = [&](int s, GemmStage& g) {
    const int off = (((s >> 2) ^ sw) << 4) + ((s & 3) << 2) + kq;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) g.s[nt] = sS[(wave * 64 + nt * 16 + (lane & 15)) * SROW + off];
  };
  auto store_a = [&](const u32x4_t* ar, int buf) {
#pragma unroll
    for (int q = 0; q < MT; ++q) *reinterpret_cast<u32x4_t*>(&sA[buf][aslot[q]]) = ar[q];
  };
  auto compute = [&](const GemmStage& g, int buf) {
    float sc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      // the empty asm anchors the scale decode here: hoisted next to its load it
      // would wait for that load within the step that issued it
      uint32_t raw = g.s[nt];
      asm volatile("" : "+v"(raw));
      sc[nt] = MODE == 0 ? e8m0_to_f32(raw) : ldexpf(1.0f, (int)raw - 127 - shf[nt]);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int phys = (kq * 4 + ks) ^ (lane & 15);
      if (MODE == 0) {
        bf16x8_t bop[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bop[nt] = fp4x8_bf16(g.b[nt][ks], sc[nt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8_t aop = *reinterpret_cast<const bf16x8_t*>(
              &sA[buf][(mt * 16 + (lane & 15)) * 256 + phys * 16]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[nt], acc[mt][nt], 0, 0, 0);
        }
      } else {
        f16x8_t bop[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bop[nt] = fp4x8_f16(g.b[nt][ks], sc[nt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f16x8_t aop = *reinterpret_cast<const f16x8_t*>(
              &sA[buf][(mt * 16 + (lane & 15)) * 256 + phys * 16]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
  };
  // step s: load the activation tile of step s+3 (ar_ld) and the weights of step s+2
  // (g2), compute step s (g, LDS half s & 1), then publish the tile of step s+1 (ar_st,
  // loaded two steps earlier) to the other half
  auto step = [&](int s, GemmStage& g, GemmStage& g2, u32x4_t* ar_ld, const u32x4_t* ar_st) {
    if (s >= nsteps) return;
    if (s + 3 < nsteps) issue_a(s + 3, ar_ld);
    if (s + 2 < nsteps) {
      issue_w(s + 2, g2);
      scales(s + 2, g2);
    }
    // keep the loads ahead of this step's MFMAs (the scheduler would sink them)
    __builtin_amdgcn_sched_barrier(0);
    compute(g, s & 1);
    if (s + 1 < nsteps) store_a(ar_st, (s & 1) ^ 1);
    __syncthreads();
  };
  // one period of the rings (3 steps): weight stage s % 3, activation tile s % 3
  auto period = [&](int s0) {
    step(s0 + 0, st0, st2, ar0, ar1);
    step(s0 + 1, st1, st0, ar1, ar2);
    step(s0 + 2, st2, st1, ar2, ar0);
  };

  // prologue, in issue order: the weights of the first two steps (they depend on the
  // tile only), this thread's row of the scale table (whole, when the step count is fixed),
  // then the activation tiles of three steps (gate_up's rows wait for perm, read first);
  // the scale table's LDS stores come last, since a wait for a load also waits for every
  // load issued before it
  issue_w(0, st0);
  if (nsteps > 1) issue_w(1, st1);
  constexpr int kSC = NSTEPS > 0 && NSTEPS % 4 == 0 ? NSTEPS / 4 : 1;   // 16-B scale chunks held
  u32x4_t sv[kSC];
  if (NSTEPS > 0 && NSTEPS % 4 == 0) {
#pragma unroll
    for (int c = 0; c < kSC; ++c) sv[c] = *reinterpret_cast<const u32x4_t*>(srow_g + c * 16);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    const int i = tid + kP_Threads * q;
    const int r = i >> 4;
    const int c = (i & 15) ^ (r & 15);
    const int rr = min(r, nrows - 1);
    const uint16_t* rowp;
    if (MODE == 0) rowp = a.x + (size_t)(prow[q] / a.k) * H;
    else rowp = reinterpret_cast<const uint16_t*>(a.ws.h) + (size_t)(row0 + rr) * I;
    aptr[q] = rowp + c * 8;
    aslot[q] = i * 16;
  }
  issue_a(0, ar0);
  if (nsteps > 1) issue_a(1, ar1);
  if (nsteps > 2) issue_a(2, ar2);
  {
    uint8_t* dst = sS + tid * SROW;
    const int swt = ((tid & 15) * SROW) >> 8;
    uint32_t xmin = 255, xmax = 0;               // the row's smallest and largest block exponent
    auto minmax4 = [&](uint32_t v) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t x = (v >> (8 * b)) & 0xFFu;
        xmin = min(xmin, x);
        xmax = max(xmax, x);
      }
    };
    auto put16 = [&](int c, const u32x4_t& v) {
      *reinterpret_cast<u32x4_t*>(dst + ((c ^ swt) << 4)) = v;
      if (MODE == 1) {
        minmax4(v[0]);
        minmax4(v[1]);
        minmax4(v[2]);
        minmax4(v[3]);
      }
    };
    if (NSTEPS > 0 && NSTEPS % 4 == 0) {
#pragma unroll
      for (int c = 0; c < kSC; ++c) put16(c, sv[c]);
    } else if ((nsteps & 3) == 0) {
      for (int c = 0; c < (nsteps >> 2); ++c) put16(c, *reinterpret_cast<const u32x4_t*>(srow_g + c * 16));
    } else {
      for (int d = 0; d < nsteps; ++d) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(srow_g + d * 4);
        *reinterpret_cast<uint32_t*>(dst + (((d >> 2) ^ swt) << 4) + ((d & 3) << 2)) = v;
        if (MODE == 1) minmax4(v);
      }
    }
    // fp16 holds e2m1 * 2^e exactly for e in [-23, 13]; a row with a block outside is
    // dequantised at 2^-shift (its largest block at 2^13) and its outputs are scaled
    // back by 2^shift in the epilogue.  Blocks more than 36 binades below the row's
    // largest one then round in fp16; their share of an output is below 2^-32 of the
    // largest block's, under the fp32 accumulation's own rounding.
    if (MODE == 1)
      s_shift[tid] = ((int)xmin - 127 >= -23 && (int)xmax - 127 <= 13) ? 0 : (int)xmax - 140;
  }
  store_a(ar0, 0);
  __syncthreads();
  if (MODE == 1) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) shf[nt] = s_shift[wave * 64 + nt * 16 + (lane & 15)];
  }
  scales(0, st0);
  if (nsteps > 1) scales(1, st1);
  if (NSTEPS > 0) {
#pragma unroll
    for (int s0 = 0; s0 < NSTEPS; s0 += 3) period(s0);
  } else {
    for (int s0 = 0; s0 < nsteps; s0 += 3) period(s0);
  }

  if (MODE == 0) {
    // h = silu(g) * u -> fp16, rows of this tile; a value beyond fp16's range is flagged
    bool h_over = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = mt * 16 + (lane >> 4) * 4 + j;
        if (r >= nrows) continue;
        _Float16* hrow = a.ws.h + (size_t)(row0 + r) * I;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float g = acc[mt][nt][j], u = acc[mt][nt + 2][j];
          const _Float16 hv = (_Float16)(silu(g) * u);
          h_over |= __builtin_isinf((float)hv);
          hrow[c0 + nt * 16 + (lane & 15)] = hv;
        }
      }
    if (__ballot(h_over) && lane == 0) atomicOr(a.ws.status, kStatusHOverflow);
  } else {
    // the route's own output row, scaled by its gate.  Every route and gate of the lane's
    // rows is read before the first store: a gate read after a store to the (float) output
    // rows could not be moved ahead of it, one dependent round trip per row.
    int route[MT][4];
    float g[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = mt * 16 + (lane >> 4) * 4 + j;
        route[mt][j] = a.ws.perm[row0 + min(r, nrows - 1)];
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) g[mt][j] = a.w[route[mt][j]];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = mt * 16 + (lane >> 4) * 4 + j;
        if (r >= nrows) continue;
        float* yrow = a.ws.yr + (size_t)route[mt][j] * H;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          yrow[c0 + nt * 16 + (lane & 15)] = ldexpf(g[mt][j] * acc[mt][nt][j], shf[nt]);
      }
  }
}

template <int MODE, int NSTEPS>
__global__ void __launch_bounds__(kP_Threads, 2)   // two blocks per CU: <= 256 registers per lane
prefill_gemm_kernel(PrefillArgs a) {
  constexpr int SROW = scale_row_bytes(NSTEPS);
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kP_StageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sS[kP_Threads * SROW];
  __shared__ int s_shift[kP_Threads];            // down: power-of-two shift of each weight row
  int e, row0, nrows, nb;
  if (!find_tile(a, xcd_remap(blockIdx.x, gridDim.x), &e, &row0, &nrows, &nb)) return;
  const int eb = a.entry_of ? a.entry_of[e] : e;   // the expert's entry of the layer buffer
  if (eb < 0) return;                              // computed by another part of the layer
  switch ((nrows + 15) >> 4) {                     // workgroup-uniform
    case 1: gemm_tile<MODE, NSTEPS, 1>(a, e, eb, row0, nrows, nb, sA, sS, s_shift); break;
    case 2: gemm_tile<MODE, NSTEPS, 2>(a, e, eb, row0, nrows, nb, sA, sS, s_shift); break;
    case 3: gemm_tile<MODE, NSTEPS, 3>(a, e, eb, row0, nrows, nb, sA, sS, s_shift); break;
    default: gemm_tile<MODE, NSTEPS, 4>(a, e, eb, row0, nrows, nb, sA, sS, s_shift); break;
  }
}

// ---------------------------------------------------------------- combine

// y[t][c] = bf16_rne(sum over valid routes j of Yr[t*k + j][c]), j ascending
constexpr int kCombineMaxK = 8;     // up to this k, a thread's k row reads are in flight together
__global__ void __launch_bounds__(256)
prefill_combine_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int H,
                       const int32_t* __restrict__ n_tok, const float* __restrict__ yr,
                       uint16_t* __restrict__ y) {
  const int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  const int64_t n4 = (int64_t)T * H / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i * 4 / H), c = (int)(i * 4 % H);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < nt && k <= kCombineMaxK) {
      // every route row of the token is read at once (rows of invalid routes too: they
      // lie inside yr and are then skipped), then summed in route order
      int idv[kCombineMaxK];
      float4 v[kCombineMaxK];
#pragma unroll
      for (int j = 0; j < kCombineMaxK; ++j) idv[j] = j < k ? ids[t * k + j] : -1;
#pragma unroll
      for (int j = 0; j < kCombineMaxK; ++j)        // j >= k re-reads row 0 (no branch)
        v[j] = *reinterpret_cast<const float4*>(yr + ((size_t)t * k + (j < k ? j : 0)) * H + c);
#pragma unroll
      for (int j = 0; j < kCombineMaxK; ++j) {
        if (idv[j] < 0 || idv[j] >= E) continue;
        s.x += v[j].x;
        s.y += v[j].y;
        s.z += v[j].z;
        s.w += v[j].w;
      }
    } else if (t < nt) {
      for (int j = 0; j < k; ++j) {
        const int id = ids[t * k + j];
        if (id < 0 || id >= E) continue;
        const float4 v = *reinterpret_cast<const float4*>(yr + ((size_t)t * k + j) * H + c);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(s.x) | ((uint32_t)f32_to_bf16_rne(s.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(s.z) | ((uint32_t)f32_to_bf16_rne(s.w) << 16);
    *reinterpret_cast<uint2*>(y + (size_t)t * H + c) = o;
  }
}

static int sort_launch(const int32_t* ids, int T, int k, const int32_t* n_tok, int E,
                       const PrefillWs& w, hipStream_t s) {
  hipLaunchKernelGGL(sort_count_kernel, dim3(E), dim3(256), 0, s, ids, T, k, n_tok, E, w.counts,
                     w.counts4, w.status);
  hipLaunchKernelGGL(sort_plan_kernel, dim3(1), dim3(1024), 0, s, E, w.counts, w.offsets,
                     w.mtile_off, w.tile_e);
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(E), dim3(256), 0, s, ids, T, k, n_tok, E, w.counts4,
                     w.offsets, w.perm);
  MC_LAUNCH_CHECK();
  return MC_OK;
}

}  // namespace mc

using namespace mc;

extern "C" size_t moe_experts_prefill_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  if (T < 0 || k < 0 || E < 0 || H < 0 || I < 0) return 0;
  return ws_layout(T, k, E, H, I, nullptr, nullptr);
}

extern "C" int mc_prefill_sort_routes(const int32_t* ids, int32_t T, int32_t k,
                                      const int32_t* n_tok, int32_t E, void* ws, size_t ws_bytes,
                                      int32_t* counts, int32_t* offsets, int32_t* perm,
                                      hipStream_t s) {
  clear_error();
  MC_REQUIRE(T >= 0 && k >= 1 && E >= 1 && E <= kP_MaxE, "mc_prefill_sort_routes: T=%d k=%d E=%d",
             T, k, E);
  MC_REQUIRE(ids && ws && counts && offsets && (perm || T == 0), "mc_prefill_sort_routes: NULL pointer");
  MC_REQUIRE(ws_bytes >= (size_t)E * 16 + (size_t)(E + 1) * 4,
             "mc_prefill_sort_routes: workspace too small");
  PrefillWs w{};
  w.counts = counts;
  w.offsets = offsets;
  w.perm = perm;
  w.counts4 = static_cast<int32_t*>(ws);
  w.mtile_off = static_cast<int32_t*>(ws) + (size_t)E * 4;
  return sort_launch(ids, T, k, n_tok, E, w, s);
}

static int check_prefill_args(const char* fn, int32_t T, int32_t k, int32_t E, const mc_banks* buf, size_t ws_bytes,
                              bool need_n) {
  int rc;
  if ((rc = check_banks(buf, fn)) != MC_OK) return rc;
  MC_REQUIRE(buf->fmt == MC_MXFP4, "%s: MXFP4 experts only", fn);
  MC_REQUIRE(T >= 0 && k >= 1 && E >= 1 && E <= kP_MaxE && k <= E, "%s: T=%d k=%d E=%d", fn, T, k, E);
  if (need_n)
    MC_REQUIRE(buf->n >= E, "%s: layer buffer holds %lld < E=%d experts", fn, (long long)buf->n, E);
  const int H = buf->H, I = buf->I;
  MC_REQUIRE(H % kP_DN_Cols == 0 && I % kP_GU_Cols == 0 && H % kP_KS == 0 && I % kP_KS == 0,
             "%s: H=%d must be a multiple of %d and I=%d of %d", fn, H, kP_DN_Cols, I, kP_GU_Cols);
  MC_REQUIRE(H <= kP_MaxK && I <= kP_MaxK, "%s: H=%d and I=%d must be <= %d", fn, H, I, kP_MaxK);
  MC_REQUIRE(ws_bytes >= moe_experts_prefill_ws_bytes(T, k, E, H, I), "%s: workspace %zu < %zu bytes", fn,
             ws_bytes, moe_experts_prefill_ws_bytes(T, k, E, H, I));
  return MC_OK;
}

// The steps of a prefill layer on one workspace: the sort, the grouped GEMMs of the
// experts in `buf` (all of the layer's experts when entry_of is null), the combine.
static int prefill_steps(const void* x_bf16, const int32_t* ids, const float* w, int32_t T, int32_t k,
                         const int32_t* n_tok, int32_t E, const mc_banks* buf, const int32_t* entry_of,
                         int32_t steps, void* ws, int32_t* counts_out, void* y_bf16, hipStream_t s) {
  int rc;
  const int H = buf->H, I = buf->I;
  PrefillWs pw{};
  ws_layout(T, k, E, H, I, &pw, static_cast<uint8_t*>(ws));
  if (steps & MC_PF_SORT) {
    if ((rc = sort_launch(ids, T, k, n_tok, E, pw, s)) != MC_OK) return rc;
    if (counts_out) MC_HIP(hipMemcpyAsync(counts_out, pw.counts, (size_t)E * 4, hipMemcpyDeviceToDevice, s));
  }
  if (steps & MC_PF_EXPERTS) {
    PrefillArgs a{};
    a.x = static_cast<const uint16_t*>(x_bf16);
    a.w = w;
    a.T = T;
    a.k = k;
    a.E = E;
    a.H = H;
    a.I = I;
    a.gu = static_cast<const uint8_t*>(buf->gate_up);
    a.gus = static_cast<const uint8_t*>(buf->gate_up_scale);
    a.dn = static_cast<const uint8_t*>(buf->down);
    a.dns = static_cast<const uint8_t*>(buf->down_scale);
    a.ws = pw;
    a.entry_of = entry_of;
    const int max_mt = max_mtiles(T, k, E);
    a.n_nb = I / kP_GU_Cols;
    int g = max_mt * a.n_nb;
    g = (g + 7) & ~7;
    if (H / kP_KS == 32)
      hipLaunchKernelGGL((prefill_gemm_kernel<0, 32>), dim3(g), dim3(kP_Threads), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_gemm_kernel<0, 0>), dim3(g), dim3(kP_Threads), 0, s, a);
    MC_LAUNCH_CHECK();
    a.n_nb = H / kP_DN_Cols;
    g = max_mt * a.n_nb;
    g = (g + 7) & ~7;
    if (I / kP_KS == 16)
      hipLaunchKernelGGL((prefill_gemm_kernel<1, 16>), dim3(g), dim3(kP_Threads), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_gemm_kernel<1, 0>), dim3(g), dim3(kP_Threads), 0, s, a);
    MC_LAUNCH_CHECK();
  }
  if (steps & MC_PF_COMBINE) {
    const int64_t n4 = (int64_t)T * H / 4;
    int64_t gc = (n4 + 255) / 256;
    if (gc > 8192) gc = 8192;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)gc), dim3(256), 0, s, ids, T, k, E, H, n_tok, pw.yr,
                       static_cast<uint16_t*>(y_bf16));
    MC_LAUNCH_CHECK();
  }
  return MC_OK;
}

extern "C" int moe_experts_prefill(const void* x_bf16, const int32_t* ids, const float* w,
                                   int32_t T, int32_t k, const int32_t* n_tok, int32_t E,
                                   const mc_banks* layer_buf, void* ws, size_t ws_bytes,
                                   void* y_bf16, hipStream_t s, const mc_prefetch* next) {
  clear_error();
  int rc;
  if ((rc = check_prefill_args("moe_experts_prefill", T, k, E, layer_buf, ws_bytes, true)) != MC_OK) return rc;
  MC_REQUIRE(((uintptr_t)x_bf16 | (uintptr_t)ws | (uintptr_t)y_bf16) % 16 == 0,
             "moe_experts_prefill: x, ws and y must be 16-byte aligned");

  // prefetch of the next layer's whole pool on the copy stream (double buffer)
  if (next) {
    MC_REQUIRE(next->host_src && next->dst && next->copy, "moe_experts_prefill: bad prefetch");
    if ((rc = check_banks(next->host_src, "prefetch host_src")) != MC_OK) return rc;
    if ((rc = check_banks(next->dst, "prefetch dst")) != MC_OK) return rc;
    MC_REQUIRE(next->host_src->fmt == next->dst->fmt && next->host_src->H == next->dst->H &&
                   next->host_src->I == next->dst->I,
               "moe_experts_prefill: prefetch source and destination differ");
    MC_REQUIRE(next->first_flat >= 0 && next->first_flat + E <= next->host_src->n && next->dst->n >= E,
               "moe_experts_prefill: prefetch range out of bounds");
    if (next->dst_free) MC_HIP(hipStreamWaitEvent(next->copy, next->dst_free, 0));
    BankBytes bb = bank_bytes(next->dst->fmt, next->dst->H, next->dst->I);
    const size_t nbytes[4] = {bb.gate_up, bb.gate_up_scale, bb.down, bb.down_scale};
    const void* src[4] = {next->host_src->gate_up, next->host_src->gate_up_scale,
                          next->host_src->down, next->host_src->down_scale};
    void* dst[4] = {next->dst->gate_up, next->dst->gate_up_scale, next->dst->down,
                    next->dst->down_scale};
    for (int b = 0; b < 4; ++b) {
      if (nbytes[b] == 0) continue;
      MC_HIP(hipMemcpyAsync(dst[b], static_cast<const uint8_t*>(src[b]) + nbytes[b] * next->first_flat,
                            nbytes[b] * (size_t)E, hipMemcpyHostToDevice, next->copy));
    }
    if (next->done) MC_HIP(hipEventRecord(next->done, next->copy));
  }
  if (T == 0) return MC_OK;
  MC_REQUIRE(x_bf16 && ids && w && ws && y_bf16, "moe_experts_prefill: NULL pointer");
  return prefill_steps(x_bf16, ids, w, T, k, n_tok, E, layer_buf, nullptr, MC_PF_ALL, ws, nullptr, y_bf16, s);
}

extern "C" int moe_experts_prefill_part(const void* x_bf16, const int32_t* ids, const float* w, int32_t T,
                                        int32_t k, const int32_t* n_tok, int32_t E, const mc_banks* part_buf,
                                        const int32_t* entry_of, int32_t steps, void* ws, size_t ws_bytes,
                                        int32_t* counts, void* y_bf16, hipStream_t s) {
  clear_error();
  int rc;
  if ((rc = check_prefill_args("moe_experts_prefill_part", T, k, E, part_buf, ws_bytes, false)) != MC_OK)
    return rc;
  MC_REQUIRE(steps != 0 && (steps & ~MC_PF_ALL) == 0, "moe_experts_prefill_part: steps=0x%x", steps);
  MC_REQUIRE(!(steps & MC_PF_EXPERTS) || entry_of, "moe_experts_prefill_part: the experts step needs entry_of");
  MC_REQUIRE(((uintptr_t)x_bf16 | (uintptr_t)ws | (uintptr_t)y_bf16) % 16 == 0,
             "moe_experts_prefill_part: x, ws and y must be 16-byte aligned");
  if (T == 0) return MC_OK;
  MC_REQUIRE(x_bf16 && ids && w && ws && (y_bf16 || !(steps & MC_PF_COMBINE)),
             "moe_experts_prefill_part: NULL pointer");
  return prefill_steps(x_bf16, ids, w, T, k, n_tok, E, part_buf, entry_of, steps, ws, counts, y_bf16, s);
}

extern "C" int moe_experts_prefill_status(const void* ws, hipStream_t s, uint32_t* status) {
  clear_error();
  MC_REQUIRE(ws && status, "moe_experts_prefill_status: NULL pointer");
  MC_REQUIRE((uintptr_t)ws % 16 == 0, "moe_experts_prefill_status: ws must be 16-byte aligned");
  MC_HIP(hipStreamSynchronize(s));
  PrefillWs pw{};
  ws_layout(0, 1, 1, 0, 0, &pw, const_cast<uint8_t*>(static_cast<const uint8_t*>(ws)));
  uint32_t v = 0;
  MC_HIP(hipMemcpy(&v, pw.status, sizeof v, hipMemcpyDeviceToHost));
  *status = v;
  if (v & kStatusHOverflow) {
    set_error("moe_experts_prefill: an activation h = silu(g) * u exceeded the fp16 range of the down "
              "GEMM's input (the affected outputs are not exact)");
    return MC_EDEVICE;
  }
  return MC_OK;
}
