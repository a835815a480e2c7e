// Copy of filled experts from the pinned host banks into slot banks, shared by the
// fill kernel and the one-token gate_up pass that carries the down-bank copy in its
// own launch.  [jjl357] "6.7" step 3 (the chosen misses go into the victim slots in one
// batch) and "8.4" (one flat id addresses the same expert in every bank).
#pragma once

#include "mc_common.h"

namespace mc {

constexpr int kFillThreads = 256;
// The fill kernel's own workgroups: kFillBlock threads with kFillUnroll 16-byte loads in
// flight each, one 256 KiB chunk per workgroup; the copy groups inside the one-token
// gate_up launch: 256 threads, 32 KiB chunks.  Measured with the fill kernel alone in graph
// replays on a box whose link profiles at 46 GB/s, time per expert beyond an empty call for
// 1 / 2 / 4 / 8 / 62 experts per call: 256 KiB chunks of 1024 threads 33.6 / 31.0 / 30.5 /
// 30.4 / 30.7 µs; 64 KiB chunks of 256 threads 30.9-32.1 / 32.0-32.7 / 35.5-35.9 / 35.7-36.1 /
// 30.7-30.9; 32 KiB chunks 35.7 / 38.7 / 38.6 / 35.8 / 30.7.  The gate_up launch moved the
// same experts at 56-59 GB/s with its 32 KiB copies.
constexpr int kFillUnroll = 16;
constexpr int kFillBlock = 1024;
constexpr int kFusedCopyUnroll = 8;

// The banks one copy covers: chunk c of an entry lies in bank `seg` where
// chunk0[seg] <= c < chunk0[seg + 1]; a bank left out has bytes 0 and no chunks.
struct FillSegs {
  const uint8_t* src[4];     // host (device-visible) bank bases
  uint8_t* dst[4];           // slot bank bases
  int64_t bytes[4];          // bytes per expert entry of each bank
  int32_t chunk0[5];         // first chunk index of each bank; chunk0[4] = chunks per entry
  int64_t n_src, n_dst;
};

// Chunk c (of chunk0[4], chunks of NTH * UNROLL * 16 bytes) of host entry f into slot s, by
// a group of NTH threads: every load of the chunk is issued before the first store.
// Entries outside the banks are skipped.
template <int UNROLL, int NTH = kFillThreads>
__device__ __forceinline__ void fill_chunk(const FillSegs& g, int64_t f, int64_t s, int c) {
  constexpr int kFillChunk = NTH * UNROLL * 16;
  if (f < 0 || f >= g.n_src || s < 0 || s >= g.n_dst) return;
  int seg = 0;
#pragma unroll
  for (int b = 1; b < 4; ++b)
    if (c >= g.chunk0[b]) seg = b;
  if (c >= g.chunk0[4] || g.bytes[seg] == 0) return;
  const int64_t nb = g.bytes[seg];
  const int64_t off0 = (int64_t)(c - g.chunk0[seg]) * kFillChunk;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(g.src[seg] + f * nb + off0);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(g.dst[seg] + s * nb + off0);
  const int64_t n16 = min((int64_t)kFillChunk, nb - off0) / 16;
  const int tid = threadIdx.x % NTH;
  // every load is issued (indexes past the chunk's end re-read its last word), so all
  // of them are in flight together; only the stores are conditional
  u32x4_t v[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int j = tid + u * NTH;
    v[u] = __builtin_nontemporal_load(src + min((int64_t)j, n16 - 1));
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int j = tid + u * NTH;
    if (j < n16) dst[j] = v[u];
  }
}

// Host side: the segments of a copy of the banks in `banks` (MC_BANK_* mask) from the
// pinned host banks into the pool banks in chunks of chunk_bytes, and the chunks per entry
// (0 if no bank has bytes).  Checks both descriptors and the host banks' pinning; MC_OK
// or an error with its message set.
int fill_segs(const mc_banks* host, const mc_banks* pool, uint32_t banks, int64_t chunk_bytes, const char* fn,
              hipStream_t s, FillSegs* g, int* chunks);
// Host side: the fill kernel over list entries [0, min(*n_fill, kcap)) with segments g
// (nothing when g has no chunks or kcap is 0).
int launch_fill(const FillSegs& g, const int32_t* fill_flat, const int32_t* fill_slot, const int32_t* n_fill,
                int32_t kcap, hipStream_t s);

}  // namespace mc
