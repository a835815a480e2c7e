// mc_fill_slots: the fill fetch of the decode path.
//
// [jjl357] "6.7" (step 3: the chosen missing experts are copied into the victim
// slots in one batch) and "6.8" (one fused expert batch copy beside the cache
// metadata update).  The copy is a kernel that reads the pinned host banks over
// the host link and writes the slot banks, so the fill list produced on the
// device by slot_cache_lookup_evict drives it directly: no host round trip, and
// the whole decode step can be captured in one hipGraph.
//
// Grid: (chunk of the expert's bytes, list entry).  Every entry copies all banks
// of one expert (one flat id across gate_up / scales / down, [jjl357] "8.4").
// Workgroups whose entry is beyond *n_fill exit at once.  Workgroups are dealt to
// the XCDs in turn, so with the chunk as the fast grid index even a single fill
// is spread over every XCD (with the entry first, one XCD carried it alone: 46
// against 51 GB/s for one 1.67 MB expert).
#include <mutex>

#include "mc_common.h"

namespace mc {

constexpr int kFillThreads = 256;
constexpr int kFillUnroll = 8;                                   // 16-byte loads in flight
constexpr int kFillChunk = kFillThreads * kFillUnroll * 16;      // 32 KiB per workgroup

struct FillSegs {
  const uint8_t* src[4];     // host (device-visible) bank bases
  uint8_t* dst[4];           // slot bank bases
  int64_t bytes[4];          // bytes per expert entry of each bank
  int32_t chunk0[5];         // first chunk index of each bank
  int64_t n_src, n_dst;
};

__global__ void __launch_bounds__(kFillThreads)
fill_kernel(FillSegs g, const int32_t* __restrict__ fill_flat, const int32_t* __restrict__ fill_slot,
            const int32_t* __restrict__ n_fill) {
  const int i = blockIdx.y;
  if (i >= *n_fill) return;
  const int64_t f = fill_flat[i];
  const int64_t s = fill_slot[i];
  if (f < 0 || f >= g.n_src || s < 0 || s >= g.n_dst) return;
  const int c = blockIdx.x;
  int seg = 0;
#pragma unroll
  for (int b = 1; b < 4; ++b)
    if (c >= g.chunk0[b]) seg = b;
  if (c >= g.chunk0[4] || g.bytes[seg] == 0) return;
  const int64_t nb = g.bytes[seg];
  const int64_t off0 = (int64_t)(c - g.chunk0[seg]) * kFillChunk;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = reinterpret_cast<const u32x4*>(g.src[seg] + f * nb + off0);
  u32x4* dst = reinterpret_cast<u32x4*>(g.dst[seg] + s * nb + off0);
  const int64_t n16 = min((int64_t)kFillChunk, nb - off0) / 16;
  u32x4 v[kFillUnroll];
#pragma unroll
  for (int u = 0; u < kFillUnroll; ++u) {
    int64_t j = threadIdx.x + (int64_t)u * kFillThreads;
    if (j < n16) v[u] = __builtin_nontemporal_load(src + j);
  }
#pragma unroll
  for (int u = 0; u < kFillUnroll; ++u) {
    int64_t j = threadIdx.x + (int64_t)u * kFillThreads;
    if (j < n16) dst[j] = v[u];
  }
}

// Device-visible address of pinned host memory.  Outside stream capture every call
// asks the runtime again (so memory that was freed and reused as pageable memory is
// refused); while `s` is being captured the translation remembered from an earlier
// call on the same address is used, so capture needs no runtime query once the banks
// were seen.  mc_host_forget drops remembered translations.
static std::mutex g_view_mu;
static const void* g_view_host[64];
static const uint8_t* g_view_dev[64];
static int g_view_n = 0, g_view_next = 0;

static bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;                 // cannot tell: take the remembered translation, query no more
  }
  return st != hipStreamCaptureStatusNone;
}

int host_device_view(const void* host, const uint8_t** out, const char* what, hipStream_t s) {
  if (host == nullptr) {
    *out = nullptr;
    return MC_OK;
  }
  if (stream_capturing(s)) {
    std::lock_guard<std::mutex> lk(g_view_mu);
    for (int i = 0; i < g_view_n; ++i)
      if (g_view_host[i] == host) {
        *out = g_view_dev[i];
        return MC_OK;
      }
  }
  void* d = nullptr;
  hipError_t e = hipHostGetDevicePointer(&d, const_cast<void*>(host), 0);
  if (e != hipSuccess || d == nullptr) {
    (void)hipGetLastError();
    host_forget(host, 1);
    set_error("%s is not pinned host memory (%s)", what, hipGetErrorString(e));
    return MC_EINVAL;
  }
  *out = static_cast<const uint8_t*>(d);
  std::lock_guard<std::mutex> lk(g_view_mu);
  for (int i = 0; i < g_view_n; ++i)
    if (g_view_host[i] == host) {
      g_view_dev[i] = *out;
      return MC_OK;
    }
  g_view_host[g_view_next] = host;
  g_view_dev[g_view_next] = *out;
  g_view_next = (g_view_next + 1) % 64;
  if (g_view_n < 64) ++g_view_n;
  return MC_OK;
}

int host_forget(const void* p, size_t bytes) {
  const uintptr_t lo = (uintptr_t)p, hi = lo + (bytes ? bytes : 1);
  int dropped = 0;
  std::lock_guard<std::mutex> lk(g_view_mu);
  for (int i = 0; i < g_view_n; ++i) {
    const uintptr_t a = (uintptr_t)g_view_host[i];
    if (a >= lo && a < hi) {
      g_view_host[i] = nullptr;
      g_view_dev[i] = nullptr;
      ++dropped;
    }
  }
  return dropped;
}

}  // namespace mc

using namespace mc;

extern "C" int mc_fill_slots(const mc_banks* host, const mc_banks* pool, const int32_t* fill_flat,
                             const int32_t* fill_slot, const int32_t* n_fill, int32_t kcap,
                             hipStream_t s) {
  return mc_fill_slots_banks(host, pool, fill_flat, fill_slot, n_fill, kcap, MC_BANK_ALL, s);
}

extern "C" int mc_fill_slots_banks(const mc_banks* host, const mc_banks* pool, const int32_t* fill_flat,
                                   const int32_t* fill_slot, const int32_t* n_fill, int32_t kcap,
                                   uint32_t banks, hipStream_t s) {
  clear_error();
  MC_REQUIRE(banks != 0 && (banks & ~(uint32_t)MC_BANK_ALL) == 0, "mc_fill_slots: bank mask 0x%x", banks);
  int rc;
  if ((rc = check_banks(host, "mc_fill_slots host")) != MC_OK) return rc;
  if ((rc = check_banks(pool, "mc_fill_slots pool")) != MC_OK) return rc;
  MC_REQUIRE(host->fmt == pool->fmt && host->H == pool->H && host->I == pool->I,
             "mc_fill_slots: host and pool banks differ in format or shape");
  MC_REQUIRE(kcap >= 0 && kcap <= 65535, "mc_fill_slots: kcap=%d (0..65535)", kcap);
  MC_REQUIRE(fill_flat && fill_slot && n_fill, "mc_fill_slots: NULL list pointer");
  if (kcap == 0) return MC_OK;
  BankBytes bb = bank_bytes(host->fmt, host->H, host->I);
  FillSegs g{};
  const void* hs[4] = {host->gate_up, host->gate_up_scale, host->down, host->down_scale};
  void* ds[4] = {pool->gate_up, pool->gate_up_scale, pool->down, pool->down_scale};
  int64_t nbytes[4] = {(int64_t)bb.gate_up, (int64_t)bb.gate_up_scale, (int64_t)bb.down,
                       (int64_t)bb.down_scale};
  int chunks = 0;
  for (int b = 0; b < 4; ++b) {
    g.chunk0[b] = chunks;
    g.bytes[b] = (banks >> b) & 1u ? nbytes[b] : 0;    // banks left out get no chunks
    if (g.bytes[b] == 0) continue;
    MC_REQUIRE(nbytes[b] % 16 == 0, "mc_fill_slots: bank %d entry is not a multiple of 16 bytes", b);
    if ((rc = host_device_view(hs[b], &g.src[b], "mc_fill_slots: host bank", s)) != MC_OK) return rc;
    g.dst[b] = static_cast<uint8_t*>(ds[b]);
    chunks += (int)((nbytes[b] + kFillChunk - 1) / kFillChunk);
  }
  g.chunk0[4] = chunks;
  g.n_src = host->n;
  g.n_dst = pool->n;
  hipLaunchKernelGGL(fill_kernel, dim3(chunks, kcap), dim3(kFillThreads), 0, s, g, fill_flat,
                     fill_slot, n_fill);
  MC_LAUNCH_CHECK();
  return MC_OK;
}

extern "C" int mc_host_forget(const void* p, size_t bytes) {
  clear_error();
  MC_REQUIRE(p != nullptr, "mc_host_forget: NULL pointer");
  return host_forget(p, bytes);
}
