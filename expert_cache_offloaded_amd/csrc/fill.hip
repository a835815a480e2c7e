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
#include <cstdio>
#include <mutex>

#include "fill_dev.h"

namespace mc {

__global__ void __launch_bounds__(kFillBlock)
fill_kernel(FillSegs g, const int32_t* __restrict__ fill_flat, const int32_t* __restrict__ fill_slot,
            const int32_t* __restrict__ n_fill) {
  const int i = blockIdx.y;
  if (i >= *n_fill) return;
  fill_chunk<kFillUnroll, kFillBlock>(g, fill_flat[i], fill_slot[i], blockIdx.x);
}

int launch_fill(const FillSegs& g, const int32_t* fill_flat, const int32_t* fill_slot, const int32_t* n_fill,
                int32_t kcap, hipStream_t s) {
  if (kcap == 0 || g.chunk0[4] == 0) return MC_OK;
  hipLaunchKernelGGL(fill_kernel, dim3(g.chunk0[4], kcap), dim3(kFillBlock), 0, s, g, fill_flat, fill_slot,
                     n_fill);
  MC_LAUNCH_CHECK();
  return MC_OK;
}

int fill_segs(const mc_banks* host, const mc_banks* pool, uint32_t banks, int64_t chunk_bytes, const char* fn,
              hipStream_t s, FillSegs* g, int* chunks) {
  MC_REQUIRE(banks != 0 && (banks & ~(uint32_t)MC_BANK_ALL) == 0, "%s: bank mask 0x%x", fn, banks);
  char what_host[96], what_pool[96];
  snprintf(what_host, sizeof what_host, "%s host", fn);
  snprintf(what_pool, sizeof what_pool, "%s pool", fn);
  int rc;
  if ((rc = check_banks(host, what_host)) != MC_OK) return rc;
  if ((rc = check_banks(pool, what_pool)) != MC_OK) return rc;
  MC_REQUIRE(host->fmt == pool->fmt && host->H == pool->H && host->I == pool->I,
             "%s: host and pool banks differ in format or shape", fn);
  BankBytes bb = bank_bytes(host->fmt, host->H, host->I);
  *g = FillSegs{};
  const void* hs[4] = {host->gate_up, host->gate_up_scale, host->down, host->down_scale};
  void* ds[4] = {pool->gate_up, pool->gate_up_scale, pool->down, pool->down_scale};
  int64_t nbytes[4] = {(int64_t)bb.gate_up, (int64_t)bb.gate_up_scale, (int64_t)bb.down,
                       (int64_t)bb.down_scale};
  int n = 0;
  for (int b = 0; b < 4; ++b) {
    g->chunk0[b] = n;
    g->bytes[b] = (banks >> b) & 1u ? nbytes[b] : 0;    // banks left out get no chunks
    if (g->bytes[b] == 0) continue;
    MC_REQUIRE(nbytes[b] % 16 == 0, "%s: bank %d entry is not a multiple of 16 bytes", fn, b);
    if ((rc = host_device_view(hs[b], &g->src[b], what_host, s)) != MC_OK) return rc;
    g->dst[b] = static_cast<uint8_t*>(ds[b]);
    n += (int)((nbytes[b] + chunk_bytes - 1) / chunk_bytes);
  }
  g->chunk0[4] = n;
  g->n_src = host->n;
  g->n_dst = pool->n;
  *chunks = n;
  return MC_OK;
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
  MC_REQUIRE(kcap >= 0 && kcap <= 65535, "mc_fill_slots: kcap=%d (0..65535)", kcap);
  MC_REQUIRE(fill_flat && fill_slot && n_fill, "mc_fill_slots: NULL list pointer");
  FillSegs g;
  int chunks = 0, rc;
  if ((rc = fill_segs(host, pool, banks, (int64_t)kFillBlock * kFillUnroll * 16, "mc_fill_slots", s, &g,
                      &chunks)) != MC_OK)
    return rc;
  return launch_fill(g, fill_flat, fill_slot, n_fill, kcap, s);
}

extern "C" int mc_host_forget(const void* p, size_t bytes) {
  clear_error();
  MC_REQUIRE(p != nullptr, "mc_host_forget: NULL pointer");
  return host_forget(p, bytes);
}
