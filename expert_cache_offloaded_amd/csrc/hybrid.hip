// hybrid_split_merge: exact split of one decode layer between GPU and host, and merge.
//
// [jjl357] "6.2 每个 miss 有两条精确执行路径": M = F (filled, run on the GPU) and
// C (run in place on the CPU); the router's ids and gates are unchanged.
// [jjl357] "6.8 CPU 与 GPU 并发执行的顺序": the CPU branch is started first; the GPU
// meanwhile updates cache metadata, copies the fills and runs hits + fills; the CPU
// writes its partial to pinned memory and the two are merged.
// [wanger] "代码全链路" / [juhe] "为什么可以直接相加": GPU routes are marked -1 for the
// host kernel and host routes get gate 0 on the GPU, so every route is computed once;
// y = y_gpu + y_host.
//
// No host function sits in the stream: the split kernel writes the host branch's
// inputs into the pinned stage and raises the stage's request number; a dispatcher
// thread of the worker pool sees it, runs the host experts and raises the completion
// number; the merge kernel waits (bounded) for that number and reads the host partial
// straight from the stage.  So the GPU goes on with fills and moe_experts_decode while
// the host computes, and the whole layer can be captured in a hipGraph.  The stage is
// fine-grained pinned memory (mc_hybrid_stage_alloc), whose accesses from the GPU and
// the host are coherent; its layout is in hybrid_stage.h.
#include <string.h>

#include "hybrid_stage.h"
#include "mc_common.h"

namespace mc {

constexpr int kSplitThreads = 1024;
constexpr int kMergeSpinPolls = 1 << 21;     // a merge wait gives up after this many polls

// gpu_w / host_ids (device): complementary masks of the valid routes.  The host branch's
// inputs go to the stage (x, host ids, gates, valid count, layer); then, once every
// store has reached memory, the request number moves on.  One workgroup.
__global__ void __launch_bounds__(kSplitThreads)
split_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ slots,
             const float* __restrict__ w, const uint16_t* __restrict__ x, int T, int k, int E, int H,
             int layer, const int32_t* __restrict__ n_tok, float* __restrict__ gpu_w,
             int32_t* __restrict__ host_ids, uint8_t* __restrict__ stage, StageHeader hd) {
  const int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  int any_host = 0;
  for (int r = threadIdx.x; r < T * k; r += kSplitThreads) {
    const bool valid = r / k < nt;
    const int id = ids[r];
    const int slot = slots[r];
    const bool on_gpu = valid && slot >= 0;
    const bool on_host = valid && slot < 0 && id >= 0 && id < E;
    gpu_w[r] = on_gpu ? w[r] : 0.0f;
    host_ids[r] = on_host ? id : -1;
    any_host |= on_host;
  }
  // a call with no host route leaves the stage alone (its merge does not wait either)
  if (!__syncthreads_or(any_host)) return;
  int32_t* st_ids = reinterpret_cast<int32_t*>(stage + hd.off_ids);
  float* st_w = reinterpret_cast<float*>(stage + hd.off_w);
  for (int r = threadIdx.x; r < T * k; r += kSplitThreads) {
    st_ids[r] = host_ids[r];
    st_w[r] = w[r];
  }
  const uint4* xs = reinterpret_cast<const uint4*>(x);
  uint4* xd = reinterpret_cast<uint4*>(stage + hd.off_x);
  for (int i = threadIdx.x; i < nt * H / 8; i += kSplitThreads) xd[i] = xs[i];
  StageReq* req = reinterpret_cast<StageReq*>(stage + hd.off_req);
  if (threadIdx.x == 0) {
    req->layer = layer;
    req->ntok = nt;
  }
  __threadfence_system();                   // this thread's stores are in host memory
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t seq = __hip_atomic_load(&req->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) + 1;
    __hip_atomic_store(&req->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// If the call has host routes, waits until the host branch has completed it (thread 0
// of each workgroup polls the completion number; bounded: a wait that runs out counts
// in req.err and the output is then wrong); then y_bf16 = bf16_rne(y_acc + y_host): one rounding of
// the summed fp32 partials; the host partial is also copied to y_host (device).
__global__ void merge_kernel(const float* __restrict__ y_acc, float* __restrict__ y_host, int T, int k, int H,
                             const int32_t* __restrict__ n_tok, const int32_t* __restrict__ host_ids,
                             uint16_t* __restrict__ out, uint8_t* __restrict__ stage, StageHeader hd) {
  StageReq* req = reinterpret_cast<StageReq*>(stage + hd.off_req);
  const StageDone* done = reinterpret_cast<const StageDone*>(stage + hd.off_done);
  int mine = 0;
  for (int r = threadIdx.x; r < T * k; r += blockDim.x) mine |= host_ids[r] >= 0;
  const bool any_host = __syncthreads_or(mine);    // the split rang the stage only then
  if (any_host && threadIdx.x == 0) {
    const uint64_t want = __hip_atomic_load(&req->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    int ok = 0;
    for (int polls = 0; polls < kMergeSpinPolls; ++polls) {
      if (__hip_atomic_load(&done->seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) >= want) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    if (!ok && blockIdx.x == 0) __hip_atomic_fetch_add(&req->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  __syncthreads();
  if (any_host) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");   // system scope: the host's stores to y
  const float* yh = reinterpret_cast<const float*>(stage + hd.off_y);
  const int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  const int64_t n = (int64_t)T * H;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool valid = (i / H) < nt;
    const float h = valid && any_host ? yh[i] : 0.0f;
    y_host[i] = h;
    out[i] = valid ? f32_to_bf16_rne(y_acc[i] + h) : (uint16_t)0;
  }
}

static unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace mc

using namespace mc;

extern "C" size_t mc_hybrid_stage_bytes(int32_t T, int32_t k, int32_t H) {
  if (T < 0 || k < 0 || H < 0) return 0;
  StageHeader h{};
  size_t total = 0;
  stage_layout(T, k, H, &h, &total);
  return total;
}

extern "C" void* mc_hybrid_stage_alloc(size_t bytes) {
  clear_error();
  if (bytes == 0) {
    set_error("mc_hybrid_stage_alloc: 0 bytes");
    return nullptr;
  }
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocCoherent | hipHostMallocMapped);
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    set_error("mc_hybrid_stage_alloc: hipHostMalloc of %zu bytes failed (%s)", bytes, hipGetErrorString(e));
    return nullptr;
  }
  memset(p, 0, bytes);
  return p;
}

extern "C" uint32_t mc_hybrid_stage_errors(const void* stage) {
  if (!stage) return 0;
  const StageHeader* h = static_cast<const StageHeader*>(stage);
  if (h->magic != kStageMagic) return 0;
  const StageReq* req = reinterpret_cast<const StageReq*>(static_cast<const uint8_t*>(stage) + h->off_req);
  return __atomic_load_n(&req->err, __ATOMIC_ACQUIRE);
}

extern "C" int mc_hybrid_stage_free(void* stage) {
  clear_error();
  if (!stage) return MC_OK;
  MC_HIP(hipDeviceSynchronize());            // no kernel may still read or write it
  host_pool_drop_stage(static_cast<StageHeader*>(stage));
  host_forget(stage, 1);
  // the header is cleared first: the pages may come back from a later pinned allocation,
  // which must not look like a stage already set up
  static_cast<StageHeader*>(stage)->magic = 0;
  MC_HIP(hipHostFree(stage));
  return MC_OK;
}

extern "C" int hybrid_split_merge(const mc_hybrid* hy, int32_t phase, hipStream_t s) {
  clear_error();
  MC_REQUIRE(hy != nullptr, "hybrid_split_merge: NULL descriptor");
  MC_REQUIRE(phase == MC_SPLIT_SUBMIT || phase == MC_MERGE, "hybrid_split_merge: phase=%d", phase);
  MC_REQUIRE(hy->T >= 0 && hy->k >= 1 && hy->E >= 1 && hy->layer >= 0,
             "hybrid_split_merge: T=%d k=%d E=%d layer=%d", hy->T, hy->k, hy->E, hy->layer);
  int rc;
  if ((rc = check_banks(hy->host, "hybrid_split_merge host")) != MC_OK) return rc;
  MC_REQUIRE(hy->pinned_stage != nullptr, "hybrid_split_merge: NULL stage");
  MC_REQUIRE((uintptr_t)hy->pinned_stage % 256 == 0, "hybrid_split_merge: stage must be 256-byte aligned");
  MC_REQUIRE(hy->host->H % 8 == 0, "hybrid_split_merge: H=%d must be a multiple of 8", hy->host->H);
  const int T = hy->T, k = hy->k, H = hy->host->H;
  size_t need = mc_hybrid_stage_bytes(T, k, H);
  if (hy->stage_bytes < need) {
    set_error("hybrid_split_merge: stage %zu < %zu bytes", hy->stage_bytes, need);
    return MC_ENOMEM;
  }
  if (T == 0) return MC_OK;
  StageHeader* h = static_cast<StageHeader*>(hy->pinned_stage);
  uint8_t* base = static_cast<uint8_t*>(hy->pinned_stage);
  const uint8_t* dev_view = nullptr;
  if ((rc = host_device_view(base, &dev_view, "hybrid_split_merge: stage", s)) != MC_OK) return rc;
  uint8_t* stage_dev = const_cast<uint8_t*>(dev_view);

  if (phase == MC_SPLIT_SUBMIT) {
    MC_REQUIRE(hy->x_bf16 && hy->ids_raw && hy->slots && hy->w && hy->gpu_w && hy->host_ids,
               "hybrid_split_merge: NULL pointer (split)");
    MC_REQUIRE(hy->pool != nullptr, "hybrid_split_merge: NULL worker pool");
    MC_REQUIRE((uintptr_t)hy->x_bf16 % 16 == 0, "hybrid_split_merge: x must be 16-byte aligned");
    if (h->magic != kStageMagic) {
      // first use: the stage must be fine-grained (coherent) pinned memory
      unsigned int flags = 0;
      MC_HIP(hipHostGetFlags(&flags, hy->pinned_stage));
      MC_REQUIRE(flags & hipHostMallocCoherent,
                 "hybrid_split_merge: the stage must come from mc_hybrid_stage_alloc (coherent pinned memory)");
      StageHeader nh{};
      size_t total;
      stage_layout(T, k, H, &nh, &total);
      nh.T = T;
      nh.k = k;
      nh.E = hy->E;
      nh.H = H;
      nh.host = *hy->host;
      nh.pool = hy->pool;
      nh.magic = kStageMagic;
      *h = nh;
      host_pool_add_stage(hy->pool, h);
    } else {
      MC_REQUIRE(h->T == T && h->k == k && h->H == H && h->E == hy->E && h->pool == hy->pool &&
                     memcmp(&h->host, hy->host, sizeof(mc_banks)) == 0,
                 "hybrid_split_merge: stage set up for another shape, host pool or worker pool");
    }
    hipLaunchKernelGGL(split_kernel, dim3(1), dim3(kSplitThreads), 0, s, hy->ids_raw, hy->slots, hy->w,
                       static_cast<const uint16_t*>(hy->x_bf16), T, k, hy->E, H, hy->layer, hy->n_tok,
                       hy->gpu_w, hy->host_ids, stage_dev, *h);
    MC_LAUNCH_CHECK();
    return MC_OK;
  }

  MC_REQUIRE(h->magic == kStageMagic && h->T == T && h->k == k && h->H == H,
             "hybrid_split_merge: MERGE without a matching SPLIT_SUBMIT on this stage");
  MC_REQUIRE(hy->y_acc && hy->y_host && hy->y_bf16, "hybrid_split_merge: NULL pointer (merge)");
  MC_REQUIRE(hy->host_ids != nullptr, "hybrid_split_merge: NULL host_ids (merge)");
  hipLaunchKernelGGL(merge_kernel, dim3(grid_for((int64_t)T * H)), dim3(256), 0, s, hy->y_acc,
                     hy->y_host, T, k, H, hy->n_tok, hy->host_ids, static_cast<uint16_t*>(hy->y_bf16),
                     stage_dev, *h);
  MC_LAUNCH_CHECK();
  return MC_OK;
}
