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
// Stage (caller-owned pinned memory): header | x bf16 [T][H] | host_ids [T][k] |
// w [T][k] | n_tok | y_host fp32 [T][H].  The header is written on the host when the
// split is enqueued; the host function only reads it, so the sequence can be
// captured in a hipGraph and replayed.
#include <string.h>

#include <functional>

#include "mc_common.h"

namespace mc {

int host_experts_run(mc_host_pool* pool, const uint16_t* x, const int32_t* ids, const float* w,
                     int T, int k, int layer, int E, const mc_banks* host, float* y);
void host_pool_submit(mc_host_pool* p, std::function<void()> job);
void host_pool_wait(mc_host_pool* p);

constexpr uint32_t kStageMagic = 0x6d634859u;   // "mcHY"

struct StageHeader {
  uint32_t magic;
  int32_t T, k, layer, E, H;
  mc_banks host;
  mc_host_pool* pool;
  size_t off_x, off_ids, off_w, off_ntok, off_y;
  int32_t has_ntok;
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static void stage_layout(int T, int k, int H, StageHeader* h, size_t* total) {
  size_t o = align256(sizeof(StageHeader));
  h->off_x = o;
  o = align256(o + (size_t)T * H * 2);
  h->off_ids = o;
  o = align256(o + (size_t)T * k * 4);
  h->off_w = o;
  o = align256(o + (size_t)T * k * 4);
  h->off_ntok = o;
  o = align256(o + 4);
  h->off_y = o;
  o = align256(o + (size_t)T * H * 4);
  *total = o;
}

// gpu_w / host_ids: complementary masks of the valid routes.
__global__ void split_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ slots,
                             const float* __restrict__ w, int T, int k, int E,
                             const int32_t* __restrict__ n_tok, float* __restrict__ gpu_w,
                             int32_t* __restrict__ host_ids) {
  const int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < T * k; r += gridDim.x * blockDim.x) {
    const bool valid = r / k < nt;
    const int id = ids[r];
    const int slot = slots[r];
    const bool on_gpu = valid && slot >= 0;
    const bool on_host = valid && slot < 0 && id >= 0 && id < E;
    gpu_w[r] = on_gpu ? w[r] : 0.0f;
    host_ids[r] = on_host ? id : -1;
  }
}

// y_bf16 = bf16_rne(y_acc + y_host): one rounding of the summed fp32 partials.
__global__ void merge_kernel(const float* __restrict__ y_acc, const float* __restrict__ y_host,
                             int T, int H, const int32_t* __restrict__ n_tok,
                             uint16_t* __restrict__ out) {
  const int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  const int64_t n = (int64_t)T * H;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (i / H) < nt ? f32_to_bf16_rne(y_acc[i] + y_host[i]) : (uint16_t)0;
}

// Host function of SPLIT_SUBMIT: start the host branch and return at once.
static void submit_host_branch(void* user) {
  StageHeader* h = static_cast<StageHeader*>(user);
  uint8_t* base = reinterpret_cast<uint8_t*>(h);
  const int nt = h->has_ntok ? *reinterpret_cast<int32_t*>(base + h->off_ntok) : h->T;
  const int ntok = nt < 0 ? 0 : (nt > h->T ? h->T : nt);
  float* y = reinterpret_cast<float*>(base + h->off_y);
  memset(y, 0, sizeof(float) * (size_t)h->T * h->H);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(base + h->off_x);
  const int32_t* ids = reinterpret_cast<const int32_t*>(base + h->off_ids);
  const float* w = reinterpret_cast<const float*>(base + h->off_w);
  host_pool_submit(h->pool, [h, x, ids, w, ntok, y] {
    host_experts_run(h->pool, x, ids, w, ntok, h->k, h->layer, h->E, &h->host, y);
  });
}

// Host function of MERGE: block until the host branch has written its partial.
static void wait_host_branch(void* user) {
  StageHeader* h = static_cast<StageHeader*>(user);
  host_pool_wait(h->pool);
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
  const int T = hy->T, k = hy->k, H = hy->host->H;
  size_t need = mc_hybrid_stage_bytes(T, k, H);
  if (hy->stage_bytes < need) {
    set_error("hybrid_split_merge: stage %zu < %zu bytes", hy->stage_bytes, need);
    return MC_ENOMEM;
  }
  if (T == 0) return MC_OK;
  StageHeader* h = static_cast<StageHeader*>(hy->pinned_stage);
  uint8_t* base = static_cast<uint8_t*>(hy->pinned_stage);

  if (phase == MC_SPLIT_SUBMIT) {
    MC_REQUIRE(hy->x_bf16 && hy->ids_raw && hy->slots && hy->w && hy->gpu_w && hy->host_ids,
               "hybrid_split_merge: NULL pointer (split)");
    size_t total;
    StageHeader nh{};
    stage_layout(T, k, H, &nh, &total);
    nh.magic = kStageMagic;
    nh.T = T;
    nh.k = k;
    nh.layer = hy->layer;
    nh.E = hy->E;
    nh.H = H;
    nh.host = *hy->host;
    nh.pool = hy->pool;
    nh.has_ntok = hy->n_tok != nullptr;
    *h = nh;
    hipLaunchKernelGGL(split_kernel, dim3(grid_for((int64_t)T * k)), dim3(256), 0, s, hy->ids_raw,
                       hy->slots, hy->w, T, k, hy->E, hy->n_tok, hy->gpu_w, hy->host_ids);
    MC_LAUNCH_CHECK();
    MC_HIP(hipMemcpyAsync(base + h->off_x, hy->x_bf16, (size_t)T * H * 2, hipMemcpyDeviceToHost, s));
    MC_HIP(hipMemcpyAsync(base + h->off_ids, hy->host_ids, (size_t)T * k * 4, hipMemcpyDeviceToHost, s));
    MC_HIP(hipMemcpyAsync(base + h->off_w, hy->w, (size_t)T * k * 4, hipMemcpyDeviceToHost, s));
    if (hy->n_tok)
      MC_HIP(hipMemcpyAsync(base + h->off_ntok, hy->n_tok, 4, hipMemcpyDeviceToHost, s));
    MC_HIP(hipLaunchHostFunc(s, submit_host_branch, h));
    return MC_OK;
  }

  MC_REQUIRE(h->magic == kStageMagic && h->T == T && h->k == k && h->H == H,
             "hybrid_split_merge: MERGE without a matching SPLIT_SUBMIT on this stage");
  MC_REQUIRE(hy->y_acc && hy->y_host && hy->y_bf16, "hybrid_split_merge: NULL pointer (merge)");
  MC_HIP(hipLaunchHostFunc(s, wait_host_branch, h));
  MC_HIP(hipMemcpyAsync(hy->y_host, base + h->off_y, (size_t)T * H * 4, hipMemcpyHostToDevice, s));
  hipLaunchKernelGGL(merge_kernel, dim3(grid_for((int64_t)T * H)), dim3(256), 0, s, hy->y_acc,
                     hy->y_host, T, H, hy->n_tok, static_cast<uint16_t*>(hy->y_bf16));
  MC_LAUNCH_CHECK();
  return MC_OK;
}
