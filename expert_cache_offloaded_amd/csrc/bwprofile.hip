// mc_bandwidth_profile / mc_recommend_backend: the start-up bandwidth profile that sets
// the hybrid split and picks the backend.
//
// [wanger] "第一层带宽比：选后端": two real kernels are measured, not memcpy figures:
// the CPU expert kernel at batch 1 reading the pinned banks (cpu_bw), and the
// host -> GPU expert gather (pcie_bw); hybrid is chosen iff cpu_bw exceeds a
// threshold (2.0 on that page) times pcie_bw.  [wanger] "实测版本：overlap 带宽取代假设":
// both kernels then run at the same time, and the bandwidths each reaches under that
// contention (p_ov, c_ov) give the fetched fraction f = p_ov / (p_ov + c_ov).
//
// Here the gather is the library's own fill kernel (mc_fill_slots) and the CPU side is
// mc_host_experts on the worker pool, i.e. exactly the two paths a hybrid decode layer
// runs.  The overlapped run sizes both sides from their stand-alone rates so that they
// take about the same time.
#include <math.h>

#include <algorithm>
#include <chrono>
#include <thread>
#include <vector>

#include "mc_common.h"

using namespace mc;

extern "C" int32_t mc_recommend_backend(double cpu_gbs, double pcie_gbs, double threshold) {
  return cpu_gbs > threshold * pcie_gbs ? 1 : 0;
}

namespace {

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

struct DevLists {
  int32_t* p = nullptr;   // [n] flat ids, [n] slots, [1] count
  ~DevLists() {
    if (p) (void)hipFree(p);
  }
};

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

}  // namespace

extern "C" int mc_bandwidth_profile(const mc_banks* host, const mc_banks* pool, mc_host_pool* workers,
                                    int32_t n_experts, double seconds, double threshold, hipStream_t s,
                                    mc_bw_profile* out) {
  clear_error();
  int rc;
  if ((rc = check_banks(host, "mc_bandwidth_profile host")) != MC_OK) return rc;
  if ((rc = check_banks(pool, "mc_bandwidth_profile pool")) != MC_OK) return rc;
  MC_REQUIRE(host->fmt == pool->fmt && host->H == pool->H && host->I == pool->I,
             "mc_bandwidth_profile: host and pool banks differ in format or shape");
  MC_REQUIRE(out != nullptr, "mc_bandwidth_profile: out is NULL");
  MC_REQUIRE(n_experts >= 1 && n_experts <= host->n && n_experts <= pool->n && n_experts <= 4096,
             "mc_bandwidth_profile: n_experts=%d must be in [1, min(host n, pool n, 4096)]", n_experts);
  MC_REQUIRE(seconds > 0.0 && seconds <= 60.0, "mc_bandwidth_profile: seconds=%g not in (0, 60]", seconds);
  MC_REQUIRE(threshold > 0.0, "mc_bandwidth_profile: threshold=%g must be > 0", threshold);
  const int n = n_experts, H = host->H;
  const double expert_bytes = (double)bank_bytes(host->fmt, H, host->I).total();
  const double bytes = expert_bytes * n;
  // Each call reads n experts of a window of W host entries and the next call the n
  // after them, so both paths stream from host DRAM as in a decode step: a few experts
  // read over and over would stay in the CPU's last-level cache and overstate the host
  // kernel.  W covers at least 1 GiB (or the whole host pool).
  int64_t W = (int64_t)ceil(1073741824.0 / expert_bytes);
  W = std::min<int64_t>(std::max<int64_t>(W, n), host->n);

  // device lists: flat ids [W + n] (entry j = j mod W, so any window of n is contiguous),
  // slots [n] = 0..n-1, count [1] = n
  DevLists dl;
  const size_t n_list = (size_t)W + 2 * (size_t)n + 1;
  MC_HIP(hipMalloc((void**)&dl.p, sizeof(int32_t) * n_list));
  int32_t* d_flat = dl.p;
  int32_t* d_slot = dl.p + W + n;
  int32_t* d_count = d_slot + n;
  {
    std::vector<int32_t> h(n_list);
    for (int64_t j = 0; j < W + n; ++j) h[j] = (int32_t)(j % W);
    for (int i = 0; i < n; ++i) h[W + n + i] = i;
    h[W + 2 * n] = n;
    MC_HIP(hipMemcpy(dl.p, h.data(), h.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  }
  // host branch inputs: one token routed to n experts of the window ("layer 0" spans
  // the whole host pool, so an id is a flat id)
  std::vector<uint16_t> x(H, 0x3F80);            // bf16 1.0
  std::vector<int32_t> ids(n);
  std::vector<float> w(n, 1.0f / n), y(H, 0.0f);
  int64_t fill_calls = 0, cpu_calls = 0;

  Events ev;
  MC_HIP(hipEventCreate(&ev.a));
  MC_HIP(hipEventCreate(&ev.b));
  auto fills = [&](int reps) -> int {
    for (int r = 0; r < reps; ++r) {
      const int64_t off = (fill_calls++ * n) % W;
      int e = mc_fill_slots(host, pool, d_flat + off, d_slot, d_count, n, s);
      if (e != MC_OK) return e;
    }
    return MC_OK;
  };
  auto cpu = [&](int reps) -> int {
    for (int r = 0; r < reps; ++r) {
      const int64_t off = (cpu_calls++ * n) % W;
      for (int i = 0; i < n; ++i) ids[i] = (int32_t)((off + i) % W);
      int e = mc_host_experts(workers, x.data(), ids.data(), w.data(), 1, n, 0, (int32_t)host->n, host,
                              y.data());
      if (e != MC_OK) return e;
    }
    return MC_OK;
  };
  auto timed_fills = [&](int reps, float* ms) -> int {
    MC_HIP(hipEventRecord(ev.a, s));
    int e = fills(reps);
    if (e != MC_OK) return e;
    MC_HIP(hipEventRecord(ev.b, s));
    MC_HIP(hipEventSynchronize(ev.b));
    MC_HIP(hipEventElapsedTime(ms, ev.a, ev.b));
    return MC_OK;
  };

  // warm both paths, then one timed call of each sizes the runs
  float ms = 0.0f;
  if ((rc = timed_fills(1, &ms)) != MC_OK) return rc;
  if ((rc = timed_fills(1, &ms)) != MC_OK) return rc;
  const double t_fill1 = ms * 1e-3 > 1e-7 ? ms * 1e-3 : 1e-7;
  if ((rc = cpu(1)) != MC_OK) return rc;
  double t0 = now_s();
  if ((rc = cpu(1)) != MC_OK) return rc;
  double dt = now_s() - t0;
  const double t_cpu1 = dt > 1e-7 ? dt : 1e-7;

  // each path alone, about seconds / 4 each
  const double quarter = seconds / 4.0;
  int rp = (int)(quarter / t_fill1) + 1, rcpu = (int)(quarter / t_cpu1) + 1;
  if ((rc = timed_fills(rp, &ms)) != MC_OK) return rc;
  const double t_fill = ms * 1e-3;
  t0 = now_s();
  if ((rc = cpu(rcpu)) != MC_OK) return rc;
  const double t_cpu = now_s() - t0;
  out->pcie_gbs = bytes * rp / t_fill * 1e-9;
  out->cpu_gbs = bytes * rcpu / t_cpu * 1e-9;

  // both at once, each sized to about seconds / 2 from its stand-alone rate
  const double half = seconds / 2.0;
  rp = (int)(half / (t_fill / rp)) + 1;
  rcpu = (int)(half / (t_cpu / rcpu)) + 1;
  // the CPU side runs on a thread of its own, so that a full launch queue on this
  // thread cannot hold it back
  double t_cpu_ov = 0.0;
  int rc_cpu = MC_OK;
  std::thread cpu_side([&] {
    const double c0 = now_s();
    rc_cpu = cpu(rcpu);
    t_cpu_ov = now_s() - c0;
  });
  int rc_fill = hipEventRecord(ev.a, s) == hipSuccess ? fills(rp) : MC_EHIP;
  if (rc_fill == MC_OK && hipEventRecord(ev.b, s) != hipSuccess) rc_fill = MC_EHIP;
  cpu_side.join();
  if (rc_fill != MC_OK) return rc_fill;
  if (rc_cpu != MC_OK) return rc_cpu;
  MC_HIP(hipEventSynchronize(ev.b));
  MC_HIP(hipEventElapsedTime(&ms, ev.a, ev.b));
  out->pcie_ov_gbs = bytes * rp / (ms * 1e-3) * 1e-9;
  out->cpu_ov_gbs = bytes * rcpu / t_cpu_ov * 1e-9;
  out->frac_q16 = mc_fetch_fraction_q16(out->pcie_gbs, out->cpu_gbs, out->pcie_ov_gbs, out->cpu_ov_gbs);
  out->hybrid = mc_recommend_backend(out->cpu_gbs, out->pcie_gbs, threshold);
  out->expert_bytes = expert_bytes;
  return MC_OK;
}
