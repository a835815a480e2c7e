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
  const double bytes = (double)bank_bytes(host->fmt, H, host->I).total() * n;

  // device fill list: entries 0..n-1 -> slots 0..n-1
  DevLists dl;
  MC_HIP(hipMalloc((void**)&dl.p, sizeof(int32_t) * (2 * (size_t)n + 1)));
  {
    std::vector<int32_t> h(2 * (size_t)n + 1);
    for (int i = 0; i < n; ++i) h[i] = h[n + i] = i;
    h[2 * n] = n;
    MC_HIP(hipMemcpy(dl.p, h.data(), h.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  }
  // host branch inputs: one token routed to the n experts of "layer 0"
  std::vector<uint16_t> x(H, 0x3F80);            // bf16 1.0
  std::vector<int32_t> ids(n);
  std::vector<float> w(n, 1.0f / n), y(H, 0.0f);
  for (int i = 0; i < n; ++i) ids[i] = i;

  Events ev;
  MC_HIP(hipEventCreate(&ev.a));
  MC_HIP(hipEventCreate(&ev.b));
  auto fills = [&](int reps) -> int {
    for (int r = 0; r < reps; ++r) {
      int e = mc_fill_slots(host, pool, dl.p, dl.p + n, dl.p + 2 * n, n, s);
      if (e != MC_OK) return e;
    }
    return MC_OK;
  };
  auto cpu = [&](int reps) -> int {
    for (int r = 0; r < reps; ++r) {
      int e = mc_host_experts(workers, x.data(), ids.data(), w.data(), 1, n, 0, n, host, y.data());
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
  out->expert_bytes = bytes / n;
  return MC_OK;
}
