// Host branch of the hybrid decode: persistent worker pool + host expert FFN.
//
// [jjl357] "8.3 CPU 分支也被纳入捕获路径": a persistent C++ worker pool pinned to
// cores runs SIMD expert kernels that dequantise inside the kernel instead of
// materialising larger temporary weights.  [jjl357] "6.2": host-computed experts
// stay in host DRAM and are run in place.  [wanger] "背景": the CPU reads the pinned
// banks directly (no PCIe) and computes a GEMV.
//
// Work split: phase 1 = (expert, 16 intermediate rows) tasks computing
// h = silu(W_gate x) * (W_up x) for every token routed to the expert; phase 2 =
// (16 hidden rows) tasks summing w * (W_down h) over the experts in a fixed order,
// so y does not depend on the number of threads.
#include <immintrin.h>
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "hybrid_stage.h"
#include "mc.h"

namespace mc {
void set_error(const char* fmt, ...);
void clear_error();
int host_experts_run(mc_host_pool* pool, const uint16_t* x, const int32_t* ids, const float* w,
                     int T, int k, int layer, int E, const mc_banks* host, float* y);

// Stages served by the dispatchers (every pool's dispatcher scans the entries of its
// own pool; the lock is held while a stage is served, so dropping a stage waits until
// no dispatcher is using it).
struct StageEntry {
  StageHeader* st;
  mc_host_pool* pool;
  uint64_t handled;   // the last request number this entry has completed
};
static std::mutex g_stage_mu;
static std::vector<StageEntry> g_stages;
}  // namespace mc

// ------------------------------------------------------------------ worker pool

// Hand-offs between the calling thread and the workers spin before they block: a
// layer's host branch runs two parallel passes a few hundred microseconds apart, and a
// condition-variable wake-up costs tens of microseconds per thread.  The spin first
// pauses, then yields the core (other runnable threads, such as the one launching GPU
// work, still get it), and blocks after kSpinUs.
constexpr int kSpinUs = 200;

template <class Pred>
static bool spin_until(Pred done) {
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0;; ++i) {
    if (done()) return true;
    if (i < 256) {
      _mm_pause();
    } else {
      if ((i & 15) == 0 &&
          std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(kSpinUs))
        return false;
      sched_yield();
    }
  }
}

struct mc_host_pool {
  std::vector<std::thread> threads;
  std::mutex mu, pf_mu;
  std::condition_variable cv_work, cv_done;
  // parallel-for state (one generation at a time; every worker acknowledges each)
  const std::function<void(int)>* fn = nullptr;
  std::atomic<int> next{0};
  int n_tasks = 0;
  std::atomic<int> generation{0};
  std::atomic<int> acked{0};
  bool stop = false;
  std::atomic<bool> stop_flag{false};
  // dispatcher of the hybrid stages (the host branch)
  std::thread driver;
  std::atomic<bool> driver_stop{false};
  std::vector<int> cpus;                 // CPU of thread i (0 = dispatcher), -1 = not pinned

  void worker_loop() {
    int seen = 0;
    for (;;) {
      spin_until([&] {
        return stop_flag.load(std::memory_order_acquire) ||
               generation.load(std::memory_order_acquire) != seen;
      });
      const std::function<void(int)>* f;
      int n;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv_work.wait(lk, [&] { return stop || generation.load() != seen; });
        if (stop) return;
        seen = generation.load();
        f = fn;
        n = n_tasks;
      }
      for (int i; (i = next.fetch_add(1)) < n;) (*f)(i);
      if (acked.fetch_add(1, std::memory_order_acq_rel) + 1 == (int)threads.size()) {
        std::lock_guard<std::mutex> lk(mu);
        cv_done.notify_all();
      }
    }
  }

  // Runs f(0..n-1) on the workers and the calling thread; returns when every task
  // is done and every worker has left this generation.
  void parallel_for(int n, const std::function<void(int)>& f) {
    if (n <= 0) return;
    if (threads.empty()) {
      for (int i = 0; i < n; ++i) f(i);
      return;
    }
    std::lock_guard<std::mutex> serial(pf_mu);
    {
      std::lock_guard<std::mutex> lk(mu);
      fn = &f;
      n_tasks = n;
      next.store(0);
      acked.store(0);
      generation.fetch_add(1, std::memory_order_acq_rel);
    }
    cv_work.notify_all();
    for (int i; (i = next.fetch_add(1)) < n;) f(i);
    const int nw = (int)threads.size();
    if (!spin_until([&] { return acked.load(std::memory_order_acquire) == nw; })) {
      std::unique_lock<std::mutex> lk(mu);
      cv_done.wait(lk, [&] { return acked.load() == nw; });
    }
    std::lock_guard<std::mutex> lk(mu);
    fn = nullptr;
  }

  // Serves the hybrid stages of this pool: a stage whose request number has moved past
  // the last one served gets its host partial computed (this thread takes part in the
  // parallel work), then its completion number raised.  Polls without pause while calls
  // keep coming; after about a millisecond without work it polls every 50 us.
  void driver_loop();
};

void mc_host_pool::driver_loop() {
  int idle = 0;
  while (!driver_stop.load(std::memory_order_relaxed)) {
    bool served = false;
    {
      std::lock_guard<std::mutex> lk(mc::g_stage_mu);
      for (auto& e : mc::g_stages) {
        if (e.pool != this) continue;
        uint8_t* base = reinterpret_cast<uint8_t*>(e.st);
        mc::StageReq* req = reinterpret_cast<mc::StageReq*>(base + e.st->off_req);
        const uint64_t seq = __atomic_load_n(&req->seq, __ATOMIC_ACQUIRE);
        if (seq == e.handled) continue;
        const mc::StageHeader& h = *e.st;
        const int nt = std::min(std::max(req->ntok, 0), h.T);
        float* y = reinterpret_cast<float*>(base + h.off_y);
        memset(y, 0, sizeof(float) * (size_t)nt * h.H);
        mc::host_experts_run(this, reinterpret_cast<const uint16_t*>(base + h.off_x),
                             reinterpret_cast<const int32_t*>(base + h.off_ids),
                             reinterpret_cast<const float*>(base + h.off_w), nt, h.k, req->layer, h.E,
                             &h.host, y);
        mc::StageDone* done = reinterpret_cast<mc::StageDone*>(base + h.off_done);
        __atomic_store_n(&done->seq, seq, __ATOMIC_RELEASE);
        e.handled = seq;
        served = true;
      }
    }
    if (served) {
      idle = 0;
    } else if (++idle < 20000) {
      _mm_pause();
    } else {
      std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
  }
}

namespace mc {

static int read_int_file(const char* path, int dflt) {
  FILE* f = fopen(path, "r");
  if (!f) return dflt;
  int v = dflt;
  if (fscanf(f, "%d", &v) != 1) v = dflt;
  fclose(f);
  return v;
}

// Default placement ([jjl357] "8.3": workers pinned to physical cores): the CPUs this
// process may run on, one hardware thread of each physical core first (the lowest
// numbered, in (package, core) order), then the cores' further hardware threads.
// Topology comes from /sys; a CPU without it counts as a core of its own.
static std::vector<int> physical_core_order() {
  cpu_set_t allowed;
  CPU_ZERO(&allowed);
  std::vector<int> cpus;
  if (sched_getaffinity(0, sizeof allowed, &allowed) == 0) {
    for (int c = 0; c < CPU_SETSIZE; ++c)
      if (CPU_ISSET(c, &allowed)) cpus.push_back(c);
  }
  struct Cpu { int pkg, core, cpu; };
  std::vector<Cpu> info;
  for (int c : cpus) {
    char path[128];
    snprintf(path, sizeof path, "/sys/devices/system/cpu/cpu%d/topology/physical_package_id", c);
    const int pkg = read_int_file(path, 0);
    snprintf(path, sizeof path, "/sys/devices/system/cpu/cpu%d/topology/core_id", c);
    const int core = read_int_file(path, 100000 + c);
    info.push_back({pkg, core, c});
  }
  std::sort(info.begin(), info.end(), [](const Cpu& a, const Cpu& b) {
    return a.pkg != b.pkg ? a.pkg < b.pkg : (a.core != b.core ? a.core < b.core : a.cpu < b.cpu);
  });
  std::vector<int> order;
  std::vector<bool> used(info.size(), false);
  for (size_t round = 0; order.size() < info.size(); ++round) {
    // round r takes the r-th hardware thread of every core that has one
    size_t i = 0;
    while (i < info.size()) {
      size_t j = i;
      while (j < info.size() && info[j].pkg == info[i].pkg && info[j].core == info[i].core) ++j;
      if (i + round < j && !used[i + round]) {
        used[i + round] = true;
        order.push_back(info[i + round].cpu);
      }
      i = j;
    }
    if (round > info.size()) break;
  }
  return order;
}

static void pin_thread(std::thread& t, int cpu) {
  if (cpu < 0) return;
  cpu_set_t set;
  CPU_ZERO(&set);
  CPU_SET(cpu, &set);
  pthread_setaffinity_np(t.native_handle(), sizeof set, &set);
}

}  // namespace mc

extern "C" mc_host_pool* mc_host_pool_create(int32_t n_threads, const int32_t* cpu_ids) {
  mc::clear_error();
  if (n_threads < 1 || n_threads > 1024) {
    mc::set_error("mc_host_pool_create: n_threads=%d must be in [1, 1024]", n_threads);
    return nullptr;
  }
  mc_host_pool* p = new (std::nothrow) mc_host_pool();
  if (!p) {
    mc::set_error("mc_host_pool_create: out of memory");
    return nullptr;
  }
  // thread i of the pool (0 = the dispatcher, which also computes; 1.. = workers) runs
  // on p->cpus[i]: the caller's list, or distinct physical cores of the allowed set.  The
  // first core of that order is left to the rest of the process (the thread that drives
  // the GPU must never share a CPU with a spinning worker); threads beyond the remaining
  // CPUs stay unpinned
  p->cpus.assign(n_threads, -1);
  if (cpu_ids) {
    for (int i = 0; i < n_threads; ++i) p->cpus[i] = cpu_ids[i];
  } else {
    const std::vector<int> order = mc::physical_core_order();
    for (int i = 0; i < n_threads && (size_t)i + 1 < order.size(); ++i) p->cpus[i] = order[i + 1];
  }
  // the calling thread takes part in parallel_for, so n_threads - 1 workers
  for (int i = 0; i + 1 < n_threads; ++i) {
    p->threads.emplace_back([p] { p->worker_loop(); });
    mc::pin_thread(p->threads.back(), p->cpus[i + 1]);
  }
  p->driver = std::thread([p] { p->driver_loop(); });
  mc::pin_thread(p->driver, p->cpus[0]);
  return p;
}

extern "C" int32_t mc_host_pool_cpus(const mc_host_pool* p, int32_t* cpus, int32_t n) {
  mc::clear_error();
  if (!p || (n > 0 && !cpus)) {
    mc::set_error("mc_host_pool_cpus: NULL pointer");
    return MC_EINVAL;
  }
  const int32_t total = (int32_t)p->cpus.size();
  for (int32_t i = 0; i < n && i < total; ++i) cpus[i] = p->cpus[i];
  return total;
}

extern "C" void mc_host_pool_destroy(mc_host_pool* p) {
  if (!p) return;
  p->driver_stop.store(true);
  p->driver.join();
  {
    std::lock_guard<std::mutex> lk(mc::g_stage_mu);
    mc::g_stages.erase(std::remove_if(mc::g_stages.begin(), mc::g_stages.end(),
                                      [p](const mc::StageEntry& e) { return e.pool == p; }),
                       mc::g_stages.end());
  }
  {
    std::lock_guard<std::mutex> lk(p->mu);
    p->stop = true;
    p->stop_flag.store(true, std::memory_order_release);
  }
  p->cv_work.notify_all();
  for (auto& t : p->threads) t.join();
  delete p;
}

namespace mc {

void host_pool_add_stage(mc_host_pool* pool, StageHeader* stage) {
  std::lock_guard<std::mutex> lk(g_stage_mu);
  for (auto& e : g_stages)
    if (e.st == stage) return;
  const StageDone* done = reinterpret_cast<const StageDone*>(reinterpret_cast<uint8_t*>(stage) + stage->off_done);
  g_stages.push_back(StageEntry{stage, pool, __atomic_load_n(&done->seq, __ATOMIC_ACQUIRE)});
}

void host_pool_drop_stage(StageHeader* stage) {
  std::lock_guard<std::mutex> lk(g_stage_mu);
  g_stages.erase(std::remove_if(g_stages.begin(), g_stages.end(),
                                [stage](const StageEntry& e) { return e.st == stage; }),
                 g_stages.end());
}

// ------------------------------------------------------------------ expert kernels

static float g_e2m1[16];
static bool init_table() {
  for (int c = 0; c < 16; ++c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    float mag = e == 0 ? 0.5f * m : ldexpf(1.0f + 0.5f * m, e - 1);
    g_e2m1[c] = s ? -mag : mag;
  }
  return true;
}
static bool g_table_ok = init_table();

// e8m0 scale byte -> 2^(X - 127), from a table built once (X = 255 never occurs)
static float g_e8m0[256];
static bool init_e8m0() {
  for (int X = 0; X < 256; ++X) g_e8m0[X] = ldexpf(1.0f, X - 127);
  return true;
}
static bool g_e8m0_ok = init_e8m0();
static inline float e8m0(uint8_t X) { return g_e8m0[X]; }
static inline float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Activation vector prepared for one format: MXFP4 blocks of 32 are stored as
// 16 even-index values followed by 16 odd-index values (matching the low/high
// nibbles of the code bytes); bf16 rows keep natural order.
static void prep_vec(const float* v, int n, int fmt, float* out) {
  if (fmt == MC_MXFP4) {
    for (int b = 0; b < n / 32; ++b)
      for (int i = 0; i < 16; ++i) {
        out[32 * b + i] = v[32 * b + 2 * i];
        out[32 * b + 16 + i] = v[32 * b + 2 * i + 1];
      }
  } else {
    memcpy(out, v, sizeof(float) * n);
  }
}

static float dot_mx_scalar(const uint8_t* codes, const uint8_t* scales, const float* xp, int n) {
  float acc = 0.0f;
  for (int b = 0; b < n / 32; ++b) {
    float part = 0.0f;
    for (int i = 0; i < 16; ++i) {
      uint8_t byte = codes[16 * b + i];
      part += g_e2m1[byte & 15] * xp[32 * b + i] + g_e2m1[byte >> 4] * xp[32 * b + 16 + i];
    }
    acc += part * e8m0(scales[b]);
  }
  return acc;
}

static float dot_bf_scalar(const uint16_t* wrow, const float* xp, int n) {
  float acc = 0.0f;
  for (int i = 0; i < n; ++i) acc += bf16f(wrow[i]) * xp[i];
  return acc;
}

__attribute__((target("avx512f,avx512bw")))
static float dot_mx_avx512(const uint8_t* codes, const uint8_t* scales, const float* xp, int n) {
  const __m512 tab = _mm512_loadu_ps(g_e2m1);
  const __m512i lo4 = _mm512_set1_epi32(15);
  __m512 acc = _mm512_setzero_ps();
  for (int b = 0; b < n / 32; ++b) {
    __m512i bytes = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)(codes + 16 * b)));
    __m512 ve = _mm512_permutexvar_ps(_mm512_and_si512(bytes, lo4), tab);
    __m512 vo = _mm512_permutexvar_ps(_mm512_srli_epi32(bytes, 4), tab);
    __m512 part = _mm512_mul_ps(ve, _mm512_loadu_ps(xp + 32 * b));
    part = _mm512_fmadd_ps(vo, _mm512_loadu_ps(xp + 32 * b + 16), part);
    acc = _mm512_fmadd_ps(part, _mm512_set1_ps(e8m0(scales[b])), acc);
  }
  return _mm512_reduce_add_ps(acc);
}

__attribute__((target("avx512f,avx512bw")))
static float dot_bf_avx512(const uint16_t* wrow, const float* xp, int n) {
  __m512 acc = _mm512_setzero_ps();
  int i = 0;
  for (; i + 16 <= n; i += 16) {
    __m512i w16 = _mm512_cvtepu16_epi32(_mm256_loadu_si256((const __m256i*)(wrow + i)));
    __m512 wf = _mm512_castsi512_ps(_mm512_slli_epi32(w16, 16));
    acc = _mm512_fmadd_ps(wf, _mm512_loadu_ps(xp + i), acc);
  }
  float s = _mm512_reduce_add_ps(acc);
  for (; i < n; ++i) s += bf16f(wrow[i]) * xp[i];
  return s;
}

static bool g_avx512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");

static inline float dot_row(int fmt, const uint8_t* row, const uint8_t* srow, const float* xp,
                            int n) {
  if (fmt == MC_MXFP4)
    return g_avx512 ? dot_mx_avx512(row, srow, xp, n) : dot_mx_scalar(row, srow, xp, n);
  const uint16_t* r = reinterpret_cast<const uint16_t*>(row);
  return g_avx512 ? dot_bf_avx512(r, xp, n) : dot_bf_scalar(r, xp, n);
}

static void run_tasks(mc_host_pool* pool, int n, const std::function<void(int)>& f) {
  if (pool)
    pool->parallel_for(n, f);
  else
    for (int i = 0; i < n; ++i) f(i);
}

struct HostUnit {
  int64_t entry;                 // host bank entry (flat id)
  std::vector<int> toks;         // tokens routed to it
  std::vector<float> gates;
};

int host_experts_run(mc_host_pool* pool, const uint16_t* x, const int32_t* ids, const float* w,
                     int T, int k, int layer, int E, const mc_banks* host, float* y) {
  const int H = host->H, I = host->I, fmt = host->fmt;
  // units in first-occurrence order
  std::vector<HostUnit> units;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      if (e < 0 || e >= E) continue;
      int64_t flat = (int64_t)layer * E + e;
      if (flat >= host->n) continue;
      HostUnit* u = nullptr;
      for (auto& v : units)
        if (v.entry == flat) u = &v;
      if (!u) {
        units.push_back(HostUnit{flat, {}, {}});
        u = &units.back();
      }
      u->toks.push_back(t);
      u->gates.push_back(w[(size_t)t * k + j]);
    }
  if (units.empty()) return MC_OK;

  // prepared activations
  std::vector<float> xp((size_t)T * H), xtmp(H);
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < H; ++c) xtmp[c] = bf16f(x[(size_t)t * H + c]);
    prep_vec(xtmp.data(), H, fmt, xp.data() + (size_t)t * H);
  }
  // h per (unit, token-of-unit), prepared for the down contraction
  std::vector<size_t> hoff(units.size() + 1, 0);
  for (size_t u = 0; u < units.size(); ++u) hoff[u + 1] = hoff[u] + units[u].toks.size();
  std::vector<float> h(hoff.back() * I), hp(hoff.back() * I);

  const size_t gu_row = fmt == MC_MXFP4 ? H / 2 : (size_t)H * 2;
  const size_t gu_per = 2 * (size_t)I * gu_row;
  const size_t gus_per = 2 * (size_t)I * H / 32;
  const size_t dn_row = fmt == MC_MXFP4 ? I / 2 : (size_t)I * 2;
  const size_t dn_per = (size_t)H * dn_row;
  const size_t dns_per = (size_t)H * I / 32;
  const uint8_t* GU = static_cast<const uint8_t*>(host->gate_up);
  const uint8_t* GUS = static_cast<const uint8_t*>(host->gate_up_scale);
  const uint8_t* DN = static_cast<const uint8_t*>(host->down);
  const uint8_t* DNS = static_cast<const uint8_t*>(host->down_scale);

  constexpr int RB = 16;
  const int nib = I / RB;
  std::function<void(int)> phase1 = [&](int task) {
    const size_t u = task / nib;
    const int i0 = (task % nib) * RB;
    const HostUnit& U = units[u];
    const uint8_t* gu = GU + U.entry * gu_per;
    const uint8_t* gus = fmt == MC_MXFP4 ? GUS + U.entry * gus_per : nullptr;
    for (int i = i0; i < i0 + RB; ++i) {
      const uint8_t* rg = gu + (size_t)i * gu_row;
      const uint8_t* ru = gu + (size_t)(I + i) * gu_row;
      const uint8_t* sg = gus ? gus + (size_t)i * (H / 32) : nullptr;
      const uint8_t* su = gus ? gus + (size_t)(I + i) * (H / 32) : nullptr;
      for (size_t n = 0; n < U.toks.size(); ++n) {
        const float* xv = xp.data() + (size_t)U.toks[n] * H;
        float g = dot_row(fmt, rg, sg, xv, H);
        float up = dot_row(fmt, ru, su, xv, H);
        h[(hoff[u] + n) * I + i] = g / (1.0f + expf(-g)) * up;
      }
    }
  };
  run_tasks(pool, (int)units.size() * nib, phase1);
  for (size_t r = 0; r < hoff.back(); ++r) prep_vec(h.data() + r * I, I, fmt, hp.data() + r * I);

  const int nrb = (H + RB - 1) / RB;
  std::function<void(int)> phase2 = [&](int task) {
    const int r0 = task * RB, r1 = std::min(H, r0 + RB);
    for (size_t u = 0; u < units.size(); ++u) {
      const HostUnit& U = units[u];
      const uint8_t* dn = DN + U.entry * dn_per;
      const uint8_t* dns = fmt == MC_MXFP4 ? DNS + U.entry * dns_per : nullptr;
      for (int r = r0; r < r1; ++r) {
        const uint8_t* row = dn + (size_t)r * dn_row;
        const uint8_t* srow = dns ? dns + (size_t)r * (I / 32) : nullptr;
        for (size_t n = 0; n < U.toks.size(); ++n) {
          float v = dot_row(fmt, row, srow, hp.data() + (hoff[u] + n) * I, I);
          y[(size_t)U.toks[n] * H + r] += U.gates[n] * v;
        }
      }
    }
  };
  run_tasks(pool, nrb, phase2);
  return MC_OK;
}

}  // namespace mc

extern "C" int mc_host_experts(mc_host_pool* pool, const void* x_bf16, const int32_t* ids,
                               const float* w, int32_t T, int32_t k, int32_t layer, int32_t E,
                               const mc_banks* host, float* y) {
  mc::clear_error();
  if (!host || !(host->fmt == MC_BF16 || host->fmt == MC_MXFP4) || host->H <= 0 ||
      host->I <= 0 || host->H % 64 || host->I % 64 || host->n <= 0 || !host->gate_up ||
      !host->down || (host->fmt == MC_MXFP4 && (!host->gate_up_scale || !host->down_scale))) {
    mc::set_error("mc_host_experts: invalid host banks");
    return MC_EINVAL;
  }
  if (T < 0 || k < 1 || E < 1 || layer < 0) {
    mc::set_error("mc_host_experts: T=%d k=%d E=%d layer=%d", T, k, E, layer);
    return MC_EINVAL;
  }
  if (T == 0) return MC_OK;
  if (!x_bf16 || !ids || !w || !y) {
    mc::set_error("mc_host_experts: NULL pointer");
    return MC_EINVAL;
  }
  return mc::host_experts_run(pool, static_cast<const uint16_t*>(x_bf16), ids, w, T, k, layer, E,
                              host, y);
}
