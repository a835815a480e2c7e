// Library-level calls: version, errors, cache reset, fetch fraction, bf16 finish.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "mc_common.h"

namespace mc {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

int check_banks(const mc_banks* b, const char* what, bool need_nonempty) {
  MC_REQUIRE(b != nullptr, "%s: bank descriptor is NULL", what);
  MC_REQUIRE(b->fmt == MC_BF16 || b->fmt == MC_MXFP4, "%s: unknown weight format %d", what, b->fmt);
  MC_REQUIRE(b->H > 0 && b->I > 0, "%s: H=%d I=%d must be positive", what, b->H, b->I);
  MC_REQUIRE(b->H % 64 == 0 && b->I % 64 == 0, "%s: H=%d and I=%d must be multiples of 64", what,
             b->H, b->I);
  MC_REQUIRE(!need_nonempty || b->n > 0, "%s: n=%lld must be positive", what, (long long)b->n);
  MC_REQUIRE(b->gate_up && b->down, "%s: NULL bank pointer", what);
  if (b->fmt == MC_MXFP4)
    MC_REQUIRE(b->gate_up_scale && b->down_scale, "%s: NULL scale bank", what);
  MC_REQUIRE(((uintptr_t)b->gate_up | (uintptr_t)b->down) % 16 == 0,
             "%s: bank bases must be 16-byte aligned", what);
  if (b->fmt == MC_MXFP4)
    MC_REQUIRE(((uintptr_t)b->gate_up_scale | (uintptr_t)b->down_scale) % 16 == 0,
               "%s: scale bank bases must be 16-byte aligned", what);
  return MC_OK;
}

__global__ void fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void fill_i64(int64_t* p, int64_t n, int64_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// y_bf16[t][c] = bf16_rne(y[t][c]) for t < n_tok, 0 beyond.
__global__ void finish_bf16_kernel(const float* __restrict__ y, int32_t T, int32_t H,
                                   const int32_t* __restrict__ n_tok, uint16_t* __restrict__ out) {
  int nt = n_tok ? min(max(*n_tok, 0), T) : T;
  int64_t n = (int64_t)T * H;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int t = (int)(i / H);
    out[i] = t < nt ? f32_to_bf16_rne(y[i]) : (uint16_t)0;
  }
}

static unsigned grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace mc

using namespace mc;

extern "C" int mc_abi_version(void) { return MC_ABI_VERSION; }

extern "C" const char* mc_last_error(void) { return g_err; }

extern "C" int mc_cache_reset(const mc_cache* c, hipStream_t s) {
  clear_error();
  MC_REQUIRE(c != nullptr, "mc_cache_reset: cache is NULL");
  MC_REQUIRE(c->L > 0 && c->E > 0 && c->S > 0, "mc_cache_reset: L=%d E=%d S=%d must be positive",
             c->L, c->E, c->S);
  MC_REQUIRE(c->slot_of && c->id_of && c->stamp && c->clock && c->stats,
             "mc_cache_reset: NULL table pointer");
  int64_t nf = (int64_t)c->L * c->E;
  hipLaunchKernelGGL(fill_i32, dim3(grid_for(nf, 256)), dim3(256), 0, s, c->slot_of, nf, -1);
  hipLaunchKernelGGL(fill_i32, dim3(grid_for(c->S, 256)), dim3(256), 0, s, c->id_of,
                     (int64_t)c->S, -1);
  hipLaunchKernelGGL(fill_i64, dim3(grid_for(c->S, 256)), dim3(256), 0, s, c->stamp,
                     (int64_t)c->S, (int64_t)0);
  hipLaunchKernelGGL(fill_i64, dim3(1), dim3(64), 0, s, c->clock, (int64_t)1, (int64_t)0);
  hipLaunchKernelGGL(fill_i64, dim3(1), dim3(64), 0, s, c->stats, (int64_t)8, (int64_t)0);
  MC_LAUNCH_CHECK();
  return MC_OK;
}

extern "C" uint32_t mc_fetch_fraction_q16(double b_p, double b_h, double p_ov, double c_ov) {
  double f;
  if (p_ov > 0.0) {
    if (!(c_ov >= 0.0)) c_ov = 0.0;
    f = p_ov / (p_ov + c_ov);
  } else {
    if (!(b_p > 0.0)) return 0;
    if (b_h <= b_p) return 65536u;
    f = b_p / b_h;
  }
  double v = floor(f * 65536.0 + 0.5);
  if (v < 1.0) v = 1.0;
  if (v > 65536.0) v = 65536.0;
  return (uint32_t)v;
}

extern "C" int mc_finish_bf16(const float* y_acc, int32_t T, int32_t H, const int32_t* n_tok,
                              void* y_bf16, hipStream_t s) {
  clear_error();
  MC_REQUIRE(T >= 0 && H > 0, "mc_finish_bf16: T=%d H=%d", T, H);
  if (T == 0) return MC_OK;
  MC_REQUIRE(y_acc && y_bf16, "mc_finish_bf16: NULL pointer");
  int64_t n = (int64_t)T * H;
  hipLaunchKernelGGL(finish_bf16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, y_acc, T, H,
                     n_tok, (uint16_t*)y_bf16);
  MC_LAUNCH_CHECK();
  return MC_OK;
}
