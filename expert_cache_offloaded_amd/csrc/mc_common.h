// Shared host/device helpers of the MoE slot-cache library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "mc.h"

namespace mc {

// ---------------------------------------------------------------- host side errors

void set_error(const char* fmt, ...);
void clear_error();

#define MC_REQUIRE(cond, ...)            \
  do {                                   \
    if (!(cond)) {                       \
      ::mc::set_error(__VA_ARGS__);      \
      return MC_EINVAL;                  \
    }                                    \
  } while (0)

#define MC_HIP(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      ::mc::set_error("%s failed: %s", #call, hipGetErrorString(e_));       \
      return MC_EHIP;                                                       \
    }                                                                       \
  } while (0)

// Checks a launch (no synchronisation).
#define MC_LAUNCH_CHECK()                                                   \
  do {                                                                      \
    hipError_t e_ = hipGetLastError();                                      \
    if (e_ != hipSuccess) {                                                 \
      ::mc::set_error("kernel launch failed: %s", hipGetErrorString(e_));   \
      return MC_EHIP;                                                       \
    }                                                                       \
  } while (0)

// Bytes of one expert entry in each bank.
struct BankBytes {
  size_t gate_up, gate_up_scale, down, down_scale;
  size_t total() const { return gate_up + gate_up_scale + down + down_scale; }
};

inline BankBytes bank_bytes(int fmt, int H, int I) {
  BankBytes b{};
  if (fmt == MC_BF16) {
    b.gate_up = (size_t)2 * I * H * 2;
    b.down = (size_t)H * I * 2;
  } else {
    b.gate_up = (size_t)2 * I * H / 2;
    b.gate_up_scale = (size_t)2 * I * H / 32;
    b.down = (size_t)H * I / 2;
    b.down_scale = (size_t)H * I / 32;
  }
  return b;
}

// Host validation of a bank descriptor; returns MC_OK or MC_EINVAL with a message.
int check_banks(const mc_banks* b, const char* what, bool need_nonempty = true);

// Device-visible address of pinned host memory (NULL maps to NULL); MC_EINVAL with a
// message if `host` is not pinned.  Checked with the runtime on every call made
// outside stream capture; during capture of `s` a translation remembered from an
// earlier call on the same address is used.
int host_device_view(const void* host, const uint8_t** out, const char* what, hipStream_t s);
// Drops remembered translations of host addresses in [p, p + bytes); returns how many.
int host_forget(const void* p, size_t bytes);

// ---------------------------------------------------------------- device helpers

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// e8m0 exponent byte -> fp32 scale 2^(X-127) (X = 0 gives 2^-127, a subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t X) {
  return X == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(X << 23);
}

// Two FP4 E2M1 values held in byte `sel` of `v`, scaled, as packed bf16 (exact for
// the scales MXFP4 weights use).
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t v, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, SEL);
}

template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t v, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, scale, SEL);
}

// 8 consecutive MXFP4 elements (one dword of codes) -> bf16x8, scaled (exact).
__device__ __forceinline__ bf16x8_t fp4x8_bf16(uint32_t v, float s) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// v plus the value a DPP lane move brings (every source lane of these moves is valid).
template <int CTRL>
__device__ __forceinline__ float dpp_add_f32(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of 4 / 16 lanes by DPP moves inside a row (no LDS).
__device__ __forceinline__ float quad_sum(float v) {
  v = dpp_add_f32<0xB1>(v);          // quad_perm [1,0,3,2]
  return dpp_add_f32<0x4E>(v);       // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float row16_sum(float v) {
  v = quad_sum(v);
  v = dpp_add_f32<0x141>(v);         // row_half_mirror: the other quad of the 8
  return dpp_add_f32<0x140>(v);      // row_mirror: the other 8 of the row
}

// Sum over all 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64); every lane
// gets its group's sum.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width == 4) return quad_sum(v);
  if (width == 16) return row16_sum(v);
  if (width == 64) return wave_sum(v);
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mc
