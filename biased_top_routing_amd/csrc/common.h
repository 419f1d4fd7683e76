// Internal helpers shared by the HIP kernels and host launchers of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;   // raw bfloat16 bits
typedef uint8_t fp8_t;     // raw OCP E4M3FN bytes

constexpr int kWave = 64;

#if defined(__HIP_DEVICE_COMPILE__)
// Logistic sigmoid of a SwiGLU gate input: the hardware reciprocal (v_rcp_f32,
// 1 ulp) of 1 + exp(-g) in place of an IEEE division, whose ~10 instructions
// per element weighed on the GEMM epilogues (FP8 gate/up 2% faster).  g = -inf
// or a large negative g gives 1 + exp(-g) = inf and a sigmoid of 0.
__device__ __forceinline__ float gate_sigmoid(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
#endif

// ----------------------------------------------------------------- host side
moe_status validate_cfg(const moe_cfg* c);
bool gemm_dtype_ok(const moe_cfg* c);
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t pairs(const moe_cfg* c) { return (int64_t)c->T * c->k; }
inline size_t act_bytes(const moe_cfg* c) { return c->act == MOE_F32 ? 4 : 2; }
inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// moe_route's workspace: room for the [T, E] fp32 affinities when the caller
// passes no `scores` (at least 256 bytes, so that a size of 0 means an invalid cfg)
inline size_t route_ws_bytes(const moe_cfg* c) {
  const size_t b = (size_t)c->T * c->E * sizeof(float);
  return align_up(b < 256 ? 256 : b, 256);
}

// ---------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// round to nearest, ties to even (inputs are finite on this path)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// fl32(v / sc) for a scale sc with y = fl32(1 / sc): the product q0 = v * y is
// within one ulp of the quotient, its remainder v - q0 * sc is exact by FMA, and
// one correction step q0 + remainder * y then rounds to the correctly rounded
// quotient (Markstein's theorem) as long as neither the remainder nor the
// quotient underflows; for |v| or |q0| below 2^-100 the IEEE division is taken.
__device__ __forceinline__ float div_by_scale(float v, float sc, float y) {
  const float q0 = v * y;
  const float r = fmaf(-q0, sc, v);
  float q = fmaf(r, y, q0);
  if (fminf(fabsf(v), fabsf(q0)) < 0x1p-100f) q = __fdiv_rn(v, sc);
  return q;
}

// Four values as OCP E4M3FN codes (bytes 0..3 = a, b, c, d) by the hardware
// conversion: nearest, ties to the even code.  For every fp32 |v| <= 448 (all the
// quantisers here produce: |v| <= amax = 448 sc) it equals an encoder written from
// the format definition (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals m/8 * 2^-6), checked over every such fp32 value.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float e4m3_to_f32(fp8_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float mag = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80) ? -mag : mag;
}

// Total order key of a float for max-selection: larger float -> larger key.
// -0.0 is first mapped to +0.0 so both rank alike.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe
