// Internal helpers shared by the HIP kernels and host launchers of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;   // raw bfloat16 bits
typedef uint8_t fp8_t;     // raw OCP E4M3FN bytes

constexpr int kWave = 64;

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

// OCP E4M3FN encoder: nearest representable value, ties to the even code,
// magnitudes above 448 saturate to 448.  Written from the format definition
// (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, exponent field 0
// holds the subnormals m/8 * 2^-6).
__device__ __forceinline__ fp8_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return (fp8_t)(sign | 0x7Eu);        // |v| >= 448
  int32_t e = (int32_t)(a >> 23) - 127;                      // unbiased exponent
  uint32_t code;
  if (e >= -6) {
    // normal range of E4M3: keep 3 mantissa bits, round the 20 dropped bits
    uint32_t m = a & 0x7FFFFFu;
    uint32_t keep = m >> 20;
    uint32_t rest = m & 0xFFFFFu;
    uint32_t c = ((uint32_t)(e + 7) << 3) | keep;
    if (rest > 0x80000u || (rest == 0x80000u && (c & 1u))) c += 1;   // may carry into the exponent
    code = c;
  } else {
    // subnormal range: value = n * 2^-9 with n in [0, 8]; round |v| * 2^9
    // (exact: a power-of-two scale of a value below 2^-6) to an integer,
    // ties to even; n == 8 is the smallest normal code 0x08.
    float scaled = __uint_as_float(a) * 512.0f;
    float fl = floorf(scaled);
    float frac = scaled - fl;
    uint32_t n = (uint32_t)fl;
    if (frac > 0.5f || (frac == 0.5f && (n & 1u))) n += 1;
    code = n;
  }
  if (code > 0x7Eu) code = 0x7Eu;
  return (fp8_t)(sign | code);
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
