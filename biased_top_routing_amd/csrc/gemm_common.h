// Device helpers shared by the bf16 MFMA GEMM engines (forward and backward):
// operand vector types, raw buffer descriptors for direct-to-LDS loads, the
// XOR swizzles of 16-byte LDS chunks, and vector-memory wait counts.
#pragma once

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// s_waitcnt immediate that waits until at most N vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima; gfx9
// encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
constexpr int kVmWaitOneStage() {
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// s_waitcnt immediate that waits for every LDS (and scalar memory) operation of
// this wave (vmcnt and expcnt left at their maxima).
constexpr int kLgkmWaitZero = 0xF | (0x3 << 14) | (0x7 << 4);

// Word 3 of a raw buffer descriptor (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

// Raw buffer descriptor over [base, base + bytes), built from wave-uniform
// values so that it lives in SGPRs.
#if defined(__HIP_DEVICE_COMPILE__)   // the descriptor type exists only for the GPU target
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, __builtin_amdgcn_readfirstlane(bytes), kBufferWord3);
}
#endif

// Physical 16-byte chunk of logical chunk c in LDS row r (CPR chunks per row).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR == 8) return c ^ ((r & 7) ^ ((r >> 3) & 1));
  else return c ^ (((r >> 1) ^ (r >> 2)) & 3);   // CPR == 4
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(kVmWaitOneStage<N>());
}

// Waits until at most `n` slices' loads (PER instructions each) of this wave
// are outstanding; n < 4.
template <int PER>
__device__ __forceinline__ void wait_slices(int n) {
  if (n <= 0) wait_vm<0>();
  else if (n == 1) wait_vm<PER>();
  else if (n == 2) wait_vm<2 * PER>();
  else wait_vm<3 * PER>();
}

}  // namespace moe
