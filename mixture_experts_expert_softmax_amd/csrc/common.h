// Shared device and host helpers of the gfx950 MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ host side
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Number of compute units of the current device (cached per device id).
int device_cu_count();

// ------------------------------------------------------------------ device side
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// register staging type for 16-byte copies: a vector, not an aggregate, so that a
// load kept in registers and stored later is not merged into one memory-to-memory copy
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// silu(z) = z / (1 + e^-z), with the hardware base-2 exponential and reciprocal.
__device__ __forceinline__ float silu_f32(float z) {
  float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe
