// Internal helpers shared by the gfx950 kernels of libmoecache.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe_cache.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN maps to a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Sticky device status: keep the first error code.
__device__ __forceinline__ void set_status(int32_t* status, int code) {
  if (status) atomicCAS(status, 0, code);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ unsigned long long lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe

// Host-side helpers.
#define MOE_HIP_CHECK(expr)                      \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return MOE_EHIP;       \
  } while (0)

#define MOE_LAUNCH_CHECK()                                  \
  do {                                                      \
    hipError_t _e = hipGetLastError();                      \
    if (_e != hipSuccess) return MOE_EHIP;                  \
  } while (0)

static inline bool moe_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
