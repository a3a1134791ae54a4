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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

typedef const __attribute__((address_space(1))) u32x4* gptr16;

// 16-byte global load (global_load_dwordx4, not a flat load).
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(gptr16)p; }

// 16-byte non-temporal global load (nt): for data streamed once in whole cache lines, such
// as expert weight rows in the decode path.
__device__ __forceinline__ u32x4 ldg16_nt(const void* p) { return __builtin_nontemporal_load((gptr16)p); }
// One byte through the global (not flat) path: a flat load would also count against the
// LDS counter, so every later LDS wait would wait for it too.
__device__ __forceinline__ uint32_t ldg_u8(const void* p) {
  return *(const __attribute__((address_space(1))) uint8_t*)p;
}

// Compiler-only fence: memory operations are not moved across it.  Placed after
// prefetch loads so they are issued where written instead of being sunk to their use.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// s_waitcnt immediate (gfx9 encoding): vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
constexpr int waitcnt_imm(int vm, int exp, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | ((exp & 0x7) << 4) | ((lgkm & 0xF) << 8);
}

// Workgroup barrier for LDS hand-off only: waits for this wave's LDS operations, then
// s_barrier.  Unlike __syncthreads() it does not drain outstanding global loads, so
// prefetches issued before the barrier stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 7, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
