// Wave-wide reductions without LDS round trips (gfx950, 64-wide waves).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// v of the lane that DPP control CTRL names (all 64 lanes active, sources inside the row).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum of v over the wave, the same in every lane: DPP moves inside each 16-lane row
// (quad swaps, then half-row and row mirrors) leave every lane with its row's maximum, and
// the four row maxima are read out as scalars.  Needs all 64 lanes active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Sum of v over the wave, the same in every lane: DPP adds inside each 16-lane row, then
// the four row sums read out as scalars and added in a fixed order.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));   // quad_perm [1,0,3,2]
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));   // quad_perm [2,3,0,1]
  v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));  // row_half_mirror
  v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));  // row_mirror
  const uint32_t b = __float_as_uint(v);
  const float a0 = __uint_as_float(__builtin_amdgcn_readlane(b, 0));
  const float a1 = __uint_as_float(__builtin_amdgcn_readlane(b, 16));
  const float a2 = __uint_as_float(__builtin_amdgcn_readlane(b, 32));
  const float a3 = __uint_as_float(__builtin_amdgcn_readlane(b, 48));
  return (a0 + a1) + (a2 + a3);
}

}  // namespace moe
