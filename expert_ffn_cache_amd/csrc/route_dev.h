// Top-k softmax routing of one token by one 64-wide wavefront (shared by the routing kernel
// and the fused routing + grouping kernel).
//
// Top-k with a softmax gate: a token chooses a few of the routed experts, e.g.
// 6 of 256 for DeepSeek-V4-Flash (FreeToken RTX-4090 page, "How the MoE memory
// hierarchy works").  Order: larger logit first, equal values by lower id.
//
// Each lane holds ceil(E/64) logits in registers (lane l owns experts l, l+64, ...).  Each
// of the k rounds is a wave-wide max over a 64-bit key (order-preserving logit bits, then the
// complemented expert id so that ties go to the lower id), taken as 32-bit maxima (the high
// word, then, only when several lanes hold it, the low word among them) with DPP moves and
// scalar read-outs, so a round makes no LDS round trip; the owner lane retires the winner.
// The softmax over the k winners is summed in rank order as they come out; lane j writes
// winner j.
#pragma once

#include "common.h"
#include "wave.h"

namespace moe {

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);  // -0 and +0 compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Keys of one token's E logits at row (lane l: experts l, l+64, ...); called by a full wave.
// All NPL loads are issued before the first is used (a lane past E reads logit E - 1 and
// gets key 0), so the row costs one memory round trip.
template <int NPL>
__device__ __forceinline__ void route_keys(const float* __restrict__ row, int E,
                                           unsigned long long (&key)[NPL]) {
  const int lane = threadIdx.x & 63;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ((unsigned long long)order_bits(v[i]) << 32) | (uint32_t)(~(uint32_t)e) : 0ull;
  }
}

// ids[j], w[j] (j < k) from a token's keys (consumed); also ids into ids2 when not null.
// A round's winner is the largest high word; the low word (the complemented id) is reduced
// over the wave only when several lanes hold that high word, so a round is usually one DPP
// reduction.  The softmax denominator is summed in rank order as the winners come out.
template <int NPL>
__device__ __forceinline__ void route_pick(unsigned long long (&key)[NPL], int k,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* ids2) {
  const int lane = threadIdx.x & 63;
  float top = 0.0f, sum = 0.0f, ex = 0.0f;
  int sel_id = 0;
  for (int r = 0; r < k; ++r) {
    unsigned long long mine = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) mine = key[i] > mine ? key[i] : mine;
    const uint32_t mhi = (uint32_t)(mine >> 32);
    const uint32_t hi = wave_max_u32(mhi);
    const unsigned long long at = __ballot(mhi == hi);
    const uint32_t lo = __popcll(at) == 1
                            ? __builtin_amdgcn_readlane((uint32_t)mine, __ffsll((long long)at) - 1)
                            : wave_max_u32(mhi == hi ? (uint32_t)mine : 0u);
    const int id = (int)(~lo);
    const float v = from_order_bits(hi);
    if (r == 0) top = v;
    const float e = expf(v - top);
    sum += e;
    if (lane == (id & 63)) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == (id >> 6)) key[i] = 0ull;
    }
    if (lane == r) {
      ex = e;
      sel_id = id;
    }
  }
  if (lane < k) {
    ids[lane] = sel_id;
    w[lane] = ex / sum;
    if (ids2) ids2[lane] = sel_id;
  }
}

// ids[j], w[j] (j < k) of the token whose E logits are at row; called by a full wave.
template <int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ w) {
  unsigned long long key[NPL];
  route_keys<NPL>(row, E, key);
  route_pick<NPL>(key, k, ids, w, nullptr);
}

}  // namespace moe
