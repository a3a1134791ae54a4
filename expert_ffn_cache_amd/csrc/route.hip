// Router logits (helper) and top-k softmax routing.
//
// Top-k with a softmax gate: a token chooses a few of the routed experts, e.g.
// 6 of 256 for DeepSeek-V4-Flash (FreeToken RTX-4090 page, "How the MoE memory
// hierarchy works").  Order: larger logit first, equal values by lower id.
//
// One 64-wide wavefront per token.  Each lane holds ceil(E/64) logits in
// registers (lane l owns experts l, l+64, ...).  Each of the k rounds is a
// wave-wide max over a 64-bit key (order-preserving logit bits, then the
// complemented expert id so that ties go to the lower id), taken as two 32-bit
// maxima (the high word, then the low word among the lanes that hold that high
// word) with DPP moves and scalar read-outs, so a round makes no LDS round trip;
// the owner lane retires the winner.  The softmax over the k winners is done
// in registers (lane j holds winner j) and written coalesced.
#include "common.h"
#include "wave.h"

using namespace moe;

namespace {

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);  // -0 and +0 compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_softmax(const float* __restrict__ logits, int T,
                                                          int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  unsigned long long key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ((unsigned long long)order_bits(row[e]) << 32) | (uint32_t)(~(uint32_t)e) : 0ull;
  }
  float sel_v = 0.0f, top = 0.0f;
  int sel_id = 0;
  for (int r = 0; r < k; ++r) {
    unsigned long long mine = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) mine = key[i] > mine ? key[i] : mine;
    const uint32_t hi = wave_max_u32((uint32_t)(mine >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(mine >> 32) == hi ? (uint32_t)mine : 0u);
    const unsigned long long best = ((unsigned long long)hi << 32) | lo;
    const int id = (int)(~(uint32_t)best);
    const float v = from_order_bits((uint32_t)(best >> 32));
    if (r == 0) top = v;
    if (lane == (id & 63)) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == (id >> 6)) key[i] = 0ull;
    }
    if (lane == r) {
      sel_v = v;
      sel_id = id;
    }
  }
  const float ex = lane < k ? expf(sel_v - top) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = sel_id;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

// logits[t][e] = sum_c x[t][c] * wr[e][c] (fp32).  One thread per (t, e); tiny shapes only.
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ x,
                                                         const float* __restrict__ wr, int T, int d,
                                                         int E, float* __restrict__ out) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * E) return;
  const int t = idx / E, e = idx % E;
  const float* xr = x + (size_t)t * d;
  const float* wrow = wr + (size_t)e * d;
  float s = 0.0f;
  for (int c = 0; c < d; ++c) s = fmaf(xr[c], wrow[c], s);
  out[idx] = s;
}

}  // namespace

extern "C" int moe_router_logits(const void* x, const void* w_router, int dtype, int T, int d, int E,
                                 float* logits, hipStream_t stream) {
  if (T < 0 || d <= 0 || E <= 0 || E > kMaxE) return MOE_EINVAL;
  if ((long long)T * E >= (1ll << 31)) return MOE_EINVAL;
  if (dtype != MOE_F32) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_EINVAL;
  const int n = T * E;
  hipLaunchKernelGGL(router_logits_f32, dim3((n + 255) / 256), dim3(256), 0, stream,
                     (const float*)x, (const float*)w_router, T, d, E, logits);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                         float* topk_w, hipStream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || k <= 0 || k > kMaxK || k > E) return MOE_EINVAL;
  if ((long long)T * E >= (1ll << 31)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_EINVAL;
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_topk_softmax<1>, grid, block, 0, stream, logits, T, E, k, topk_ids, topk_w);
  else if (E <= 128)
    hipLaunchKernelGGL(route_topk_softmax<2>, grid, block, 0, stream, logits, T, E, k, topk_ids, topk_w);
  else if (E <= 256)
    hipLaunchKernelGGL(route_topk_softmax<4>, grid, block, 0, stream, logits, T, E, k, topk_ids, topk_w);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_softmax<8>, grid, block, 0, stream, logits, T, E, k, topk_ids, topk_w);
  else
    hipLaunchKernelGGL(route_topk_softmax<16>, grid, block, 0, stream, logits, T, E, k, topk_ids, topk_w);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
