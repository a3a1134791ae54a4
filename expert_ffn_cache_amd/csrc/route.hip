// Router logits (helper) and top-k softmax routing: one 64-wide wavefront per token,
// four tokens per workgroup (the per-token routing is in route_dev.h).
#include "route_dev.h"

using namespace moe;

namespace {

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_softmax(const float* __restrict__ logits, int T,
                                                          int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<NPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
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
