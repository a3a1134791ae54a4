// Weighted combine: out[t] = sum_j w[t][j] * y_perm[inv[t*k + j]], j ascending.
//
// A gather, not a scatter: each output row reads its k expert rows, so no
// atomics are needed and the sum order is fixed.  One workgroup per (token,
// 2048-column slice); each thread owns 8 consecutive columns (two float4 of
// fp32 rows or one 16-byte load of bf16 rows).  HBM-bound.
#include "common.h"

using namespace moe;

namespace {

template <int YDT>
__global__ __launch_bounds__(256) void combine_gather(const void* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k, int d,
                                                      float* __restrict__ out) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 2048 + threadIdx.x * 8;
  if (c >= d) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = inv[(size_t)t * k + j];
    const float wj = w[(size_t)t * k + j];
    if (YDT == MOE_F32) {
      const float* row = (const float*)y + (size_t)p * d + c;
      const f32x4 v0 = *(const f32x4*)row, v1 = *(const f32x4*)(row + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = fmaf(wj, v0[q], acc[q]);
        acc[4 + q] = fmaf(wj, v1[q], acc[4 + q]);
      }
    } else {
      const u32x4 v = ldg16((const uint16_t*)y + (size_t)p * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wj, __uint_as_float(v[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj, __uint_as_float(v[q] & 0xFFFF0000u), acc[2 * q + 1]);
      }
    }
  }
  float* o = out + (size_t)t * d + c;
  *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

}  // namespace

extern "C" int moe_combine(const void* y_perm, int y_dtype, const int32_t* inv, const float* topk_w,
                           int T, int k, int d, float* out, hipStream_t stream) {
  if (T < 0 || k <= 0 || k > kMaxK || d <= 0 || d % 64 != 0) return MOE_EINVAL;
  if ((long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv || !topk_w || !out) return MOE_EINVAL;
  if (!moe_aligned16(y_perm) || !moe_aligned16(out)) return MOE_EINVAL;
  const dim3 grid(T, (d + 2047) / 2048);
  if (y_dtype == MOE_F32)
    hipLaunchKernelGGL(combine_gather<MOE_F32>, grid, dim3(256), 0, stream, y_perm, inv, topk_w, k, d, out);
  else
    hipLaunchKernelGGL(combine_gather<MOE_BF16>, grid, dim3(256), 0, stream, y_perm, inv, topk_w, k, d, out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
