// Weighted combine: out[t] = sum_j w[t][j] * y_perm[inv[t*k + j]], j ascending.
//
// A gather, not a scatter: each output row reads its k expert rows, so no
// atomics are needed and the sum order is fixed.  One workgroup per (token,
// 2048-column slice); each thread owns 8 consecutive columns (two float4 of
// fp32 rows or one 16-byte load of bf16 rows).  HBM-bound.
#include "common.h"

using namespace moe;

namespace {

// KMAX >= k: the k row indices and weights are read first, then all k rows are loaded
// together (independent loads in flight), then summed in ascending j.
template <int YDT, int KMAX>
__global__ __launch_bounds__(256) void combine_gather(const void* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k, int d,
                                                      float* __restrict__ out) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 2048 + threadIdx.x * 8;
  if (c >= d) return;
  int p[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      p[j] = inv[(size_t)t * k + j];
      wj[j] = w[(size_t)t * k + j];
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (YDT == MOE_F32) {
    f32x4 v0[KMAX], v1[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const float* row = (const float*)y + (size_t)p[j] * d + c;
        v0[j] = *(const f32x4*)row;
        v1[j] = *(const f32x4*)(row + 4);
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[q] = fmaf(wj[j], v0[j][q], acc[q]);
          acc[4 + q] = fmaf(wj[j], v1[j][q], acc[4 + q]);
        }
      }
    }
  } else {
    u32x4 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) v[j] = ldg16((const uint16_t*)y + (size_t)p[j] * d + c);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(wj[j], __uint_as_float(v[j][q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wj[j], __uint_as_float(v[j][q] & 0xFFFF0000u), acc[2 * q + 1]);
        }
      }
    }
  }
  float* o = out + (size_t)t * d + c;
  *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

template <int YDT>
void launch_combine(dim3 grid, hipStream_t stream, const void* y, const int32_t* inv,
                    const float* w, int k, int d, float* out) {
  if (k <= 8)
    hipLaunchKernelGGL((combine_gather<YDT, 8>), grid, dim3(256), 0, stream, y, inv, w, k, d, out);
  else
    hipLaunchKernelGGL((combine_gather<YDT, kMaxK>), grid, dim3(256), 0, stream, y, inv, w, k, d, out);
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
    launch_combine<MOE_F32>(grid, stream, y_perm, inv, topk_w, k, d, out);
  else
    launch_combine<MOE_BF16>(grid, stream, y_perm, inv, topk_w, k, d, out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
