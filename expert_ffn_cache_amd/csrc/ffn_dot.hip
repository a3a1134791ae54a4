// Decode-shaped expert FFN for a handful of tokens per expert: contiguous weight streaming
// with packed bf16 dot products on the vector ALUs.
//
// With one or a few tokens per expert the contraction has no reuse worth a matrix core, and
// the time is the HBM stream of the weights.  The MFMA layout (16 rows x 64 bytes per load
// instruction) caps that stream near 5.5 TB/s on MI355X; here a wave reads each weight row
// as whole 1 KB instructions (lane l takes the 16-byte chunks l, l+64, ... of the row), so
// consecutive instructions of a wave walk memory sequentially, and the loads are marked
// non-temporal (every weight byte is used once).  A wave loads the rows of its kDotUPW
// units into registers once, up front; the expert's token rows are then staged through LDS
// kDotNTL at a time (shared by the workgroup's four waves), and each lane multiplies its
// weight chunks against the same chunks of the staged rows (v_dot2_f32_bf16, fp32
// accumulation); one cross-lane sum per (weight row, token) finishes each dot product.
// Weights are read once whatever the number of rows.  Gate and up rows of a unit are
// streamed together so SiLU(g)*u is formed at once and h is written once as bf16.
#include <algorithm>

#include "ffn_args.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kDotNTL = 2;  // token rows staged in LDS at a time
constexpr int kDotUPW = 2;  // weight rows (units / output channels) per wave
constexpr int kDotUPB = 4 * kDotUPW;

// acc + a . b over 8 bf16 pairs.  The pairs are taken with shufflevector: built instead by
// bit-casting the 32-bit words of a u32x4, the chained builtin was compiled with the first
// word's registers for every step on this toolchain.
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
  const bf16x8 x = as_bf16x8(a), y = as_bf16x8(b);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                        __builtin_shufflevector(y, y, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                        __builtin_shufflevector(y, y, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                        __builtin_shufflevector(y, y, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                        __builtin_shufflevector(y, y, 6, 7), acc, false);
  return acc;
}

// One cross-lane sum per (weight row, token): DPP adds inside each 16-lane row, then the
// four row sums as scalars (no LDS round trips).
__device__ __forceinline__ float wave_sum(float v) { return wave_sum_f32(v); }

__device__ __forceinline__ u32x4 ldw_nt(const uint16_t* p, bool ok) {
  return ok ? ldg16_nt(p) : u32x4{0u, 0u, 0u, 0u};
}

// Workgroup -> active expert (one wave finds it, shared through LDS).
struct DotItem {
  int e;
  const uint16_t* w;
};

template <bool LOOP>
__device__ __forceinline__ DotItem dot_item(const FfnArgs& p, int a) {
  __shared__ int s_e;
  __shared__ const char* s_w;
  if (LOOP) __syncthreads();  // every wave has read the previous item's s_e / s_w
  if (threadIdx.x < 64) {
    const int e = nth_active_expert(p, a);
    if (threadIdx.x == 0) {
      s_e = e;
      s_w = e >= 0 ? entry_of(p, e) : nullptr;
    }
  }
  __syncthreads();
  return DotItem{s_e, (const uint16_t*)s_w};
}

// Stage rows src_row(t), t < nt, of length K (elements) into LDS rows of K.
template <typename RowOf>
__device__ __forceinline__ void stage_rows(uint16_t* lds, const uint16_t* src, int K, int nt,
                                           RowOf src_row) {
  const int nck = K >> 3;
  __syncthreads();  // the previous pass's readers are done
  for (int q = threadIdx.x; q < nt * nck; q += blockDim.x) {
    const int t = q / nck, c = q - t * nck;
    *(u32x4*)&lds[t * K + c * 8] = ldg16(src + (size_t)src_row(t) * K + c * 8);
  }
  __syncthreads();
}

// Gate/up item j = (a, unit block): kDotUPB units of the a-th active expert, one workgroup
// (4 waves); NCH = 16-byte chunks per lane per row (d <= 512 * NCH).  Dynamic LDS:
// kDotNTL x d bf16.  Returns false once the a-th active expert does not exist.
template <int NCH, bool LOOP>
__device__ __forceinline__ bool gateup_item(const FfnArgs& p, uint16_t* xs, int j) {
  const int nub = p.f / kDotUPB;
  const int a = (int)((unsigned)j / (unsigned)nub), ub = j - a * nub;
  const DotItem it = dot_item<LOOP>(p, a);
  if (it.e < 0) return false;
  if (!it.w) return true;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  int tid = threadIdx.x;
  if (LOOP) asm volatile("" : "+v"(tid));  // lane offsets recomputed per item, not held across items
  const int lane = tid & 63, wave = threadIdx.x >> 6;
  const int d = p.d, nck = d >> 3;
  uint16_t* H = (uint16_t*)p.h;
  const int u0 = ub * kDotUPB + wave * kDotUPW;
  u32x4 wg[kDotUPW][NCH], wu[kDotUPW][NCH];
#pragma unroll
  for (int uu = 0; uu < kDotUPW; ++uu) {
    const uint16_t* pg = it.w + (size_t)(u0 + uu) * d;
    const uint16_t* pu = pg + (size_t)p.f * d;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      wg[uu][i] = ldw_nt(pg + c * 8, c < nck);
      wu[uu][i] = ldw_nt(pu + c * 8, c < nck);
    }
  }
  issue_fence();
  for (int m0 = 0; m0 < n; m0 += kDotNTL) {
    const int nt = min(kDotNTL, n - m0);
    stage_rows(xs, (const uint16_t*)p.x, d, nt, [&](int t) { return p.perm[n0 + m0 + t] / p.k; });
#pragma unroll
    for (int uu = 0; uu < kDotUPW; ++uu) {
      float g[kDotNTL], u[kDotNTL];
#pragma unroll
      for (int t = 0; t < kDotNTL; ++t) g[t] = u[t] = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nck) {
#pragma unroll
          for (int t = 0; t < kDotNTL; ++t) {
            if (t < nt) {
              const u32x4 xv = *(const u32x4*)&xs[t * d + c * 8];
              g[t] = dot8(xv, wg[uu][i], g[t]);
              u[t] = dot8(xv, wu[uu][i], u[t]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kDotNTL; ++t) {
        if (t < nt) {
          const float gs = wave_sum(g[t]), us = wave_sum(u[t]);
          if (lane == 0) H[(size_t)(n0 + m0 + t) * p.f + u0 + uu] = f32_to_bf16(silu(gs) * us);
        }
      }
    }
  }
  return true;
}

// One item per workgroup, or (LOOP) a capped grid whose workgroups take items j = blockIdx.x,
// blockIdx.x + gridDim.x, ... < p.items: items are a-major, so once one finds no expert no
// later one has one.  The looping form is held to the single-item form's occupancy at d=4096.
template <int NCH, bool LOOP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LOOP && NCH == 8 ? 3 : 1)))
void dot_gateup(FfnArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  if (!LOOP) {
    gateup_item<NCH, false>(p, xs, blockIdx.x);
    return;
  }
  for (int j = blockIdx.x; j < p.items; j += gridDim.x)
    if (!gateup_item<NCH, true>(p, xs, j)) break;
}

// Down: workgroup = kDotUPB output channels of one expert; NCH chunks per lane per W_down
// row (f <= 512 * NCH); the expert's rows of h are contiguous.  Dynamic LDS: kDotNTL x f.
template <int NCH, int YDT, bool LOOP>
__device__ __forceinline__ bool down_item(const FfnArgs& p, uint16_t* hs, int j) {
  const int nub = p.d / kDotUPB;
  const int a = (int)((unsigned)j / (unsigned)nub), ub = j - a * nub;
  const DotItem it = dot_item<LOOP>(p, a);
  if (it.e < 0) return false;
  if (!it.w) return true;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int f = p.f, nck = f >> 3;
  const uint16_t* Wd = it.w + 2 * (size_t)f * p.d;
  const int o0 = ub * kDotUPB + wave * kDotUPW;
  u32x4 wv[kDotUPW][NCH];
#pragma unroll
  for (int uu = 0; uu < kDotUPW; ++uu) {
    const uint16_t* pw = Wd + (size_t)(o0 + uu) * f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      wv[uu][i] = ldw_nt(pw + c * 8, c < nck);
    }
  }
  issue_fence();
  for (int m0 = 0; m0 < n; m0 += kDotNTL) {
    const int nt = min(kDotNTL, n - m0);
    stage_rows(hs, (const uint16_t*)p.h, f, nt, [&](int t) { return n0 + m0 + t; });
#pragma unroll
    for (int uu = 0; uu < kDotUPW; ++uu) {
      float acc[kDotNTL];
#pragma unroll
      for (int t = 0; t < kDotNTL; ++t) acc[t] = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nck) {
#pragma unroll
          for (int t = 0; t < kDotNTL; ++t)
            if (t < nt) acc[t] = dot8(*(const u32x4*)&hs[t * f + c * 8], wv[uu][i], acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < kDotNTL; ++t) {
        if (t < nt) {
          const float s = wave_sum(acc[t]);
          if (lane == 0) {
            const size_t o = (size_t)(n0 + m0 + t) * p.d + o0 + uu;
            if (YDT == MOE_F32) ((float*)p.y)[o] = s;
            else ((uint16_t*)p.y)[o] = f32_to_bf16(s);
          }
        }
      }
    }
  }
  return true;
}

template <int NCH, int YDT, bool LOOP>
__global__ __launch_bounds__(256) void dot_down(FfnArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
  if (!LOOP) {
    down_item<NCH, YDT, false>(p, hs, blockIdx.x);
    return;
  }
  for (int j = blockIdx.x; j < p.items; j += gridDim.x)
    if (!down_item<NCH, YDT, true>(p, hs, j)) break;
}

int nch_of(int k_elems) {  // 16-byte chunks per lane for a row of k_elems, or 0 if too long
  const int c = (k_elems / 8 + 63) / 64;
  return c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : c <= 16 ? 16 : 0;
}

// Grid of a launch over `items` items: one workgroup per item, or with rounds > 0 and more
// items than that many full rounds of resident workgroups, exactly those rounds (the kernel's
// occupancy at this LDS size, queried from the runtime) of looping workgroups.
template <typename K>
int dot_grid(K kernel, size_t lds, int items, int rounds, bool& loop) {
  loop = false;
  if (rounds <= 0) return items;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, lds) != hipSuccess || occ <= 0)
    occ = 1;
  const long long cap = (long long)rounds * occ * num_cus();
  if (items <= cap) return items;
  loop = true;
  return (int)cap;
}

template <int NCH>
void launch_gu(const FfnArgs& p, int rounds, hipStream_t s) {
  const size_t lds = (size_t)kDotNTL * p.d * 2;
  bool loop;
  const int g = dot_grid(dot_gateup<NCH, true>, lds, p.items, rounds, loop);
  if (loop) hipLaunchKernelGGL((dot_gateup<NCH, true>), dim3(g), dim3(256), lds, s, p);
  else hipLaunchKernelGGL((dot_gateup<NCH, false>), dim3(g), dim3(256), lds, s, p);
}

template <int NCH, int YDT>
void launch_dn_t(const FfnArgs& p, int rounds, hipStream_t s) {
  const size_t lds = (size_t)kDotNTL * p.f * 2;
  bool loop;
  const int g = dot_grid(dot_down<NCH, YDT, true>, lds, p.items, rounds, loop);
  if (loop) hipLaunchKernelGGL((dot_down<NCH, YDT, true>), dim3(g), dim3(256), lds, s, p);
  else hipLaunchKernelGGL((dot_down<NCH, YDT, false>), dim3(g), dim3(256), lds, s, p);
}

template <int NCH>
void launch_dn(const FfnArgs& p, bool yf, int rounds, hipStream_t s) {
  if (yf) launch_dn_t<NCH, MOE_F32>(p, rounds, s);
  else launch_dn_t<NCH, MOE_BF16>(p, rounds, s);
}

}  // namespace

bool ffn_dot_supported(int d, int f) { return nch_of(d) > 0 && nch_of(f) > 0; }

int launch_ffn_dot(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts, int parts,
                   int rounds) {
  if (experts <= 0) return MOE_OK;
  FfnArgs pg = p, pd = p;
  pg.items = experts * (p.f / kDotUPB);
  pd.items = experts * (p.d / kDotUPB);
  const bool yf = y_dtype == MOE_F32;
  if (parts & 1) {
    switch (nch_of(p.d)) {
      case 2: launch_gu<2>(pg, rounds, stream); break;
      case 4: launch_gu<4>(pg, rounds, stream); break;
      case 8: launch_gu<8>(pg, rounds, stream); break;
      case 16: launch_gu<16>(pg, rounds, stream); break;
      default: return MOE_EINVAL;
    }
    MOE_LAUNCH_CHECK();
  }
  if (parts & 2) {
    switch (nch_of(p.f)) {
      case 2: launch_dn<2>(pd, yf, rounds, stream); break;
      case 4: launch_dn<4>(pd, yf, rounds, stream); break;
      case 8: launch_dn<8>(pd, yf, rounds, stream); break;
      case 16: launch_dn<16>(pd, yf, rounds, stream); break;
      default: return MOE_EINVAL;
    }
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
