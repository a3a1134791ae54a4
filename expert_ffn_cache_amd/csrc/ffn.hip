// Expert SwiGLU FFNs over tokens grouped by expert.
//
// For every active expert e and its grouped rows p in [offsets[e], offsets[e+1]):
//   h = SiLU(x[perm[p]/k] W_gate^T) * (x[perm[p]/k] W_up^T),   y_perm[p] = h W_down^T
// (the GPU runs the experts it holds on the tokens routed to them: FreeToken
// RTX-4090 page, component table; SwiGLU form and no biases are a reading).
// Weights of e are the cache entry at arena + expert_slot[e] * stride:
//   [W_gate f x d][W_up f x d][W_down d x f], contraction index contiguous.
//
// Three paths:
//  * fp32 (MOE_F32 weights): plain fp32 FMA loops; small shapes only.
//  * GEMV (bf16, decode-shaped counts, n_e <= a few tokens): weight streaming.
//    Each wavefront owns 16 weight rows and streams them straight from HBM into
//    registers with 16-byte loads (4 lanes cover 64 contiguous bytes of a row,
//    two loads per step make a full 128-byte line), multiplying against up to
//    16*MC token rows with v_mfma_f32_16x16x32_bf16.  No LDS staging: every
//    weight byte is used once, so the kernel is HBM-bound and latency is hidden
//    by occupancy plus one step of register prefetch.
//  * GEMM (bf16, prefill-shaped counts): LDS-tiled grouped GEMM on
//    v_mfma_f32_32x32x16_bf16, 128x128x64 tiles, double-buffered LDS with an
//    XOR swizzle, A rows gathered through perm, persistent workgroups walking
//    a device-derived (expert, n-tile, m-tile) list.
// Both bf16 paths fuse SiLU(g)*u into the gate/up epilogue: gate and up rows
// of the same unit land in the same lane and register, so h is formed without
// data exchange and written once as bf16.
//
// The MFMA reduction index is a permutation of the physical k inside each
// 64-wide step (A and B fragments use the same permutation), which is what
// lets each lane load 32 contiguous bytes per row.
#include <algorithm>

#include "common.h"

using namespace moe;

namespace {

struct FfnArgs {
  const void* x;
  const int32_t* perm;
  const int32_t* offsets;
  int k, E, d, f;
  const int32_t* expert_slot;
  const char* arena;
  size_t stride;
  const uint8_t* mask;
  const int32_t* slot_key;
  int key_base;
  void* h;
  void* y;
  int32_t* status;
};

// Weights of expert e, or nullptr (and MOE_ERANGE) for a missing or stale slot.
__device__ __forceinline__ const char* entry_of(const FfnArgs& p, int e) {
  const int s = p.expert_slot ? p.expert_slot[e] : e;
  if (s < 0 || (p.slot_key && p.slot_key[s] != p.key_base + e)) {
    set_status(p.status, MOE_ERANGE);
    return nullptr;
  }
  return p.arena + (size_t)s * p.stride;
}

__device__ __forceinline__ bool active(const FfnArgs& p, int e) {
  return p.offsets[e + 1] > p.offsets[e] && (!p.mask || p.mask[e]);
}

// The a-th active expert in ascending id order, or -1; called by one full wave.
__device__ int nth_active_expert(const FfnArgs& p, int a) {
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int e0 = 0; e0 < p.E; e0 += 64) {
    const int e = e0 + lane;
    const bool act = e < p.E && active(p, e);
    const unsigned long long m = __ballot(act);
    const int c = __popcll(m);
    if (a < seen + c) {
      const bool mine = act && __popcll(m & lanemask_lt(lane)) == a - seen;
      return e0 + __ffsll((long long)__ballot(mine)) - 1;
    }
    seen += c;
  }
  return -1;
}

// ------------------------------------------------------------------ fp32 path
__global__ __launch_bounds__(64) void f32_gateup(FfnArgs p) {
  const int e = blockIdx.x;
  if (!active(p, e)) return;
  const char* w = entry_of(p, e);
  if (!w) return;
  const int i = blockIdx.y * 64 + threadIdx.x;
  const float* wg = (const float*)w + (size_t)i * p.d;
  const float* wu = wg + (size_t)p.f * p.d;
  const float* X = (const float*)p.x;
  float* H = (float*)p.h;
  for (int q = p.offsets[e]; q < p.offsets[e + 1]; ++q) {
    const float* xr = X + (size_t)(p.perm[q] / p.k) * p.d;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < p.d; ++c) {
      g = fmaf(xr[c], wg[c], g);
      u = fmaf(xr[c], wu[c], u);
    }
    H[(size_t)q * p.f + i] = g / (1.0f + expf(-g)) * u;
  }
}

__global__ __launch_bounds__(64) void f32_down(FfnArgs p) {
  const int e = blockIdx.x;
  if (!active(p, e)) return;
  const char* w = entry_of(p, e);
  if (!w) return;
  const int o = blockIdx.y * 64 + threadIdx.x;
  const float* wd = (const float*)w + 2 * (size_t)p.f * p.d + (size_t)o * p.f;
  const float* H = (const float*)p.h;
  float* Y = (float*)p.y;
  for (int q = p.offsets[e]; q < p.offsets[e + 1]; ++q) {
    const float* hr = H + (size_t)q * p.f;
    float s = 0.f;
    for (int i = 0; i < p.f; ++i) s = fmaf(hr[i], wd[i], s);
    Y[(size_t)q * p.d + o] = s;
  }
}

// ------------------------------------------------------------------ GEMV path
// Shared prologue: workgroup -> (active expert, 64-row block).
struct GemvItem {
  int e;
  const uint16_t* w;
};

__device__ __forceinline__ GemvItem gemv_item(const FfnArgs& p, int a) {
  __shared__ int s_e;
  __shared__ const char* s_w;
  if (threadIdx.x < 64) {
    const int e = nth_active_expert(p, a);
    if (threadIdx.x == 0) {
      s_e = e;
      s_w = e >= 0 ? entry_of(p, e) : nullptr;
    }
  }
  __syncthreads();
  return GemvItem{s_e, (const uint16_t*)s_w};
}

// Gate/up: wave owns units i0..i0+15 of W_gate and W_up; MC chunks of 16 tokens.
template <int MC>
__global__ __launch_bounds__(256) void gemv_gateup(FfnArgs p) {
  const int nrb = p.f >> 6;
  const int a = blockIdx.x / nrb, rb = blockIdx.x - a * nrb;
  const GemvItem it = gemv_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int i0 = rb * 64 + wave * 16;
  const int d = p.d;
  const uint16_t* pg = it.w + (size_t)(i0 + col) * d + kg * 16;
  const uint16_t* pu = pg + (size_t)p.f * d;
  const uint16_t* X = (const uint16_t*)p.x;
  uint16_t* H = (uint16_t*)p.h;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
    const uint16_t* px[MC];
    bool vx[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      const int r = m0 + mc * 16 + col;
      vx[mc] = r < n;
      px[mc] = X + (size_t)(vx[mc] ? p.perm[n0 + r] / p.k : 0) * d + kg * 16;
    }
    f32x4 ag[MC], au[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      ag[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mc] = ag[mc];
    }
    u32x4 bg0 = ldg16(pg), bg1 = ldg16(pg + 8), bu0 = ldg16(pu), bu1 = ldg16(pu + 8);
    u32x4 ax0[MC], ax1[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      ax0[mc] = vx[mc] ? ldg16(px[mc]) : zero;
      ax1[mc] = vx[mc] ? ldg16(px[mc] + 8) : zero;
    }
    for (int kk = 0; kk < d; kk += 64) {
      u32x4 nbg0 = zero, nbg1 = zero, nbu0 = zero, nbu1 = zero, nax0[MC], nax1[MC];
      const int kn = kk + 64;
      if (kn < d) {
        nbg0 = ldg16(pg + kn);
        nbg1 = ldg16(pg + kn + 8);
        nbu0 = ldg16(pu + kn);
        nbu1 = ldg16(pu + kn + 8);
      }
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        nax0[mc] = (kn < d && vx[mc]) ? ldg16(px[mc] + kn) : zero;
        nax1[mc] = (kn < d && vx[mc]) ? ldg16(px[mc] + kn + 8) : zero;
      }
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        if (m0 + mc * 16 < n) {
          ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax0[mc]), as_bf16x8(bg0), ag[mc], 0, 0, 0);
          au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax0[mc]), as_bf16x8(bu0), au[mc], 0, 0, 0);
          ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax1[mc]), as_bf16x8(bg1), ag[mc], 0, 0, 0);
          au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax1[mc]), as_bf16x8(bu1), au[mc], 0, 0, 0);
        }
      }
      bg0 = nbg0; bg1 = nbg1; bu0 = nbu0; bu1 = nbu1;
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        ax0[mc] = nax0[mc];
        ax1[mc] = nax1[mc];
      }
    }
    // lane holds C[4*kg + i][col] of each 16x16 tile: token rows, unit columns
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mc * 16 + kg * 4 + i;
        if (m < n)
          H[(size_t)(n0 + m) * p.f + i0 + col] = f32_to_bf16(silu(ag[mc][i]) * au[mc][i]);
      }
    }
  }
}

// Down: wave owns output channels o0..o0+15 of W_down; rows of h are contiguous.
template <int MC, int YDT>
__global__ __launch_bounds__(256) void gemv_down(FfnArgs p) {
  const int nrb = p.d >> 6;
  const int a = blockIdx.x / nrb, rb = blockIdx.x - a * nrb;
  const GemvItem it = gemv_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int o0 = rb * 64 + wave * 16;
  const int f = p.f;
  const uint16_t* pw = it.w + 2 * (size_t)f * p.d + (size_t)(o0 + col) * f + kg * 16;
  const uint16_t* H = (const uint16_t*)p.h;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
    const uint16_t* ph[MC];
    bool vh[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      const int r = m0 + mc * 16 + col;
      vh[mc] = r < n;
      ph[mc] = H + (size_t)(n0 + (vh[mc] ? r : 0)) * f + kg * 16;
    }
    f32x4 acc[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) acc[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 b0 = ldg16(pw), b1 = ldg16(pw + 8);
    u32x4 a0[MC], a1[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      a0[mc] = vh[mc] ? ldg16(ph[mc]) : zero;
      a1[mc] = vh[mc] ? ldg16(ph[mc] + 8) : zero;
    }
    for (int kk = 0; kk < f; kk += 64) {
      const int kn = kk + 64;
      u32x4 nb0 = zero, nb1 = zero, na0[MC], na1[MC];
      if (kn < f) {
        nb0 = ldg16(pw + kn);
        nb1 = ldg16(pw + kn + 8);
      }
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        na0[mc] = (kn < f && vh[mc]) ? ldg16(ph[mc] + kn) : zero;
        na1[mc] = (kn < f && vh[mc]) ? ldg16(ph[mc] + kn + 8) : zero;
      }
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        if (m0 + mc * 16 < n) {
          acc[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[mc]), as_bf16x8(b0), acc[mc], 0, 0, 0);
          acc[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[mc]), as_bf16x8(b1), acc[mc], 0, 0, 0);
        }
      }
      b0 = nb0; b1 = nb1;
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) {
        a0[mc] = na0[mc];
        a1[mc] = na1[mc];
      }
    }
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mc * 16 + kg * 4 + i;
        if (m < n) {
          const size_t o = (size_t)(n0 + m) * p.d + o0 + col;
          if (YDT == MOE_F32) ((float*)p.y)[o] = acc[mc][i];
          else ((uint16_t*)p.y)[o] = f32_to_bf16(acc[mc][i]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ GEMM path
constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int kGateUp = 0, kDown = 1;

__device__ __forceinline__ int swz(int r, int c) { return r * GBK + ((c ^ (r & 7)) << 3); }

template <int MODE, int YDT>
__global__ __launch_bounds__(256, 2) void gemm_grouped(FfnArgs p, int n_ntiles) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][GBM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][GBN * GBK];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_wave[4];
  __shared__ int s_total;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // m-tiles per expert, prefix over experts (4 experts per thread, E <= 1024)
  {
    int c[4], tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      c[q] = 0;
      if (e < p.E && active(p, e)) c[q] = (p.offsets[e + 1] - p.offsets[e] + GBM - 1) / GBM;
      tot += c[q];
    }
    int x = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int w = 0; w < 4; ++w) { const int v = s_wave[w]; s_wave[w] = run; run += v; }
      s_total = run;
    }
    __syncthreads();
    int run = s_wave[wave] + x - tot;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e < p.E) s_pref[e] = run;
      run += c[q];
    }
    if (tid == 0) s_pref[p.E] = s_total;
    __syncthreads();
  }
  const int total_items = s_total * n_ntiles;
  const int K = MODE == kGateUp ? p.d : p.f;
  const int wm = wave >> 1, wn = wave & 1;
  const int cc = tid & 7, r0 = tid >> 3;  // loader: rows r0 + 32q, 16-byte chunk cc

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int q = item / n_ntiles;
    int lo = 0, hi = p.E;  // largest e with s_pref[e] <= q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int mt_e = s_pref[e + 1] - s_pref[e];
    const int local = item - s_pref[e] * n_ntiles;
    const int nt = local / mt_e, mt = local - nt * mt_e;
    const char* wbase = entry_of(p, e);
    if (!wbase) continue;
    const uint16_t* W = (const uint16_t*)wbase;
    const int n0 = p.offsets[e] + mt * GBM;
    const int rows = min(GBM, p.offsets[e + 1] - n0);

    const uint16_t* srcA[4];
    const uint16_t* srcB[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 32 * qq;
      if (MODE == kGateUp) {
        srcA[qq] = r < rows ? (const uint16_t*)p.x + (size_t)(p.perm[n0 + r] / p.k) * p.d + cc * 8 : nullptr;
        const int unit = nt * 64 + (r & 63);
        srcB[qq] = W + (r >= 64 ? (size_t)p.f * p.d : 0) + (size_t)unit * p.d + cc * 8;
      } else {
        srcA[qq] = r < rows ? (const uint16_t*)p.h + (size_t)(n0 + r) * p.f + cc * 8 : nullptr;
        const int o = nt * GBN + r;
        srcB[qq] = o < p.d ? W + 2 * (size_t)p.f * p.d + (size_t)o * p.f + cc * 8 : nullptr;
      }
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 ra[4], rb[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      ra[qq] = srcA[qq] ? ldg16(srcA[qq]) : zero;
      rb[qq] = srcB[qq] ? ldg16(srcB[qq]) : zero;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    __syncthreads();  // previous item's readers are done with buffer 0
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      *(u32x4*)&sA[0][swz(r0 + 32 * qq, cc)] = ra[qq];
      *(u32x4*)&sB[0][swz(r0 + 32 * qq, cc)] = rb[qq];
    }
    __syncthreads();
    const int nk = K / GBK;
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      const bool more = ks + 1 < nk;
      if (more) {
        const int kn = (ks + 1) * GBK;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          ra[qq] = srcA[qq] ? ldg16(srcA[qq] + kn) : zero;
          rb[qq] = srcB[qq] ? ldg16(srcB[qq] + kn) : zero;
        }
      }
#pragma unroll
      for (int s = 0; s < GBK / 16; ++s) {
        const int ch = s * 2 + (lane >> 5);
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + (lane & 31);
          af[i] = as_bf16x8(*(const u32x4*)&sA[buf][swz(r, ch)]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = MODE == kGateUp ? j * 64 + wn * 32 + (lane & 31) : wn * 64 + j * 32 + (lane & 31);
          bfr[j] = as_bf16x8(*(const u32x4*)&sB[buf][swz(r, ch)]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (more) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          *(u32x4*)&sA[buf ^ 1][swz(r0 + 32 * qq, cc)] = ra[qq];
          *(u32x4*)&sB[buf ^ 1][swz(r0 + 32 * qq, cc)] = rb[qq];
        }
      }
      __syncthreads();
    }
    // epilogue: lane holds C[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 tile
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= rows) continue;
        if (MODE == kGateUp) {
          const int unit = nt * 64 + wn * 32 + (lane & 31);
          ((uint16_t*)p.h)[(size_t)(n0 + m) * p.f + unit] = f32_to_bf16(silu(acc[i][0][v]) * acc[i][1][v]);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int o = nt * GBN + wn * 64 + j * 32 + (lane & 31);
            if (o < p.d) {
              const size_t idx = (size_t)(n0 + m) * p.d + o;
              if (YDT == MOE_F32) ((float*)p.y)[idx] = acc[i][j][v];
              else ((uint16_t*)p.y)[idx] = f32_to_bf16(acc[i][j][v]);
            }
          }
        }
      }
    }
  }
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

extern "C" size_t moe_expert_ffn_workspace_bytes(int T, int k, int f, int act_dtype) {
  if (T <= 0 || k <= 0 || f <= 0) return 256;
  const size_t el = act_dtype == MOE_F32 ? 4 : 2;
  return ((size_t)T * k * f * el + 255) / 256 * 256;
}

extern "C" int moe_expert_ffn(const void* x, int act_dtype, const int32_t* perm,
                              const int32_t* offsets, int T, int k, int E, int d, int f,
                              const int32_t* expert_slot, const void* arena, size_t entry_stride,
                              int w_dtype, const uint8_t* expert_mask, const int32_t* slot_key,
                              int key_base, void* ws, size_t ws_bytes, void* y_perm, int y_dtype,
                              int path, int32_t* status, hipStream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || k <= 0 || k > kMaxK || k > E) return MOE_EINVAL;
  if (d <= 0 || f <= 0 || d % 64 != 0 || f % 64 != 0) return MOE_EINVAL;
  if ((long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM) return MOE_EINVAL;
  const bool f32 = w_dtype == MOE_F32;
  if (f32) {
    if (act_dtype != MOE_F32 || y_dtype != MOE_F32) return MOE_EUNSUPPORTED;
  } else if (w_dtype == MOE_BF16) {
    if (act_dtype != MOE_BF16 || (y_dtype != MOE_F32 && y_dtype != MOE_BF16)) return MOE_EUNSUPPORTED;
  } else {
    return MOE_EUNSUPPORTED;
  }
  const size_t el = f32 ? 4 : 2;
  if (entry_stride < 3 * (size_t)d * f * el || entry_stride % 16 != 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !perm || !offsets || !arena || !ws || !y_perm) return MOE_EINVAL;
  if (!moe_aligned16(x) || !moe_aligned16(arena) || !moe_aligned16(ws) || !moe_aligned16(y_perm))
    return MOE_EINVAL;
  if (ws_bytes < moe_expert_ffn_workspace_bytes(T, k, f, act_dtype)) return MOE_EINVAL;

  FfnArgs p{x, perm, offsets, k, E, d, f, expert_slot, (const char*)arena, entry_stride,
            expert_mask, slot_key, key_base, ws, y_perm, status};
  if (f32) {
    hipLaunchKernelGGL(f32_gateup, dim3(E, f / 64), dim3(64), 0, stream, p);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(f32_down, dim3(E, d / 64), dim3(64), 0, stream, p);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  if (path == MOE_PATH_AUTO) path = (long long)T * k <= 8ll * E ? MOE_PATH_GEMV : MOE_PATH_GEMM;
  if (path == MOE_PATH_GEMV) {
    const int amax = (int)std::min<long long>(E, (long long)T * k);
    const dim3 gu(amax * (f / 64)), dn(amax * (d / 64)), blk(256);
    const bool yf = y_dtype == MOE_F32;
    if (T <= 16) {
      hipLaunchKernelGGL(gemv_gateup<1>, gu, blk, 0, stream, p);
      MOE_LAUNCH_CHECK();
      if (yf) hipLaunchKernelGGL((gemv_down<1, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<1, MOE_BF16>), dn, blk, 0, stream, p);
    } else if (T <= 32) {
      hipLaunchKernelGGL(gemv_gateup<2>, gu, blk, 0, stream, p);
      MOE_LAUNCH_CHECK();
      if (yf) hipLaunchKernelGGL((gemv_down<2, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<2, MOE_BF16>), dn, blk, 0, stream, p);
    } else {
      hipLaunchKernelGGL(gemv_gateup<4>, gu, blk, 0, stream, p);
      MOE_LAUNCH_CHECK();
      if (yf) hipLaunchKernelGGL((gemv_down<4, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<4, MOE_BF16>), dn, blk, 0, stream, p);
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  const dim3 grid(num_cus() * 2), blk(256);
  hipLaunchKernelGGL((gemm_grouped<kGateUp, MOE_BF16>), grid, blk, 0, stream, p, f / 64);
  MOE_LAUNCH_CHECK();
  const int ntd = (d + GBN - 1) / GBN;
  if (y_dtype == MOE_F32)
    hipLaunchKernelGGL((gemm_grouped<kDown, MOE_F32>), grid, blk, 0, stream, p, ntd);
  else
    hipLaunchKernelGGL((gemm_grouped<kDown, MOE_BF16>), grid, blk, 0, stream, p, ntd);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
