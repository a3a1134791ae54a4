// Decode-shaped expert FFN: weight streaming with v_mfma_f32_16x16x32_bf16.
//
// Each wavefront owns 16 weight rows (or two groups of 16, sharing every token fragment it
// loads) and streams them straight from HBM into registers with 16-byte loads (4 lanes
// cover 64 contiguous bytes of a row, two loads per step make a full 128-byte line),
// multiplying against up to 16*MC token rows read from L2.  No LDS staging: every
// weight byte is used once, so the kernels are HBM-bound and latency is hidden by
// occupancy plus one step of register prefetch.  SiLU(g)*u is fused into the gate/up
// epilogue: gate and up rows of one unit land in the same lane and register.
//
// The MFMA reduction index is a permutation of the physical k inside each 64-wide step
// (A and B fragments use the same permutation), which lets each lane load 32 contiguous
// bytes per row.
#include <algorithm>

#include "ffn_args.h"

namespace moe {
namespace {

// Shared prologue: workgroup -> (active expert, block of 64 or 128 rows).
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

// Gate/up: wave owns units i0..i0+16NG-1 of W_gate and W_up; MC chunks of 16 tokens.
// Two register sets alternate (no register rotation), so the next step's loads stay in
// flight while the current step's MFMAs run.  Token rows beyond the expert load a valid
// row and their (unused) output rows are not stored: an MFMA output row depends only
// on its own input row.
template <int MC, int NG>
struct GuStage {
  u32x4 g0[NG], g1[NG], u0[NG], u1[NG];
  u32x4 a0[MC], a1[MC];
};

// gstride: elements between the wave's unit groups (16 rows)
template <int MC, int NG>
__device__ __forceinline__ void gu_load(GuStage<MC, NG>& s, const uint16_t* pg, const uint16_t* pu,
                                        size_t gstride, const uint16_t* const (&px)[MC], int kk) {
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    s.g0[q] = ldg16(pg + q * gstride + kk);
    s.g1[q] = ldg16(pg + q * gstride + kk + 8);
    s.u0[q] = ldg16(pu + q * gstride + kk);
    s.u1[q] = ldg16(pu + q * gstride + kk + 8);
  }
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    s.a0[mc] = ldg16(px[mc] + kk);
    s.a1[mc] = ldg16(px[mc] + kk + 8);
  }
  issue_fence();
}

template <int MC, int NG>
__device__ __forceinline__ void gu_mma(const GuStage<MC, NG>& s, f32x4 (&ag)[NG][MC],
                                       f32x4 (&au)[NG][MC], int live) {
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    if (mc < live) {
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        ag[q][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a0[mc]), as_bf16x8(s.g0[q]), ag[q][mc], 0, 0, 0);
        au[q][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a0[mc]), as_bf16x8(s.u0[q]), au[q][mc], 0, 0, 0);
        ag[q][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a1[mc]), as_bf16x8(s.g1[q]), ag[q][mc], 0, 0, 0);
        au[q][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a1[mc]), as_bf16x8(s.u1[q]), au[q][mc], 0, 0, 0);
      }
    }
  }
}

// One pass over up to 16 MC token rows m0.. of the expert (MC chunks of 16 rows); the wave's
// NG groups of 16 units share every token fragment it loads.
template <int MC, int NG>
__device__ __forceinline__ void gu_pass(const FfnArgs& p, const uint16_t* pg, const uint16_t* pu,
                                        int n0, int n, int m0, int i0, int col, int kg) {
  const int d = p.d, nst = d >> 6;
  const size_t gstride = (size_t)16 * d;
  const uint16_t* X = (const uint16_t*)p.x;
  const uint16_t* px[MC];
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    const int r = min(m0 + mc * 16 + col, n - 1);
    px[mc] = X + (size_t)(p.perm[n0 + r] / p.k) * d + kg * 16;
  }
  const int live = (n - m0 + 15) >> 4;  // 16-row chunks with tokens
  f32x4 ag[NG][MC], au[NG][MC];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      ag[q][mc] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[q][mc] = ag[q][mc];
    }
  GuStage<MC, NG> s0, s1;
  gu_load(s0, pg, pu, gstride, px, 0);
  for (int st = 0; st < nst; st += 2) {
    gu_load(s1, pg, pu, gstride, px, min(st + 1, nst - 1) * 64);
    gu_mma(s0, ag, au, live);
    gu_load(s0, pg, pu, gstride, px, min(st + 2, nst - 1) * 64);
    if (st + 1 < nst) gu_mma(s1, ag, au, live);
  }
  // lane holds C[4*kg + i][col] of each 16x16 tile: token rows, unit columns
  uint16_t* H = (uint16_t*)p.h;
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mc * 16 + kg * 4 + i;
        if (m < n)
          H[(size_t)(n0 + m) * p.f + i0 + q * 16 + col] = f32_to_bf16(silu(ag[q][mc][i]) * au[q][mc][i]);
      }
    }
}

// MC: 16-row chunks per pass at most; a pass with fewer rows left takes the 1- or 2-chunk
// form, so no token fragment is loaded for a chunk without tokens.  NG: 16-unit groups per
// wave (a workgroup covers 64 NG units).
template <int MC, int NG>
__global__ __launch_bounds__(256) void gemv_gateup(FfnArgs p) {
  const int nrb = p.f / (64 * NG);
  const int a = blockIdx.x / nrb, rb = blockIdx.x - a * nrb;
  const GemvItem it = gemv_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int i0 = rb * 64 * NG + wave * 16 * NG;
  const uint16_t* pg = it.w + (size_t)(i0 + col) * p.d + kg * 16;
  const uint16_t* pu = pg + (size_t)p.f * p.d;
  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
    const int chunks = (n - m0 + 15) >> 4;
    if (MC >= 4 && chunks > 2) gu_pass<(MC >= 4 ? 4 : 1), NG>(p, pg, pu, n0, n, m0, i0, col, kg);
    else if (MC >= 2 && chunks == 2) gu_pass<(MC >= 2 ? 2 : 1), NG>(p, pg, pu, n0, n, m0, i0, col, kg);
    else gu_pass<1, NG>(p, pg, pu, n0, n, m0, i0, col, kg);
  }
}

// Down: wave owns output channels o0..o0+16NG-1 of W_down; rows of h are contiguous.
template <int MC, int NG>
struct DnStage {
  u32x4 b0[NG], b1[NG];
  u32x4 a0[MC], a1[MC];
};

template <int MC, int NG>
__device__ __forceinline__ void dn_load(DnStage<MC, NG>& s, const uint16_t* pw, size_t gstride,
                                        const uint16_t* const (&ph)[MC], int kk) {
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    s.b0[q] = ldg16(pw + q * gstride + kk);
    s.b1[q] = ldg16(pw + q * gstride + kk + 8);
  }
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    s.a0[mc] = ldg16(ph[mc] + kk);
    s.a1[mc] = ldg16(ph[mc] + kk + 8);
  }
  issue_fence();
}

template <int MC, int NG>
__device__ __forceinline__ void dn_mma(const DnStage<MC, NG>& s, f32x4 (&acc)[NG][MC], int live) {
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    if (mc < live) {
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        acc[q][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a0[mc]), as_bf16x8(s.b0[q]), acc[q][mc], 0, 0, 0);
        acc[q][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a1[mc]), as_bf16x8(s.b1[q]), acc[q][mc], 0, 0, 0);
      }
    }
  }
}

template <int MC, int NG, int YDT>
__device__ __forceinline__ void dn_pass(const FfnArgs& p, const uint16_t* pw, int n0, int n,
                                        int m0, int o0, int col, int kg) {
  const int f = p.f, nst = f >> 6;
  const size_t gstride = (size_t)16 * f;
  const uint16_t* H = (const uint16_t*)p.h;
  const uint16_t* ph[MC];
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    const int r = min(m0 + mc * 16 + col, n - 1);
    ph[mc] = H + (size_t)(n0 + r) * f + kg * 16;
  }
  const int live = (n - m0 + 15) >> 4;
  f32x4 acc[NG][MC];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) acc[q][mc] = f32x4{0.f, 0.f, 0.f, 0.f};
  DnStage<MC, NG> s0, s1;
  dn_load(s0, pw, gstride, ph, 0);
  for (int st = 0; st < nst; st += 2) {
    dn_load(s1, pw, gstride, ph, min(st + 1, nst - 1) * 64);
    dn_mma(s0, acc, live);
    dn_load(s0, pw, gstride, ph, min(st + 2, nst - 1) * 64);
    if (st + 1 < nst) dn_mma(s1, acc, live);
  }
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mc * 16 + kg * 4 + i;
        if (m < n) {
          const size_t o = (size_t)(n0 + m) * p.d + o0 + q * 16 + col;
          if (YDT == MOE_F32) ((float*)p.y)[o] = acc[q][mc][i];
          else ((uint16_t*)p.y)[o] = f32_to_bf16(acc[q][mc][i]);
        }
      }
    }
}

template <int MC, int NG, int YDT>
__global__ __launch_bounds__(256) void gemv_down(FfnArgs p) {
  const int nrb = p.d / (64 * NG);
  const int a = blockIdx.x / nrb, rb = blockIdx.x - a * nrb;
  const GemvItem it = gemv_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int o0 = rb * 64 * NG + wave * 16 * NG;
  const uint16_t* pw = it.w + 2 * (size_t)p.f * p.d + (size_t)(o0 + col) * p.f + kg * 16;
  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
    const int chunks = (n - m0 + 15) >> 4;
    if (MC >= 4 && chunks > 2) dn_pass<(MC >= 4 ? 4 : 1), NG, YDT>(p, pw, n0, n, m0, o0, col, kg);
    else if (MC >= 2 && chunks == 2) dn_pass<(MC >= 2 ? 2 : 1), NG, YDT>(p, pw, n0, n, m0, o0, col, kg);
    else dn_pass<1, NG, YDT>(p, pw, n0, n, m0, o0, col, kg);
  }
}


template <int NG>
int launch_gemv_ng(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts,
                   int parts) {
  const dim3 gu(experts * (p.f / (64 * NG))), dn(experts * (p.d / (64 * NG))), blk(256);
  const bool yf = y_dtype == MOE_F32;
  if (parts & 1) {
    if (T <= 16) hipLaunchKernelGGL((gemv_gateup<1, NG>), gu, blk, 0, stream, p);
    else if (T <= 32) hipLaunchKernelGGL((gemv_gateup<2, NG>), gu, blk, 0, stream, p);
    else hipLaunchKernelGGL((gemv_gateup<4, NG>), gu, blk, 0, stream, p);
    MOE_LAUNCH_CHECK();
  }
  if (parts & 2) {
    if (T <= 16) {
      if (yf) hipLaunchKernelGGL((gemv_down<1, NG, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<1, NG, MOE_BF16>), dn, blk, 0, stream, p);
    } else if (T <= 32) {
      if (yf) hipLaunchKernelGGL((gemv_down<2, NG, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<2, NG, MOE_BF16>), dn, blk, 0, stream, p);
    } else {
      if (yf) hipLaunchKernelGGL((gemv_down<4, NG, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<4, NG, MOE_BF16>), dn, blk, 0, stream, p);
    }
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace

int launch_ffn_gemv(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts,
                    int parts) {
  if (experts <= 0) return MOE_OK;
  // Above 32 tokens (passes of up to 4 chunks) a wave takes two 16-row groups, which halves
  // the token fragments loaded per weight byte (T=64, Zipf 1: 450 -> 428 us); with fewer
  // tokens the halved grid costs more than that saves (T=16: 233 -> 248 us).  Needs the
  // workgroup's 128 rows to divide the matrix.
  const bool wide = T > 32;
  int rc = MOE_OK;
  if ((parts & 1) && wide && p.f % 128 == 0) rc = launch_gemv_ng<2>(p, T, y_dtype, stream, experts, 1);
  else if (parts & 1) rc = launch_gemv_ng<1>(p, T, y_dtype, stream, experts, 1);
  if (rc != MOE_OK) return rc;
  if ((parts & 2) && wide && p.d % 128 == 0) rc = launch_gemv_ng<2>(p, T, y_dtype, stream, experts, 2);
  else if (parts & 2) rc = launch_gemv_ng<1>(p, T, y_dtype, stream, experts, 2);
  return rc;
}

}  // namespace moe
