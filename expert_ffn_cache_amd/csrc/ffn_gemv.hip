// Decode-shaped expert FFN: weight streaming with v_mfma_f32_16x16x32_bf16.
//
// Each wavefront owns 16 weight rows and streams them straight from HBM into registers
// with 16-byte loads (4 lanes cover 64 contiguous bytes of a row, two loads per step make a
// full 128-byte line), multiplying against up to 16*MC token rows.  No LDS staging: every
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
// Two register sets alternate (no register rotation), so the next step's loads stay in
// flight while the current step's MFMAs run.  Token rows beyond the expert load a valid
// row and their (unused) output rows are not stored: an MFMA output row depends only
// on its own input row.
template <int MC>
struct GuStage {
  u32x4 g0, g1, u0, u1;
  u32x4 a0[MC], a1[MC];
};

template <int MC>
__device__ __forceinline__ void gu_load(GuStage<MC>& s, const uint16_t* pg, const uint16_t* pu,
                                        const uint16_t* const (&px)[MC], int kk) {
  s.g0 = ldg16(pg + kk);
  s.g1 = ldg16(pg + kk + 8);
  s.u0 = ldg16(pu + kk);
  s.u1 = ldg16(pu + kk + 8);
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    s.a0[mc] = ldg16(px[mc] + kk);
    s.a1[mc] = ldg16(px[mc] + kk + 8);
  }
  issue_fence();
}

template <int MC>
__device__ __forceinline__ void gu_mma(const GuStage<MC>& s, f32x4 (&ag)[MC], f32x4 (&au)[MC],
                                       int live) {
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    if (mc < live) {
      ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a0[mc]), as_bf16x8(s.g0), ag[mc], 0, 0, 0);
      au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a0[mc]), as_bf16x8(s.u0), au[mc], 0, 0, 0);
      ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a1[mc]), as_bf16x8(s.g1), ag[mc], 0, 0, 0);
      au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a1[mc]), as_bf16x8(s.u1), au[mc], 0, 0, 0);
    }
  }
}

// One pass over up to 16 MC token rows m0.. of the expert (MC chunks of 16 rows).
template <int MC>
__device__ __forceinline__ void gu_pass(const FfnArgs& p, const uint16_t* pg, const uint16_t* pu,
                                        int n0, int n, int m0, int i0, int col, int kg) {
  const int d = p.d, nst = d >> 6;
  const uint16_t* X = (const uint16_t*)p.x;
  const uint16_t* px[MC];
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    const int r = min(m0 + mc * 16 + col, n - 1);
    px[mc] = X + (size_t)(p.perm[n0 + r] / p.k) * d + kg * 16;
  }
  const int live = (n - m0 + 15) >> 4;  // 16-row chunks with tokens
  f32x4 ag[MC], au[MC];
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    ag[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    au[mc] = ag[mc];
  }
  GuStage<MC> s0, s1;
  gu_load(s0, pg, pu, px, 0);
  for (int st = 0; st < nst; st += 2) {
    gu_load(s1, pg, pu, px, min(st + 1, nst - 1) * 64);
    gu_mma(s0, ag, au, live);
    gu_load(s0, pg, pu, px, min(st + 2, nst - 1) * 64);
    if (st + 1 < nst) gu_mma(s1, ag, au, live);
  }
  // lane holds C[4*kg + i][col] of each 16x16 tile: token rows, unit columns
  uint16_t* H = (uint16_t*)p.h;
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

// MC: 16-row chunks per pass at most; a pass with fewer rows left takes the 1- or 2-chunk
// form, so no token fragment is loaded for a chunk without tokens.
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
  const uint16_t* pg = it.w + (size_t)(i0 + col) * p.d + kg * 16;
  const uint16_t* pu = pg + (size_t)p.f * p.d;
  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
    const int chunks = (n - m0 + 15) >> 4;
    if (MC >= 4 && chunks > 2) gu_pass<(MC >= 4 ? 4 : 1)>(p, pg, pu, n0, n, m0, i0, col, kg);
    else if (MC >= 2 && chunks == 2) gu_pass<(MC >= 2 ? 2 : 1)>(p, pg, pu, n0, n, m0, i0, col, kg);
    else gu_pass<1>(p, pg, pu, n0, n, m0, i0, col, kg);
  }
}

// Down: wave owns output channels o0..o0+15 of W_down; rows of h are contiguous.
template <int MC>
struct DnStage {
  u32x4 b0, b1;
  u32x4 a0[MC], a1[MC];
};

template <int MC>
__device__ __forceinline__ void dn_load(DnStage<MC>& s, const uint16_t* pw,
                                        const uint16_t* const (&ph)[MC], int kk) {
  s.b0 = ldg16(pw + kk);
  s.b1 = ldg16(pw + kk + 8);
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    s.a0[mc] = ldg16(ph[mc] + kk);
    s.a1[mc] = ldg16(ph[mc] + kk + 8);
  }
  issue_fence();
}

template <int MC>
__device__ __forceinline__ void dn_mma(const DnStage<MC>& s, f32x4 (&acc)[MC], int live) {
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    if (mc < live) {
      acc[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a0[mc]), as_bf16x8(s.b0), acc[mc], 0, 0, 0);
      acc[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s.a1[mc]), as_bf16x8(s.b1), acc[mc], 0, 0, 0);
    }
  }
}

template <int MC, int YDT>
__device__ __forceinline__ void dn_pass(const FfnArgs& p, const uint16_t* pw, int n0, int n,
                                        int m0, int o0, int col, int kg) {
  const int f = p.f, nst = f >> 6;
  const uint16_t* H = (const uint16_t*)p.h;
  const uint16_t* ph[MC];
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) {
    const int r = min(m0 + mc * 16 + col, n - 1);
    ph[mc] = H + (size_t)(n0 + r) * f + kg * 16;
  }
  const int live = (n - m0 + 15) >> 4;
  f32x4 acc[MC];
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) acc[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
  DnStage<MC> s0, s1;
  dn_load(s0, pw, ph, 0);
  for (int st = 0; st < nst; st += 2) {
    dn_load(s1, pw, ph, min(st + 1, nst - 1) * 64);
    dn_mma(s0, acc, live);
    dn_load(s0, pw, ph, min(st + 2, nst - 1) * 64);
    if (st + 1 < nst) dn_mma(s1, acc, live);
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
  const uint16_t* pw = it.w + 2 * (size_t)p.f * p.d + (size_t)(o0 + col) * p.f + kg * 16;
  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
    const int chunks = (n - m0 + 15) >> 4;
    if (MC >= 4 && chunks > 2) dn_pass<(MC >= 4 ? 4 : 1), YDT>(p, pw, n0, n, m0, o0, col, kg);
    else if (MC >= 2 && chunks == 2) dn_pass<(MC >= 2 ? 2 : 1), YDT>(p, pw, n0, n, m0, o0, col, kg);
    else dn_pass<1, YDT>(p, pw, n0, n, m0, o0, col, kg);
  }
}

}  // namespace

int launch_ffn_gemv(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts,
                    int parts) {
  if (experts <= 0) return MOE_OK;
  const dim3 gu(experts * (p.f / 64)), dn(experts * (p.d / 64)), blk(256);
  const bool yf = y_dtype == MOE_F32;
  if (parts & 1) {
    if (T <= 16) hipLaunchKernelGGL(gemv_gateup<1>, gu, blk, 0, stream, p);
    else if (T <= 32) hipLaunchKernelGGL(gemv_gateup<2>, gu, blk, 0, stream, p);
    else hipLaunchKernelGGL(gemv_gateup<4>, gu, blk, 0, stream, p);
    MOE_LAUNCH_CHECK();
  }
  if (parts & 2) {
    if (T <= 16) {
      if (yf) hipLaunchKernelGGL((gemv_down<1, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<1, MOE_BF16>), dn, blk, 0, stream, p);
    } else if (T <= 32) {
      if (yf) hipLaunchKernelGGL((gemv_down<2, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<2, MOE_BF16>), dn, blk, 0, stream, p);
    } else {
      if (yf) hipLaunchKernelGGL((gemv_down<4, MOE_F32>), dn, blk, 0, stream, p);
      else hipLaunchKernelGGL((gemv_down<4, MOE_BF16>), dn, blk, 0, stream, p);
    }
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
