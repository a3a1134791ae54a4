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
#include <type_traits>

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
  const int d = p.d, nst = d >> 6;
  const uint16_t* pg = it.w + (size_t)(i0 + col) * d + kg * 16;
  const uint16_t* pu = pg + (size_t)p.f * d;
  const uint16_t* X = (const uint16_t*)p.x;
  uint16_t* H = (uint16_t*)p.h;

  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
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
__global__ __launch_bounds__(256) void gemv_down(FfnArgs p) {
  const int nrb = p.d >> 6;
  const int a = blockIdx.x / nrb, rb = blockIdx.x - a * nrb;
  const GemvItem it = gemv_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int o0 = rb * 64 + wave * 16;
  const int f = p.f, nst = f >> 6;
  const uint16_t* pw = it.w + 2 * (size_t)f * p.d + (size_t)(o0 + col) * f + kg * 16;
  const uint16_t* H = (const uint16_t*)p.h;

  for (int m0 = 0; m0 < n; m0 += 16 * MC) {
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
}

// ------------------------------------------------------------------ GEMM path
// Tile: 256 grouped token rows x 256 weight rows per workgroup of 8 waves (two per SIMD,
// so one wave's LDS-read latency is covered by the other's MFMAs), k in steps of 64.
// Both operands go global -> LDS with direct loads (global_load_lds_dwordx4: lane i lands
// at LDS base + 16 i), one full 128-byte line per row per step, into a 2-stage ring of
// 64 KB stages [256 token rows x 128 B | 256 weight rows x 128 B]: the next step's loads
// are in flight while this step's MFMAs run, and no VGPR holds staging data.  A wave's own
// counter (s_waitcnt vmcnt) says when its part of a stage has landed; one LDS-only barrier
// per step publishes the stage and frees the other one.
// Wave (wm, wn) computes token rows wm*128 + [0,128) (up to four 32-row m-tiles) against
// weight rows wn*64 + [0,64) (two 32-row n-tiles; for gate/up, 32 gate units and the same
// 32 up units, so SiLU(g)*u is formed in registers) with v_mfma_f32_32x32x16_bf16.  Only
// m-tiles that hold expert rows are computed (the count is a compile-time parameter of the
// k-loop, chosen per item, so the loop body stays branch-free).  Token rows are gathered
// through perm (gate/up) or read contiguously (down); rows past the expert repeat a valid
// row and their outputs are not stored.  Workgroups are persistent; the (expert, n-tile,
// m-tile) list is derived on the device from offsets and dealt XCD-major so consecutive
// items (sharing weight rows or token rows) run at the same time on one XCD's L2.
constexpr int QBM = 256, QBN = 256, QBK = 64;
constexpr int kGateUp = 0, kDown = 1;

// Element index of 16-byte chunk c (0..3) of row r in a 64-byte-row tile; the XOR spreads
// the 16 rows served by one ds_read_b128 cycle over all LDS banks.
__device__ __forceinline__ int qswz(int r, int c) { return r * QBK + ((c ^ ((r >> 1) & 7)) << 3); }

// 16 bytes per lane, global -> LDS (lane i lands at lds_wave_base + 16 i).  Issued from
// inline assembly so the compiler does not drain every outstanding load before each LDS
// read (it cannot tell which stage a direct load writes); stage readiness is tracked
// with explicit s_waitcnt vmcnt below.  Sets M0 itself (nothing else in these kernels
// uses M0); has no output registers.
__device__ __forceinline__ void g2lds16(const uint16_t* g, const uint16_t* lds_wave_base) {
  const uint32_t l = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(l)), "v"(g) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 7, 15));
  asm volatile("" ::: "memory");
}

template <int MODE, int YDT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tile256(FfnArgs p, int n_ntiles) {
  // one array per ring stage: [token rows | weight rows], 32 KB each
  __shared__ __attribute__((aligned(1024))) uint16_t sm0[2 * QBM * QBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sm1[2 * QBM * QBK];

  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_wave[8];
  __shared__ int s_total;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {  // 256-row m-tiles per expert and their prefix (2 experts per thread, E <= 1024)
    int c[2], tot = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      c[q] = 0;
      if (e < p.E && active(p, e)) c[q] = (p.offsets[e + 1] - p.offsets[e] + QBM - 1) / QBM;
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
      for (int w = 0; w < 8; ++w) { const int v = s_wave[w]; s_wave[w] = run; run += v; }
      s_total = run;
    }
    __syncthreads();
    int run = s_wave[wave] + x - tot;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      if (e < p.E) s_pref[e] = run;
      run += c[q];
    }
    if (tid == 0) s_pref[p.E] = s_total;
    __syncthreads();
  }
  const int total_items = s_total * n_ntiles;
  const int K = MODE == kGateUp ? p.d : p.f;
  const int nk = K / QBK;
  const int G = gridDim.x, per_xcd = G >> 3;
  const int pos = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);  // XCD-major dealing
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;
  // loader geometry: load instruction q (0..15) fills tile rows q*16 + lane/4, chunk lane&3
  // of LDS, i.e. logical chunk lc of the source row; wave w issues q = 2w, 2w+1 for the
  // token tile and for the weight tile
  const int lrow = lane >> 3;  // 8 rows x 128 B per load instruction

  for (int j = pos; j < total_items; j += G) {
    const int q = j / n_ntiles;
    int lo = 0, hi = p.E;  // largest e with s_pref[e] <= q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int m_e = s_pref[e + 1] - s_pref[e];
    const int local = j - s_pref[e] * n_ntiles;
    const int nt = local / m_e, mt = local - nt * m_e;
    const char* wbase = entry_of(p, e);
    if (!wbase) continue;
    const uint16_t* W = (const uint16_t*)wbase;
    const int n0 = p.offsets[e] + mt * QBM;
    const int rows = min(QBM, p.offsets[e + 1] - n0);
    const int mtiles = (rows + 31) >> 5;

    // per-lane source rows of this item (element offsets, + logical chunk)
    const uint16_t* abase = MODE == kGateUp ? (const uint16_t*)p.x : (const uint16_t*)p.h;
    uint32_t oa[4], ob[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int R = (4 * wave + t) * 8 + lrow;  // tile row 0..255
      const int lc = (lane & 7) ^ ((R >> 1) & 7);
      const int r = min(R, rows - 1);
      oa[t] = (MODE == kGateUp ? (uint32_t)(p.perm[n0 + r] / p.k) * (uint32_t)p.d
                               : (uint32_t)(n0 + r) * (uint32_t)p.f) + lc * 8;
      if (MODE == kGateUp) {  // weight rows 64w'..64w'+31: gate units, +32..63: same up units
        const int wq = R >> 6, rr = R & 63;
        const int unit = nt * (QBN / 2) + wq * 32 + (rr & 31);
        ob[t] = (uint32_t)((rr >> 5) * p.f + (unit < p.f ? unit : 0)) * (uint32_t)p.d + lc * 8;
      } else {
        const int o = nt * QBN + R;
        ob[t] = (uint32_t)(2 * p.f * p.d) + (uint32_t)(o < p.d ? o : 0) * (uint32_t)p.f + lc * 8;
      }
    }
    auto stage_ptr = [&](auto tag) -> uint16_t* {
      constexpr int S = decltype(tag)::value;
      return S == 0 ? sm0 : sm1;
    };
    auto issue = [&](auto tag, int ks) {
      uint16_t* st = stage_ptr(tag);
      const int kk = ks * QBK;
#pragma unroll
      for (int t = 0; t < 4; ++t) g2lds16(abase + oa[t] + kk, st + ((4 * wave + t) * 8) * QBK);
#pragma unroll
      for (int t = 0; t < 4; ++t) g2lds16(W + ob[t] + kk, st + QBM * QBK + ((4 * wave + t) * 8) * QBK);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    __syncthreads();  // the previous item's readers of the ring are done
    issue(I0{}, 0);
    // step ks on stage S = ks % 4: wait for this wave's part of the stage, publish it,
    // refill the stage freed by step ks-1 with step ks+3, then 2 x 8 MFMAs
    auto step = [&](auto tag, auto am_tag, int ks) {
      constexpr int S = decltype(tag)::value;
      constexpr int AM = decltype(am_tag)::value;
      wait_vmcnt<0>();  // this wave's part of stage ks has landed
      lds_barrier();     // ... and every wave's; stage ks^1 is free again
      if (ks + 1 < nk) issue(std::integral_constant<int, (S + 1) & 1>{}, ks + 1);
      const uint16_t* st = stage_ptr(tag);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = s * 2 + g;
        bf16x8 bfr[2], af[4];
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          bfr[jn] = as_bf16x8(*(const u32x4*)&st[QBM * QBK + qswz(wn * 64 + jn * 32 + r32, ch)]);
#pragma unroll
        for (int i = 0; i < AM; ++i)
          af[i] = as_bf16x8(*(const u32x4*)&st[qswz(wm * 128 + i * 32 + r32, ch)]);
#pragma unroll
        for (int i = 0; i < AM; ++i) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[0], acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[1], acc[i][1], 0, 0, 0);
        }
      }
    };
    // only this wave's m-tiles that hold expert rows are computed (compile-time count,
    // so the inner loop stays branch-free)
    auto run_k = [&](auto am_tag) {
      for (int ks = 0; ks < nk; ks += 2) {
        step(I0{}, am_tag, ks);
        if (ks + 1 < nk) step(I1{}, am_tag, ks + 1);
      }
    };
    const int am = min(4, max(0, mtiles - wm * 4));
    switch (am) {
      case 0: run_k(std::integral_constant<int, 0>{}); break;
      case 1: run_k(std::integral_constant<int, 1>{}); break;
      case 2: run_k(std::integral_constant<int, 2>{}); break;
      case 3: run_k(std::integral_constant<int, 3>{}); break;
      default: run_k(std::integral_constant<int, 4>{}); break;
    }

    // epilogue: lane holds C[8*(v/4) + 4*g + v%4][r32] of each 32x32 tile
    int ld = MODE == kGateUp ? p.f : p.d;
    asm volatile("" : "+s"(ld));  // keep row-offset products inside the item loop
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (wm * 4 + i >= mtiles) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m >= rows) continue;
        if (MODE == kGateUp) {
          const int unit = nt * (QBN / 2) + wn * 32 + r32;
          if (unit < p.f)
            ((uint16_t*)p.h)[(size_t)(n0 + m) * ld + unit] = f32_to_bf16(silu(acc[i][0][v]) * acc[i][1][v]);
        } else {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const int o = nt * QBN + wn * 64 + jn * 32 + r32;
            if (o < p.d) {
              const size_t idx = (size_t)(n0 + m) * ld + o;
              if (YDT == MOE_F32) ((float*)p.y)[idx] = acc[i][jn][v];
              else ((uint16_t*)p.y)[idx] = f32_to_bf16(acc[i][jn][v]);
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
  const dim3 grid((num_cus() + 7) / 8 * 8), blk(512);
  hipLaunchKernelGGL((gemm_tile256<kGateUp, MOE_BF16>), grid, blk, 0, stream, p, (f + QBN / 2 - 1) / (QBN / 2));
  MOE_LAUNCH_CHECK();
  const int ntd = (d + QBN - 1) / QBN;
  if (y_dtype == MOE_F32)
    hipLaunchKernelGGL((gemm_tile256<kDown, MOE_F32>), grid, blk, 0, stream, p, ntd);
  else
    hipLaunchKernelGGL((gemm_tile256<kDown, MOE_BF16>), grid, blk, 0, stream, p, ntd);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
