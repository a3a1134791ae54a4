// Prefill-shaped expert FFN: LDS-tiled grouped GEMM on v_mfma_f32_32x32x16_bf16.
#include <algorithm>
#include <type_traits>

#include "ffn_args.h"

namespace moe {
namespace {

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
// Inside a step, the fragments of the next 16-wide k substep are read from LDS while the
// current substep's MFMAs run.
constexpr int QBM = 256, QBN = 256, QBK = 64;
constexpr int kGateUp = 0, kDown = 1;

// Element index of 16-byte chunk c (0..7) of row r in a 128-byte-row tile; the XOR spreads
// the 16 rows served by one ds_read_b128 cycle over all LDS banks.
__device__ __forceinline__ int qswz(int r, int c) { return r * QBK + ((c ^ ((r >> 1) & 7)) << 3); }

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane, global -> LDS (lane i lands at lds + 16 i; lds is wave-uniform).  Issued
// from inline assembly so the compiler does not drain every outstanding load before each
// LDS read (it cannot tell which stage a direct load writes); stage readiness is tracked
// with explicit s_waitcnt vmcnt below.  Writes M0, declared clobbered (clang warns that M0
// is a reserved register; listing it is what tells the compiler that any value it kept there
// is gone); has no output registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void g2lds16(const uint16_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 7, 15));
  asm volatile("" ::: "memory");
}

// SiLU(g) * u with the hardware reciprocal (about 1 ulp in fp32): h is rounded to bf16 right
// after, so an exact division would change nothing but the cost.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets in SGPRs
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
  // loader geometry: load instruction q (0..31) fills tile rows q*8 + lane/8, LDS chunk
  // lane&7, i.e. logical chunk lc of the source row; wave w issues q = 4w..4w+3 for the
  // token tile and for the weight tile

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
    // items of one expert in groups of up to 4 m-tiles x all n-tiles, m-tile fastest: the 32
    // consecutive items one XCD runs together form a 4 x 8 block of tiles, so each token slice
    // and each weight slice of a step is fetched into that XCD's L2 once and read from it by
    // 8 (resp. 4) workgroups (10% fewer L2 miss bytes than n-tile-major order)
    const int grp = local / (4 * n_ntiles), first_m = grp * 4;
    const int gsz = min(4, m_e - first_m), in = local - grp * 4 * n_ntiles;
    const int nt = in / gsz, mt = first_m + (in - nt * gsz);
    const char* wbase = entry_of(p, e);
    if (!wbase) continue;
    const uint16_t* W = (const uint16_t*)wbase;
    const int n0 = p.offsets[e] + mt * QBM;
    const int rows = min(QBM, p.offsets[e + 1] - n0);
    const int mtiles = (rows + 31) >> 5;

    // per-lane source rows of this item (element offsets, + logical chunk)
    const uint16_t* abase = MODE == kGateUp ? (const uint16_t*)p.x : (const uint16_t*)p.h;
    uint32_t oa[4], ob[4];
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per item rather than held across the k-loop
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int R = (4 * wave + t) * 8 + (ln >> 3);  // tile row 0..255
      const int lc = (ln & 7) ^ ((R >> 1) & 7);
      const int r = min(R, rows - 1);
      oa[t] = (MODE == kGateUp ? (uint32_t)(p.perm[n0 + r] / p.k) * (uint32_t)p.d
                               : (uint32_t)(n0 + r) * (uint32_t)p.f) + lc * 8;
      if (MODE == kGateUp) {  // weight rows 64w'..64w'+31: gate units, +32..63: same up units
        const int wq = R >> 6, rr = R & 63;
        const int unit = nt * (QBN / 2) + wq * 32 + (rr & 31);
        ob[t] = (uint32_t)((rr >> 5) * p.f + (unit < p.f ? unit : 0)) * (uint32_t)p.d + lc * 8;
      } else {
        const int o = nt * QBN + R;
        ob[t] = 2u * (uint32_t)p.f * (uint32_t)p.d + (uint32_t)(o < p.d ? o : 0) * (uint32_t)p.f + lc * 8;
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
      for (int t = 0; t < 4; ++t) g2lds16(abase + oa[t] + kk, lds_addr(st) + (4 * wave + t) * 8 * QBK * 2);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        g2lds16(W + ob[t] + kk, lds_addr(st) + QBM * QBK * 2 + (4 * wave + t) * 8 * QBK * 2);
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
    // step ks on stage S = ks % 2: wait for this wave's part of the stage, publish it
    // (which also frees the other stage, read by step ks-1), refill that stage with step
    // ks+1, then 4 substeps of up to 8 MFMAs
    auto step = [&](auto tag, auto am_tag, int ks) {
      constexpr int S = decltype(tag)::value;
      constexpr int AM = decltype(am_tag)::value;
      wait_vmcnt<0>();  // this wave's part of stage ks has landed
      lds_barrier();     // ... and every wave's; stage ks^1 is free again
      if (ks + 1 < nk) issue(std::integral_constant<int, (S + 1) & 1>{}, ks + 1);
      const uint16_t* st = stage_ptr(tag);
      // fragments of substep s+1 are read while substep s's MFMAs run (two register sets)
      bf16x8 bq[2][2], aq[2][4];
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        bq[0][jn] = as_bf16x8(*(const u32x4*)&st[QBM * QBK + qswz(wn * 64 + jn * 32 + r32, g)]);
#pragma unroll
      for (int i = 0; i < AM; ++i) aq[0][i] = as_bf16x8(*(const u32x4*)&st[qswz(wm * 128 + i * 32 + r32, g)]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int cur = s & 1, nxt = cur ^ 1;
        if (s + 1 < 4) {
          const int ch = (s + 1) * 2 + g;
#pragma unroll
          for (int jn = 0; jn < 2; ++jn)
            bq[nxt][jn] = as_bf16x8(*(const u32x4*)&st[QBM * QBK + qswz(wn * 64 + jn * 32 + r32, ch)]);
#pragma unroll
          for (int i = 0; i < AM; ++i)
            aq[nxt][i] = as_bf16x8(*(const u32x4*)&st[qswz(wm * 128 + i * 32 + r32, ch)]);
        }
#pragma unroll
        for (int i = 0; i < AM; ++i) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[cur][i], bq[cur][0], acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[cur][i], bq[cur][1], acc[i][1], 0, 0, 0);
        }
      }
      // Pin that order for the scheduler (left alone it serialises each LDS read with the
      // MFMA that consumes it): substep 0's reads, then each substep's MFMAs interleaved
      // one-for-one with the next substep's reads (masks: 0x100 LDS read, 0x008 MFMA).
      if constexpr (AM > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2 + AM, 0);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
          for (int q = 0; q < 2 * AM || q < 2 + AM; ++q) {
            if (q < 2 * AM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < 2 + AM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * AM, 0);
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
            ((uint16_t*)p.h)[(size_t)(n0 + m) * ld + unit] = f32_to_bf16(swiglu(acc[i][0][v], acc[i][1][v]));
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

}  // namespace

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// The loaders keep element offsets in 32 bits (token rows of x and h, rows of an entry).
bool ffn_gemm_supported(long long T, int k, int d, int f) {
  constexpr long long lim = 1ll << 32;
  return T * d <= lim && T * k * f <= lim && 3ll * d * f <= lim;
}

int launch_ffn_gemm(const FfnArgs& p, int y_dtype, hipStream_t stream) {
  const dim3 grid((num_cus() + 7) / 8 * 8), blk(512);
  hipLaunchKernelGGL((gemm_tile256<kGateUp, MOE_BF16>), grid, blk, 0, stream, p,
                     (p.f + QBN / 2 - 1) / (QBN / 2));
  MOE_LAUNCH_CHECK();
  const int ntd = (p.d + QBN - 1) / QBN;
  if (y_dtype == MOE_F32)
    hipLaunchKernelGGL((gemm_tile256<kDown, MOE_F32>), grid, blk, 0, stream, p, ntd);
  else
    hipLaunchKernelGGL((gemm_tile256<kDown, MOE_BF16>), grid, blk, 0, stream, p, ntd);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
