// Prefill-shaped expert FFN with MXFP4 expert weights: a grouped GEMM over the experts' token
// rows.  The activations stay bf16, so the products run on v_mfma_f32_16x16x32_bf16 with
// the FP4 codes expanded to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4, exact for E8M0
// scales): the same arithmetic as the decode kernels, with the weights of an expert reused
// across 64 token rows per workgroup instead of streamed once per token group.
//
// Tile: a workgroup computes 64 token rows of one expert x 128 weight rows (4 waves, each 2
// strips of 16 rows), stepping over K one 128-element tile column at a time.  The entry's
// tiled layout (16 rows x 128 elements per tile, slot l = 16 q + i = row i, block q) means
// a wave's 16-byte loads of one tile column are contiguous and each lane then holds its
// MFMA B operands for four k-groups (as in the decode kernels).  The token rows of the
// current tile column sit in LDS (double-buffered, rows padded by 16 bytes so a 16-row
// operand read hits 16 distinct bank groups); the next column's rows and weight codes are
// loaded into registers while the current one is multiplied.  Rows past an expert's count
// read row 0 of the block and their outputs are dropped; elements past K stage as zero.
//
// Work list: workgroup -> (expert, 64-row block) in expert order, found on the device from
// the offsets (one wave scans the experts' block counts), x 128-row weight block; blocks
// are dealt XCD-major so the workgroups sharing an expert's token rows share an L2.
#include <algorithm>
#include <type_traits>

#include "ffn_args.h"
#include "mx_dev.h"

namespace moe {
namespace {

constexpr int kMgM = 64;             // token rows per workgroup
constexpr int kMgS = 2;              // 16-row strips per wave
constexpr int kMgN = 4 * 16 * kMgS;  // weight rows per workgroup
constexpr int kMgLd = 128 + 8;       // LDS row stride (bf16) of a staged tile column

__device__ __forceinline__ float mg_e8m0(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);  // 2^(s - 127)
}

__device__ __forceinline__ bf16x8 mg_expand8(uint32_t w, float sc) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                 __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

struct MgItem {
  int e;       // expert, or -1 past the end of the work list
  int m0;      // first row of the block within the expert's rows
  int n0, n;   // the expert's grouped rows [n0, n0 + n)
  const uint8_t* w;
};

// The mb-th (expert, 64-row block) pair over the active experts in ascending id.
__device__ __forceinline__ MgItem mg_item(const FfnArgs& p, int mb) {
  __shared__ int s_e, s_m0;
  __shared__ const char* s_w;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int seen = 0, ef = -1, m0 = 0;
    for (int e0 = 0; e0 < p.E; e0 += 64) {
      const int e = e0 + lane;
      const int nb = e < p.E && active(p, e) ? (p.offsets[e + 1] - p.offsets[e] + kMgM - 1) / kMgM : 0;
      int incl = nb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int total = __shfl(incl, 63);
      if (mb < seen + total) {
        const bool mine = mb >= seen + incl - nb && mb < seen + incl;
        const int src = __ffsll((long long)__ballot(mine)) - 1;
        ef = e0 + src;
        m0 = (mb - seen - __shfl(incl - nb, src)) * kMgM;
        break;
      }
      seen += total;
    }
    if (lane == 0) {
      s_e = ef;
      s_m0 = m0;
      s_w = ef >= 0 ? entry_of(p, ef) : nullptr;
    }
  }
  __syncthreads();
  MgItem it{s_e, s_m0, 0, 0, (const uint8_t*)s_w};
  if (it.e >= 0) {
    it.n0 = p.offsets[it.e];
    it.n = p.offsets[it.e + 1] - it.n0;
  }
  return it;
}

// This thread's share of one staged tile column: 64 rows x 16 chunks of 8 elements, four
// chunks per thread; src_row(t) gives the source row of block row t (rows past the expert
// repeat block row 0).
struct MgStage {
  u32x4 v[4];
};

template <typename RowOf>
__device__ __forceinline__ void mg_load_a(MgStage& st, const uint16_t* src, int K, int kt,
                                          int rows, RowOf src_row) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i, t = c >> 4, ch = c & 15;
    const int k = kt * 128 + ch * 8;
    st.v[i] = k < K ? ldg16(src + (size_t)src_row(t < rows ? t : 0) * K + k) : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void mg_store_a(const MgStage& st, uint16_t* lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + 256 * i, t = c >> 4, ch = c & 15;
    *(u32x4*)&lds[t * kMgLd + ch * 8] = st.v[i];
  }
}

template <int NMAT>
struct MgB {
  u32x4 c[kMgS][NMAT];
  uint32_t s[kMgS][NMAT];
};

// Tile column kt of the wave's strips (cb/sb: strip 0's codes/scales of each matrix, the
// next strip 8 K / K/2 bytes further); nstr strips exist (the last workgroup of a matrix
// may own fewer); lanes whose block is past K load zeros.
template <int NMAT>
__device__ __forceinline__ void mg_load_b(MgB<NMAT>& b, const uint8_t* const (&cb)[NMAT],
                                          const uint8_t* const (&sb)[NMAT], int K, int kt,
                                          int nstr, int lane) {
  const bool ok = kt * 128 + 32 * (lane >> 4) < K;
#pragma unroll
  for (int s = 0; s < kMgS; ++s)
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      if (ok && s < nstr) {
        b.c[s][m] = ldg16(cb[m] + (size_t)s * 8 * K + (size_t)kt * 1024 + lane * 16);
        b.s[s][m] = ldg_u8(sb[m] + (size_t)s * (K / 2) + (size_t)kt * 64 + lane);
      } else {
        b.c[s][m] = u32x4{0u, 0u, 0u, 0u};
        b.s[s][m] = 0u;
      }
    }
  issue_fence();
}

// acc[s][m][mt] += A(mt) x B(s, m)^T over one tile column.
template <int NMAT>
__device__ __forceinline__ void mg_mma(const MgB<NMAT>& b, const uint16_t* lds, int lane,
                                       f32x4 (&acc)[kMgS][NMAT][4]) {
  bf16x8 w[kMgS][NMAT][4];
#pragma unroll
  for (int s = 0; s < kMgS; ++s)
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const float sc = mg_e8m0(b.s[s][m]);
#pragma unroll
      for (int j = 0; j < 4; ++j) w[s][m][j] = mg_expand8(b.c[s][m][j], sc);
    }
  const uint16_t* ar = lds + (lane & 15) * kMgLd + 32 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    bf16x8 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = as_bf16x8(*(const u32x4*)(ar + mt * 16 * kMgLd + 8 * j));
#pragma unroll
    for (int s = 0; s < kMgS; ++s)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[s][m][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], w[s][m][j], acc[s][m][mt], 0, 0, 0);
  }
}

// Workgroup id -> logical block, XCD-major: workgroups are dealt round-robin over the 8 XCDs,
// so consecutive logical blocks (the weight blocks of one token block) land on one XCD.
__device__ __forceinline__ int mg_logical_block() {
  const int g = gridDim.x;  // a multiple of 8
  return (blockIdx.x & 7) * (g >> 3) + (blockIdx.x >> 3);
}

// The K loop shared by both kernels: stages token rows, streams the weight tiles.
template <int NMAT, typename RowOf>
__device__ __forceinline__ void mg_run(const uint16_t* src, int K, int rows, RowOf src_row,
                                       const uint8_t* const (&cb)[NMAT],
                                       const uint8_t* const (&sb)[NMAT], int nstr, int lane,
                                       uint16_t* lds, f32x4 (&acc)[kMgS][NMAT][4]) {
  const int nk = (K + 127) >> 7;
  MgStage st;
  MgB<NMAT> b;
  mg_load_b<NMAT>(b, cb, sb, K, 0, nstr, lane);
  mg_load_a(st, src, K, 0, rows, src_row);
  mg_store_a(st, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const MgB<NMAT> cur = b;
    uint16_t* cur_lds = lds + (kt & 1) * kMgM * kMgLd;
    if (kt + 1 < nk) {
      mg_load_b<NMAT>(b, cb, sb, K, kt + 1, nstr, lane);
      mg_load_a(st, src, K, kt + 1, rows, src_row);
    }
    mg_mma<NMAT>(cur, cur_lds, lane, acc);
    if (kt + 1 < nk) mg_store_a(st, lds + ((kt + 1) & 1) * kMgM * kMgLd);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void mg_gateup(FfnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kMgM * kMgLd];
  const int nnb = (p.f + kMgN - 1) / kMgN;
  const int L = mg_logical_block();
  const MgItem it = mg_item(p, L / nnb);
  if (it.e < 0 || !it.w) return;
  const int nb = L - (L / nnb) * nnb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt0 = nb * (kMgN / 16) + wave * kMgS;  // first strip of this wave
  const int nstr = min(kMgS, p.f / 16 - rt0);
  const int rows = min(kMgM, it.n - it.m0);
  const int K = p.d;
  const size_t fd = (size_t)p.f * K;
  const uint8_t* W = it.w;
  const size_t so = (size_t)rt0 * 8 * K, ss = (size_t)rt0 * (K / 2);
  const uint8_t* const cb[2] = {W + so, W + fd / 2 + so};
  const uint8_t* const sb[2] = {W + 3 * fd / 2 + ss, W + 3 * fd / 2 + fd / 32 + ss};
  f32x4 acc[kMgS][2][4];
#pragma unroll
  for (int s = 0; s < kMgS; ++s)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[s][m][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int base = it.n0 + it.m0;
  mg_run<2>((const uint16_t*)p.x, K, rows, [&](int t) { return p.perm[base + t] / p.k; }, cb, sb,
            nstr, lane, lds, acc);
  uint16_t* H = (uint16_t*)p.h;
  const int col = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int s = 0; s < kMgS; ++s) {
    if (s >= nstr) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + kg * 4 + i;  // lane holds C[4 kg + i][col] of the 16x16 tile
        if (t < rows)
          H[(size_t)(base + t) * p.f + 16 * (rt0 + s) + col] = f32_to_bf16(silu(acc[s][0][mt][i]) * acc[s][1][mt][i]);
      }
  }
}

template <int YDT>
__global__ __launch_bounds__(256) void mg_down(FfnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kMgM * kMgLd];
  const int nnb = (p.d + kMgN - 1) / kMgN;
  const int L = mg_logical_block();
  const MgItem it = mg_item(p, L / nnb);
  if (it.e < 0 || !it.w) return;
  const int nb = L - (L / nnb) * nnb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt0 = nb * (kMgN / 16) + wave * kMgS;
  const int nstr = min(kMgS, p.d / 16 - rt0);
  const int rows = min(kMgM, it.n - it.m0);
  const int K = p.f;
  const size_t fd = (size_t)K * p.d;
  const uint8_t* W = it.w;
  const size_t so = (size_t)rt0 * 8 * K, ss = (size_t)rt0 * (K / 2);
  const uint8_t* const cb[1] = {W + fd + so};
  const uint8_t* const sb[1] = {W + 3 * fd / 2 + 2 * (fd / 32) + ss};
  f32x4 acc[kMgS][1][4];
#pragma unroll
  for (int s = 0; s < kMgS; ++s)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[s][0][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int base = it.n0 + it.m0;
  mg_run<1>((const uint16_t*)p.h, K, rows, [&](int t) { return base + t; }, cb, sb, nstr, lane,
            lds, acc);
  const int col = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int s = 0; s < kMgS; ++s) {
    if (s >= nstr) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + kg * 4 + i;
        if (t < rows) {
          const size_t o = (size_t)(base + t) * p.d + 16 * (rt0 + s) + col;
          if (YDT == MOE_F32) ((float*)p.y)[o] = acc[s][0][mt][i];
          else ((uint16_t*)p.y)[o] = f32_to_bf16(acc[s][0][mt][i]);
        }
      }
  }
}

// ------------------------------------------------------------ 256 x 256 tiles
// The grouped GEMM of the bf16 weights (256 token rows x 256 weight rows per 8-wave
// workgroup, k steps of 64, a 2-stage direct-to-LDS ring, 32x32x16 MFMAs, persistent
// workgroups over a device-derived (expert, n-tile, m-tile) list), with the weight side of a
// stage holding FP4 codes and scales instead of bf16 rows: per stage 16 strips x 512 bytes of
// codes (half a tile column each) and 16 x 32 scale bytes.  Each wave expands its B operand
// (4 code bytes and a scale per lane per MFMA) to bf16 with v_cvt_scalef32_pk_bf16_fp4
// right before the MFMAs; the products and their order are those of the bf16 kernel.
constexpr int XBM = 256, XBK = 64;
constexpr int XA_BYTES = XBM * XBK * 2;           // token rows: 256 x 128 B, swizzled
constexpr int XC_BYTES = 16 * 512;                // codes: strip s at s * 512, slot 16 q + i
constexpr int XS_BYTES = 16 * 32;                 // scales: strip s at s * 32
constexpr int XSTAGE = XA_BYTES + XC_BYTES + XS_BYTES;

__device__ __forceinline__ int xswz(int r, int c) { return r * XBK + ((c ^ ((r >> 1) & 7)) << 3); }

__device__ __forceinline__ uint32_t x_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void x_g2lds16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void x_g2lds4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" :: "s"(lds), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void x_wait_vm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 7, 15));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float x_swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <int MODE, int YDT>  // MODE 0: gate/up (h out), 1: down (y out)
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mx_tile256(FfnArgs p, int n_ntiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[2][XSTAGE];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_wave[8];
  __shared__ int s_total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  {  // 256-row m-tiles per expert and their prefix (2 experts per thread, E <= 1024)
    int c[2], tot = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      c[q] = 0;
      if (e < p.E && active(p, e)) c[q] = (p.offsets[e + 1] - p.offsets[e] + XBM - 1) / XBM;
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
  const int K = MODE == 0 ? p.d : p.f;
  const int nk = K / XBK;
  const size_t fd = (size_t)p.f * p.d;
  const int G = gridDim.x, per_xcd = G >> 3;
  const int pos = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;

  for (int j = pos; j < total_items; j += G) {
    const int q = j / n_ntiles;
    int lo = 0, hi = p.E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int m_e = s_pref[e + 1] - s_pref[e];
    const int local = j - s_pref[e] * n_ntiles;
    const int grp = local / (4 * n_ntiles), first_m = grp * 4;
    const int gsz = min(4, m_e - first_m), in = local - grp * 4 * n_ntiles;
    const int nt = in / gsz, mt = first_m + (in - nt * gsz);
    const char* wbase = entry_of(p, e);
    if (!wbase) continue;
    const uint8_t* W = (const uint8_t*)wbase;
    const int n0 = p.offsets[e] + mt * XBM;
    const int rows = min(XBM, p.offsets[e + 1] - n0);
    const int mtiles = (rows + 31) >> 5;

    const uint16_t* abase = MODE == 0 ? (const uint16_t*)p.x : (const uint16_t*)p.h;
    uint32_t oa[4];
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // token rows (4w + t) * 8 + lane / 8, chunk lane & 7
      const int R = (4 * wave + t) * 8 + (ln >> 3);
      const int lc = (ln & 7) ^ ((R >> 1) & 7);
      const int r = min(R, rows - 1);
      oa[t] = (MODE == 0 ? (uint32_t)(p.perm[n0 + r] / p.k) * (uint32_t)p.d
                         : (uint32_t)(n0 + r) * (uint32_t)p.f) + lc * 8;
    }
    // codes: wave w loads strips 2w, 2w + 1 (512 B each); scales: waves 0, 1 load 8 strips each
    const uint8_t* cptr;
    const uint8_t* sptr = nullptr;
    {
      auto strip_base = [&](int sidx, size_t& coff, size_t& soff) {
        int rt;
        size_t cm, sm_;
        if (MODE == 0) {
          const int m = (sidx >> 1) & 1;
          int u0 = nt * 128 + (sidx >> 2) * 32 + (sidx & 1) * 16;
          if (u0 >= p.f) u0 = 0;
          rt = u0 >> 4;
          cm = (size_t)m * (fd / 2);
          sm_ = 3 * fd / 2 + (size_t)m * (fd / 32);
        } else {
          int o0 = nt * 256 + sidx * 16;
          if (o0 >= p.d) o0 = 0;
          rt = o0 >> 4;
          cm = fd;
          sm_ = 3 * fd / 2 + 2 * (fd / 32);
        }
        coff = cm + (size_t)rt * 8 * K;
        soff = sm_ + (size_t)rt * (K / 2);
      };
      size_t co, so;
      strip_base(2 * wave + (ln >> 5), co, so);
      cptr = W + co + (ln & 31) * 16;
      if (wave < 2) {
        size_t co2, so2;
        strip_base(8 * wave + (ln >> 3), co2, so2);
        sptr = W + so2 + (ln & 7) * 4;
      }
    }
    auto issue = [&](int S, int ks) {
      uint8_t* st = sm[S];
      const uint32_t sa = x_lds_addr(st);
      const int kk = ks * XBK, kt = ks >> 1, h = ks & 1;
#pragma unroll
      for (int t = 0; t < 4; ++t) x_g2lds16(abase + oa[t] + kk, sa + (4 * wave + t) * 8 * XBK * 2);
      x_g2lds16(cptr + (size_t)kt * 1024 + h * 512, sa + XA_BYTES + wave * 1024);
      if (wave < 2) x_g2lds4(sptr + (size_t)kt * 64 + h * 32, sa + XA_BYTES + XC_BYTES + wave * 256);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;

    __syncthreads();  // the previous item's readers of the ring are done
    issue(0, 0);
    auto step = [&](int S, auto am_tag, int ks) {
      constexpr int AM = decltype(am_tag)::value;
      x_wait_vm0();
      lds_barrier();
      if (ks + 1 < nk) issue(S ^ 1, ks + 1);
      const uint8_t* st = sm[S];
      const uint16_t* sa16 = (const uint16_t*)st;
      const uint8_t* sc = st + XA_BYTES;
      const uint8_t* ss = st + XA_BYTES + XC_BYTES;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 aq[4], bq[2];
#pragma unroll
        for (int i = 0; i < AM; ++i) aq[i] = as_bf16x8(*(const u32x4*)&sa16[xswz(wm * 128 + i * 32 + r32, 2 * s + g)]);
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
          const int R = wn * 64 + jn * 32 + r32, sidx = R >> 4, i16 = R & 15, qq = s >> 1;
          const uint32_t w = *(const uint32_t*)(sc + sidx * 512 + (16 * qq + i16) * 16 + (s & 1) * 8 + g * 4);
          const uint32_t sv = ss[sidx * 32 + 16 * qq + i16];
          bq[jn] = mx_expand8(w, e8m0_scale(sv));
        }
#pragma unroll
        for (int i = 0; i < AM; ++i) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[i], bq[0], acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[i], bq[1], acc[i][1], 0, 0, 0);
        }
      }
    };
    auto run_k = [&](auto am_tag) {
      for (int ks = 0; ks < nk; ks += 2) {
        step(0, am_tag, ks);
        if (ks + 1 < nk) step(1, am_tag, ks + 1);
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

    int ld = MODE == 0 ? p.f : p.d;
    asm volatile("" : "+s"(ld));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (wm * 4 + i >= mtiles) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m >= rows) continue;
        if (MODE == 0) {
          const int unit = nt * 128 + wn * 32 + r32;
          if (unit < p.f)
            ((uint16_t*)p.h)[(size_t)(n0 + m) * ld + unit] = f32_to_bf16(x_swiglu(acc[i][0][v], acc[i][1][v]));
        } else {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const int o = nt * 256 + wn * 64 + jn * 32 + r32;
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

namespace {

int launch_tile256(const FfnArgs& p, int y_dtype, hipStream_t stream) {
  const dim3 grid((num_cus() + 7) / 8 * 8), blk(512);
  hipLaunchKernelGGL((mx_tile256<0, MOE_BF16>), grid, blk, 0, stream, p, (p.f + 127) / 128);
  MOE_LAUNCH_CHECK();
  const int ntd = (p.d + 255) / 256;
  if (y_dtype == MOE_F32) hipLaunchKernelGGL((mx_tile256<1, MOE_F32>), grid, blk, 0, stream, p, ntd);
  else hipLaunchKernelGGL((mx_tile256<1, MOE_BF16>), grid, blk, 0, stream, p, ntd);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

// The 256 x 256 tiles for experts with many rows: the experts of a decode call that have more
// rows than the weight-streaming kernels take (nmin > 1), and calls that average at least 32
// rows per expert (at 256 experts, top 6: from about 1400 tokens).  With fewer rows per expert
// the 64 x 128 tiles keep more workgroups streaming per CU: at Zipf 0.2, T = 512 and 1024,
// they take 1.07 and 1.25 ms against 1.31 and 1.36 (at Zipf 1, where a few hot experts hold
// most rows, the large tiles are ahead at every T measured: 0.52 vs 1.03 ms at T = 512).
int launch_ffn_mx_gemm(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts) {
  if (p.nmin > 1 || (long long)T * p.k >= 32ll * p.E) return launch_tile256(p, y_dtype, stream);
  // (expert, 64-row block) pairs: at most T*k/64 + (number of experts with rows)
  const long A = (long)T * p.k;
  const long mbs = A / kMgM + std::min<long>(experts > 0 ? std::min(experts, p.E) : p.E, A);
  auto grid = [&](int R) {
    const long g = mbs * ((R + kMgN - 1) / kMgN);
    return dim3((unsigned)((g + 7) / 8 * 8));
  };
  hipLaunchKernelGGL(mg_gateup, grid(p.f), dim3(256), 0, stream, p);
  MOE_LAUNCH_CHECK();
  if (y_dtype == MOE_F32) hipLaunchKernelGGL(mg_down<MOE_F32>, grid(p.d), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(mg_down<MOE_BF16>, grid(p.d), dim3(256), 0, stream, p);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
