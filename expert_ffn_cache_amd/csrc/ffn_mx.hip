// Decode-shaped expert FFN with MXFP4 expert weights: FP4 codes are expanded to bf16 in
// registers (v_cvt_scalef32_pk_bf16_fp4, exact for E8M0 scales) and multiplied on the matrix
// cores (v_mfma_f32_16x16x32_bf16) against bf16 token rows staged in LDS.
//
// Entry layout (bytes): [codes of W_gate][codes of W_up][codes of W_down][scales of W_gate]
// [scales of W_up][scales of W_down].  Each R x K matrix (R a multiple of 16, K of 32) is
// stored in tiles of 16 rows x 128 elements: row strip rt (rows 16 rt .. 16 rt + 15) starts
// at byte 8 K rt of the matrix's codes and K/2 rt of its scales, tile kt of the strip at
// +1024 kt / +64 kt (the strip's last tile holds the K mod 128 elements left, if any), and
// slot l = 16 q + i of a tile holds the 16 code bytes / the scale byte of row i, elements
// 32 q .. 32 q + 31 of the tile (element 2j in the low nibble of code byte j).
//
// So one 16-byte load per lane brings a whole tile (1 KB per wave, contiguous in memory),
// and lane l = 16 q + i then holds exactly what the MFMA B operand wants in lane l for four
// consecutive MFMAs: column i (weight row), reduction group q, 8 elements each.  The MFMA
// reduction index is thereby a permutation of the tile's 128 elements; the A operand (token
// rows, 16 per MFMA; rows past the expert's count repeat a staged row and their outputs are
// dropped) is read from LDS under the same permutation.  With the dot products on the
// matrix cores the vector ALUs only expand codes (half an instruction per weight), which
// keeps the kernels bound by the HBM stream of the codes.
//
// Work split: a wave streams a whole strip of 16 weight rows (a workgroup's four waves take
// four strips of one expert), keeping kMxAhead tiles in flight.  When that leaves too few
// workgroups to fill the chip (one or two tokens), KS = 2 or 4 waves share a strip, wave ks
// taking tiles ks, ks + KS, ...; their partial sums meet in LDS and the strip's first wave
// writes the result.
#include <algorithm>

#include "ffn_args.h"

namespace moe {
namespace {

constexpr int kMxNTL = 4;    // token rows staged per pass
constexpr int kMxAhead = 4;  // tiles in flight per wave

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);  // 2^(s - 127)
}

// The 8 weights of code word w (element order: low nibble of byte 0 first), times scale.
__device__ __forceinline__ bf16x8 mx_expand8(uint32_t w, float sc) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                 __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int NMAT>
struct MxTile {
  u32x4 c[NMAT];  // this lane's 16 code bytes of the tile, per matrix
  uint32_t s[NMAT];
};

// Tile kt of the wave's strip(s).  ok: the lane's block exists (false only in a short last
// tile); missing blocks read as zero weights.
template <int NMAT>
__device__ __forceinline__ void mx_load_tile(MxTile<NMAT>& t, const uint8_t* const (&cb)[NMAT],
                                             const uint8_t* const (&sb)[NMAT], int kt, int lane,
                                             bool ok) {
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    if (ok) {
      t.c[m] = ldg16_nt(cb[m] + (size_t)kt * 1024 + lane * 16);
      t.s[m] = ldg_u8(sb[m] + (size_t)kt * 64 + lane);
    } else {
      t.c[m] = u32x4{0u, 0u, 0u, 0u};
      t.s[m] = 0u;
    }
  }
  issue_fence();
}

// acc[m] += (16 staged rows) x (tile of matrix m)^T; xa = this lane's activations of the tile.
template <int NMAT>
__device__ __forceinline__ void mx_tile_mma(const MxTile<NMAT>& t, const uint16_t* xa,
                                            f32x4 (&acc)[NMAT]) {
  bf16x8 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = as_bf16x8(*(const u32x4*)(xa + 8 * j));
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const float sc = e8m0_scale(t.s[m]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[j], mx_expand8(t.c[m][j], sc), acc[m], 0, 0, 0);
  }
}

// One wave's share of a strip: tiles ks, ks + KS, ... of the nk tiles over K (the last
// one short when krem = (K mod 128) / 32 > 0), kMxAhead of them in flight in `ring`.
// mx_ring_fill issues the first loads (before the token rows are staged, so the two
// overlap); mx_ring_run multiplies every tile and issues the rest.  xrow: start of the
// lane's staged row; cb/sb: the strip's codes and scales.
template <int NMAT, int KS>
__device__ __forceinline__ void mx_ring_fill(MxTile<NMAT> (&ring)[kMxAhead],
                                             const uint8_t* const (&cb)[NMAT],
                                             const uint8_t* const (&sb)[NMAT], int ks, int nk,
                                             int krem, int lane) {
  const int q = lane >> 4;
  const int ntw = nk > ks ? (nk - ks + KS - 1) / KS : 0;
  const int kshort = krem ? nk - 1 : -1;
#pragma unroll
  for (int r = 0; r < kMxAhead; ++r) {
    const int kt = ks + KS * r;
    if (r < ntw) mx_load_tile<NMAT>(ring[r], cb, sb, kt, lane, kt != kshort || q < krem);
  }
}

template <int NMAT, int KS>
__device__ __forceinline__ void mx_ring_run(MxTile<NMAT> (&ring)[kMxAhead],
                                            const uint8_t* const (&cb)[NMAT],
                                            const uint8_t* const (&sb)[NMAT], const uint16_t* xrow,
                                            int ks, int nk, int krem, int lane, f32x4 (&acc)[NMAT]) {
  const int q = lane >> 4;
  const int ntw = nk > ks ? (nk - ks + KS - 1) / KS : 0;  // tiles of this wave
  const int kshort = krem ? nk - 1 : -1;                  // index of a short last tile
  for (int i = 0; i < ntw; i += kMxAhead) {
#pragma unroll
    for (int r = 0; r < kMxAhead; ++r) {
      const int ii = i + r;
      if (ii < ntw) {
        const int kt = ks + KS * ii;
        const bool ok = kt != kshort || q < krem;
        mx_tile_mma<NMAT>(ring[r], xrow + kt * 128 + (ok ? 32 * q : 0), acc);
        const int kn = kt + KS * kMxAhead;
        if (ii + kMxAhead < ntw) mx_load_tile<NMAT>(ring[r], cb, sb, kn, lane, kn != kshort || q < krem);
      }
    }
  }
}

// Workgroup -> active expert (one wave finds it, shared through LDS).
struct MxItem {
  int e;
  const uint8_t* w;
};

// The a-th active expert in ascending id (called by one full wave), the offsets of 256
// experts read in one round trip: a workgroup here streams little, so its start-up latency
// shows.
__device__ __forceinline__ int mx_nth_active(const FfnArgs& p, int a) {
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int e0 = 0; e0 < p.E; e0 += 256) {
    int n[4];
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = min(e0 + 64 * j + lane, p.E - 1);
      n[j] = p.offsets[e + 1] - p.offsets[e];
      ok[j] = !p.mask || p.mask[e];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 64 * j + lane;
      const bool act = e < p.E && n[j] > 0 && n[j] >= p.nmin && n[j] <= p.nmax && ok[j];
      const unsigned long long m = __ballot(act);
      const int c = __popcll(m);
      if (a < seen + c) {
        const bool mine = act && __popcll(m & lanemask_lt(lane)) == a - seen;
        return e0 + 64 * j + __ffsll((long long)__ballot(mine)) - 1;
      }
      seen += c;
    }
  }
  return -1;
}

__device__ __forceinline__ MxItem mx_item(const FfnArgs& p, int a) {
  __shared__ int s_e;
  __shared__ const char* s_w;
  if (threadIdx.x < 64) {
    const int e = mx_nth_active(p, a);
    if (threadIdx.x == 0) {
      s_e = e;
      s_w = e >= 0 ? entry_of(p, e) : nullptr;
    }
  }
  __syncthreads();
  return MxItem{s_e, (const uint8_t*)s_w};
}

// nt token rows of K bf16 into LDS at row stride K + 8 (the 16-byte pad spreads the rows
// that one MFMA operand read touches over distinct banks).
template <typename RowOf>
__device__ __forceinline__ void mx_stage(uint16_t* lds, const uint16_t* src, int K, int nt,
                                         RowOf src_row) {
  const int nck = K >> 3;
  __syncthreads();  // the previous pass's readers are done
  for (int c = threadIdx.x; c < nt * nck; c += blockDim.x) {
    const int t = c / nck, k8 = c - t * nck;
    *(u32x4*)&lds[t * (K + 8) + k8 * 8] = ldg16(src + (size_t)src_row(t) * K + k8 * 8);
  }
  __syncthreads();
}

// Partial sums of the KS waves of each strip: waves ks > 0 store, then the first wave adds.
template <int NMAT, int KS>
__device__ __forceinline__ void mx_reduce(f32x4 (&acc)[NMAT], int strip, int ks, int lane) {
  if (KS == 1) return;
  __shared__ f32x4 red[3][NMAT][64];
  if (ks > 0) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) red[strip * (KS - 1) + ks - 1][m][lane] = acc[m];
  }
  __syncthreads();
  if (ks == 0) {
#pragma unroll
    for (int j = 1; j < KS; ++j)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[m] += red[strip * (KS - 1) + j - 1][m][lane];
  }
}

// Gate/up: workgroup = 4/KS strips of 16 units of one expert.
template <int KS>
__global__ __launch_bounds__(256) void mx_gateup(FfnArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  constexpr int TR = 4 / KS;
  const int nb = p.f / (16 * TR);
  const int a = blockIdx.x / nb, sb0 = blockIdx.x - a * nb;
  const MxItem it = mx_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = wave / KS, ks = wave - strip * KS, rt = sb0 * TR + strip;
  const int K = p.d, nk = (K + 127) >> 7, krem = (K & 127) >> 5;
  const size_t fd = (size_t)p.f * K;
  const uint8_t* W = it.w;
  const uint8_t* const cb[2] = {W + (size_t)rt * 8 * K, W + fd / 2 + (size_t)rt * 8 * K};
  const uint8_t* const sb[2] = {W + 3 * fd / 2 + (size_t)rt * (K / 2),
                                W + 3 * fd / 2 + fd / 32 + (size_t)rt * (K / 2)};
  uint16_t* H = (uint16_t*)p.h;
  const int col = lane & 15, kg = lane >> 4;
  for (int m0 = 0; m0 < n; m0 += kMxNTL) {
    const int nt = min(kMxNTL, n - m0);
    MxTile<2> ring[kMxAhead];
    mx_ring_fill<2, KS>(ring, cb, sb, ks, nk, krem, lane);
    mx_stage(xs, (const uint16_t*)p.x, K, nt, [&](int t) { return p.perm[n0 + m0 + t] / p.k; });
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    mx_ring_run<2, KS>(ring, cb, sb, xs + min(col, nt - 1) * (K + 8), ks, nk, krem, lane, acc);
    mx_reduce<2, KS>(acc, strip, ks, lane);
    if (ks == 0) {
      // lane holds C[4 kg + i][col]: token rows 4 kg + i, unit 16 rt + col
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * kg + i;
        if (t < nt) H[(size_t)(n0 + m0 + t) * p.f + 16 * rt + col] = f32_to_bf16(silu(acc[0][i]) * acc[1][i]);
      }
    }
  }
}

// Down: workgroup = 4/KS strips of 16 output channels of one expert.
template <int KS, int YDT>
__global__ __launch_bounds__(256) void mx_down(FfnArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
  constexpr int TR = 4 / KS;
  const int nb = p.d / (16 * TR);
  const int a = blockIdx.x / nb, sb0 = blockIdx.x - a * nb;
  const MxItem it = mx_item(p, a);
  if (it.e < 0 || !it.w) return;
  const int n0 = p.offsets[it.e], n = p.offsets[it.e + 1] - n0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = wave / KS, ks = wave - strip * KS, rt = sb0 * TR + strip;
  const int K = p.f, nk = (K + 127) >> 7, krem = (K & 127) >> 5;
  const size_t fd = (size_t)K * p.d;
  const uint8_t* W = it.w;
  const uint8_t* const cb[1] = {W + fd + (size_t)rt * 8 * K};
  const uint8_t* const sb[1] = {W + 3 * fd / 2 + 2 * (fd / 32) + (size_t)rt * (K / 2)};
  const int col = lane & 15, kg = lane >> 4;
  for (int m0 = 0; m0 < n; m0 += kMxNTL) {
    const int nt = min(kMxNTL, n - m0);
    MxTile<1> ring[kMxAhead];
    mx_ring_fill<1, KS>(ring, cb, sb, ks, nk, krem, lane);
    mx_stage(hs, (const uint16_t*)p.h, K, nt, [&](int t) { return n0 + m0 + t; });
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    mx_ring_run<1, KS>(ring, cb, sb, hs + min(col, nt - 1) * (K + 8), ks, nk, krem, lane, acc);
    mx_reduce<1, KS>(acc, strip, ks, lane);
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * kg + i;
        if (t < nt) {
          const size_t o = (size_t)(n0 + m0 + t) * p.d + 16 * rt + col;
          if (YDT == MOE_F32) ((float*)p.y)[o] = acc[0][i];
          else ((uint16_t*)p.y)[o] = f32_to_bf16(acc[0][i]);
        }
      }
    }
  }
}

// Waves per strip: one (a wave streams whole strips, no partial sums) unless that leaves
// fewer than 4 workgroups per CU, as with one or two tokens; then the strips' tiles are
// split over 2 or 4 waves.
int mx_ks(int experts, int R) {
  const long strips = (long)experts * (R / 16);
  return strips / 4 >= 1024 ? 1 : strips / 2 >= 1024 ? 2 : 4;
}

template <int KS>
void launch_gu(const FfnArgs& p, int experts, hipStream_t stream) {
  const dim3 grid(experts * (p.f / (16 * (4 / KS))));
  hipLaunchKernelGGL(mx_gateup<KS>, grid, dim3(256), (size_t)kMxNTL * (p.d + 8) * 2, stream, p);
}

template <int KS, int YDT>
void launch_dn(const FfnArgs& p, int experts, hipStream_t stream) {
  const dim3 grid(experts * (p.d / (16 * (4 / KS))));
  hipLaunchKernelGGL((mx_down<KS, YDT>), grid, dim3(256), (size_t)kMxNTL * (p.f + 8) * 2, stream, p);
}

template <int YDT>
void launch_dn_ks(const FfnArgs& p, int experts, hipStream_t stream) {
  switch (mx_ks(experts, p.d)) {
    case 1: launch_dn<1, YDT>(p, experts, stream); break;
    case 2: launch_dn<2, YDT>(p, experts, stream); break;
    default: launch_dn<4, YDT>(p, experts, stream); break;
  }
}

}  // namespace

bool ffn_mx_supported(int d, int f) {
  // strips of 16 rows grouped 4/KS per workgroup (d, f multiples of 64 cover every KS);
  // staged rows must fit the LDS (64 KB per workgroup)
  return d % 64 == 0 && f % 64 == 0 && (size_t)kMxNTL * (std::max(d, f) + 8) * 2 <= 65536;
}

int launch_ffn_mx(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts) {
  if (experts <= 0) return MOE_OK;
  switch (mx_ks(experts, p.f)) {
    case 1: launch_gu<1>(p, experts, stream); break;
    case 2: launch_gu<2>(p, experts, stream); break;
    default: launch_gu<4>(p, experts, stream); break;
  }
  MOE_LAUNCH_CHECK();
  if (y_dtype == MOE_F32) launch_dn_ks<MOE_F32>(p, experts, stream);
  else launch_dn_ks<MOE_BF16>(p, experts, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
