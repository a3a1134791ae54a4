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
#include <type_traits>

#include "ffn_args.h"
#include "mx_dev.h"

namespace moe {
namespace {

// An expert's token rows are staged in LDS in blocks over slices of the contraction: up to 4
// rows over all of K, up to 8 over each half, up to 16 over each quarter (the same 33 KB at
// K = 4096, so 4 workgroups per CU whatever the row count), the accumulators carrying over from
// slice to slice.  An expert with up to 16 rows thus streams its weights once, and the
// MFMA's 16 token columns do the work of 9-16 rows in one stream; with 4 rows per pass over all
// of K it streamed them once per 4 rows.  Slices are whole tiles; fewer slices are taken where
// the staged block would not fit 64 KB of LDS.
__host__ __device__ constexpr int mx_slice_tiles(int nk, int C) { return (nk + C - 1) / C; }
__host__ __device__ constexpr int mx_slice_stride(int K, int C) {  // LDS row stride (elements)
  return C == 1 ? K + 8 : mx_slice_tiles((K + 127) >> 7, C) * 128 + 8;
}
__host__ __device__ constexpr int mx_block_elems(int K, int C) { return 4 * C * mx_slice_stride(K, C); }
__host__ __device__ constexpr int mx_max_slices(int K) {
  return mx_block_elems(K, 4) <= 32768 ? 4 : mx_block_elems(K, 2) <= 32768 ? 2 : 1;
}
// slices for an expert of n rows (a block holds 4 rows per slice), and the LDS bytes a launch
// stages the rows in
__host__ __device__ constexpr int mx_slices(int n, int K) {
  return n <= 4 ? 1 : n <= 8 && mx_max_slices(K) >= 2 ? 2 : mx_max_slices(K);
}
__host__ __device__ constexpr size_t mx_stage_bytes(int K) {
  const int cm = mx_max_slices(K);
  int e = mx_block_elems(K, 1);
  if (cm >= 2 && mx_block_elems(K, 2) > e) e = mx_block_elems(K, 2);
  if (cm >= 4 && mx_block_elems(K, 4) > e) e = mx_block_elems(K, 4);
  return 2 * (size_t)e;
}
constexpr int kMxAhead = 4;  // tiles in flight per wave

// One wave's share of a strip's tiles t0 .. t1 - 1 (one slice): tiles t0 + ks, t0 + ks + KS,
// ... of the nk tiles over K (the last one short when krem = (K mod 128) / 32 > 0), kMxAhead
// of them in flight in `ring`.  mx_ring_fill issues the first loads (before the token rows
// are staged, so the two overlap); mx_ring_run multiplies every tile and issues the rest.
// xrow: start of the lane's staged row (the slice's elements); cb/sb: the strip's codes and
// scales.
template <int NMAT, int KS>
__device__ __forceinline__ void mx_ring_fill(MxTile<NMAT> (&ring)[kMxAhead],
                                             const uint8_t* const (&cb)[NMAT],
                                             const uint8_t* const (&sb)[NMAT], int ks, int t0,
                                             int t1, int nk, int krem, int lane) {
  const int q = lane >> 4;
  const int ntw = t1 - t0 > ks ? (t1 - t0 - ks + KS - 1) / KS : 0;
  const int kshort = krem ? nk - 1 : -1;
#pragma unroll
  for (int r = 0; r < kMxAhead; ++r) {
    const int kt = t0 + ks + KS * r;
    if (r < ntw) mx_load_tile<NMAT>(ring[r], cb, sb, kt, lane, kt != kshort || q < krem);
  }
}

template <int NMAT, int KS>
__device__ __forceinline__ void mx_ring_run(MxTile<NMAT> (&ring)[kMxAhead],
                                            const uint8_t* const (&cb)[NMAT],
                                            const uint8_t* const (&sb)[NMAT], const uint16_t* xrow,
                                            int ks, int t0, int t1, int nk, int krem, int lane,
                                            f32x4 (&acc)[NMAT]) {
  const int q = lane >> 4;
  const int ntw = t1 - t0 > ks ? (t1 - t0 - ks + KS - 1) / KS : 0;  // tiles of this wave
  const int kshort = krem ? nk - 1 : -1;                            // index of a short last tile
  for (int i = 0; i < ntw; i += kMxAhead) {
#pragma unroll
    for (int r = 0; r < kMxAhead; ++r) {
      const int ii = i + r;
      if (ii < ntw) {
        const int kt = t0 + ks + KS * ii;
        const bool ok = kt != kshort || q < krem;
        mx_tile_mma<NMAT>(ring[r], xrow + (kt - t0) * 128 + (ok ? 32 * q : 0), acc);
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

// Elements e0 .. e0 + len - 1 of nt token rows of K bf16 into LDS at row stride `stride`
// (K + 8 or a slice's tiles + 8: the 16-byte pad spreads the rows that one MFMA operand read
// touches over distinct banks).
template <typename RowOf>
__device__ __forceinline__ void mx_stage(uint16_t* lds, const uint16_t* src, int K, int e0,
                                         int len, int stride, int nt, RowOf src_row) {
  const int nck = len >> 3;
  __syncthreads();  // the previous slice's readers are done
  for (int c = threadIdx.x; c < nt * nck; c += blockDim.x) {
    const int t = c / nck, k8 = c - t * nck;
    *(u32x4*)&lds[t * stride + k8 * 8] = ldg16(src + (size_t)src_row(t) * K + e0 + k8 * 8);
  }
  __syncthreads();
}

// One launch for both projections (up to kMxMaxRows tokens): gate/up workgroups come first
// in the grid and publish h as 8-byte entries, units 2c and 2c + 1 of a row (bf16, low half
// first) in the low word and kMxTag in the high word, each written with one device-coherent
// single-copy-atomic store; a down workgroup reads its expert's entries device-coherently
// and uses them once every one carries the tag.  The eight L2 caches are not coherent with
// one another, and this keeps the exchange free of cache maintenance (see the single-token
// launch, which exchanges h the same way).  The entries are zeroed by a small kernel before
// the launch, so the tag is the same on every call.  Workgroups are dispatched in grid order,
// so every gate/up workgroup is dispatched before any down workgroup, and gate/up workgroups
// never wait: every wait ends.  It is bounded all the same (MOE_ETIMEOUT).
constexpr uint32_t kMxTag = 1u;
constexpr unsigned kMxSpinLimit = 1u << 18;  // polls of a row block of h (about a second)

__device__ __forceinline__ uint64_t mx_coh_load64(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void mx_coh_store64(uint64_t* a, uint64_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Units e0 .. e0 + len - 1 of nt rows of h (K units each, entries of rows row0 ..) into LDS
// at row stride `stride`, once every entry carries the tag: each thread loads its entries
// (eight in flight) and writes the values, and the workgroup repeats until no thread found an
// untagged one.
template <bool WHOLE>
__device__ __forceinline__ void mx_stage_ent(uint16_t* lds, const uint64_t* hent, int K, int e0,
                                             int len, int stride, int nt, int row0,
                                             int32_t* status) {
  const int ne = K >> 1, nes = len >> 1, n = nt * nes;
  const uint64_t* src = hent + (size_t)row0 * ne + (e0 >> 1);
  uint32_t* dst = (uint32_t*)lds;
  __syncthreads();  // the previous slice's readers are done
  for (unsigned polls = 1;; ++polls) {
    int stale = 0;
    for (int c0 = 0; c0 < n; c0 += 8 * 256) {
      uint64_t v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int c = min(c0 + r * 256 + (int)threadIdx.x, n - 1);
        if (WHOLE) {  // rows are contiguous
          v[r] = mx_coh_load64(src + c);
        } else {
          const int t = c / nes;
          v[r] = mx_coh_load64(src + (size_t)t * ne + (c - t * nes));
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int c = c0 + r * 256 + threadIdx.x;
        if (c < n) {
          const int t = c / nes, q = c - t * nes;
          stale |= (uint32_t)(v[r] >> 32) != kMxTag;
          dst[t * (stride >> 1) + q] = (uint32_t)v[r];
        }
      }
    }
    if (!__syncthreads_or(stale)) return;
    if (polls >= kMxSpinLimit) {
      if (threadIdx.x == 0) set_status(status, MOE_ETIMEOUT);
      return;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Partial sums of the KS waves of each strip through red ([3][NMAT][64] in LDS), as
// mx_reduce does through its own array.
template <int NMAT, int KS>
__device__ __forceinline__ void mx_reduce_buf(f32x4 (&acc)[NMAT], int strip, int ks, int lane,
                                              f32x4* red) {
  if (KS == 1) return;
  if (ks > 0) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) red[((strip * (KS - 1) + ks - 1) * NMAT + m) * 64 + lane] = acc[m];
  }
  __syncthreads();
  if (ks == 0) {
#pragma unroll
    for (int j = 1; j < KS; ++j)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[m] += red[((strip * (KS - 1) + j - 1) * NMAT + m) * 64 + lane];
  }
}

// Gate/up: workgroup = 4/KS strips of 16 units of one expert.  ENT: h as tagged entries,
// partial sums through red.
template <int KS, bool ENT>
__device__ __forceinline__ void gu_body(const FfnArgs& p, int bid, f32x4* red) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  constexpr int TR = 4 / KS;
  const int nb = p.f / (16 * TR);
  const int a = bid / nb, sb0 = bid - a * nb;
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
  // blocks of up to 4 C rows, each over C slices of K (compiled per C, so one slice is the
  // plain pass over all of K)
  auto blocks = [&](auto c_tag) {
    constexpr int C = decltype(c_tag)::value;
    const int rb = 4 * C, tps = mx_slice_tiles(nk, C), stride = mx_slice_stride(K, C);
    for (int m0 = 0; m0 < n; m0 += rb) {
      const int nt = min(rb, n - m0);
      auto row_of = [&](int t) { return p.perm[n0 + m0 + t] / p.k; };
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (C == 1) {
        MxTile<2> ring[kMxAhead];
        mx_ring_fill<2, KS>(ring, cb, sb, ks, 0, nk, nk, krem, lane);
        mx_stage(xs, (const uint16_t*)p.x, K, 0, K, K + 8, nt, row_of);
        mx_ring_run<2, KS>(ring, cb, sb, xs + min(col, nt - 1) * (K + 8), ks, 0, nk, nk, krem, lane, acc);
      } else {
        for (int t0 = 0; t0 < nk; t0 += tps) {
          const int t1 = min(nk, t0 + tps), e0 = t0 * 128, len = min(K, t1 * 128) - e0;
          MxTile<2> ring[kMxAhead];
          mx_ring_fill<2, KS>(ring, cb, sb, ks, t0, t1, nk, krem, lane);
          mx_stage(xs, (const uint16_t*)p.x, K, e0, len, stride, nt, row_of);
          mx_ring_run<2, KS>(ring, cb, sb, xs + min(col, nt - 1) * stride, ks, t0, t1, nk, krem, lane, acc);
        }
      }
      if (ENT) mx_reduce_buf<2, KS>(acc, strip, ks, lane, red);
      else mx_reduce<2, KS>(acc, strip, ks, lane);
      if (ks == 0) {
        // lane holds C[4 kg + i][col]: token rows 4 kg + i, unit 16 rt + col
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * kg + i;
          const uint32_t hv = f32_to_bf16(silu(acc[0][i]) * acc[1][i]);
          if (ENT) {
            const uint32_t nv = (uint32_t)__shfl_xor((int)hv, 1);  // unit 16 rt + (col ^ 1)
            if (t < nt && !(col & 1))
              mx_coh_store64((uint64_t*)p.h + ((size_t)(n0 + m0 + t) * p.f + 16 * rt + col) / 2,
                             (uint64_t)(hv | nv << 16) | (uint64_t)kMxTag << 32);
          } else if (t < nt) {
            H[(size_t)(n0 + m0 + t) * p.f + 16 * rt + col] = (uint16_t)hv;
          }
        }
      }
    }
  };
  switch (mx_slices(n, K)) {
    case 1: blocks(std::integral_constant<int, 1>{}); break;
    case 2: blocks(std::integral_constant<int, 2>{}); break;
    default: blocks(std::integral_constant<int, 4>{}); break;
  }
}

template <int KS>
__global__ __launch_bounds__(256) void mx_gateup(FfnArgs p) { gu_body<KS, false>(p, blockIdx.x, nullptr); }

// Down: workgroup = 4/KS strips of 16 output channels of one expert.  ENT: h read from the
// tagged entries, partial sums through red.
template <int KS, int YDT, bool ENT>
__device__ __forceinline__ void dn_body(const FfnArgs& p, int bid, f32x4* red) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
  constexpr int TR = 4 / KS;
  const int nb = p.d / (16 * TR);
  const int a = bid / nb, sb0 = bid - a * nb;
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
  auto blocks = [&](auto c_tag) {  // as in gate/up
    constexpr int C = decltype(c_tag)::value;
    const int rb = 4 * C, tps = mx_slice_tiles(nk, C), stride = mx_slice_stride(K, C);
    for (int m0 = 0; m0 < n; m0 += rb) {
      const int nt = min(rb, n - m0);
      auto row_of = [&](int t) { return n0 + m0 + t; };
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (C == 1) {
        MxTile<1> ring[kMxAhead];
        mx_ring_fill<1, KS>(ring, cb, sb, ks, 0, nk, nk, krem, lane);
        if (ENT) mx_stage_ent<true>(hs, (const uint64_t*)p.h, K, 0, K, K + 8, nt, n0 + m0, p.status);
        else mx_stage(hs, (const uint16_t*)p.h, K, 0, K, K + 8, nt, row_of);
        mx_ring_run<1, KS>(ring, cb, sb, hs + min(col, nt - 1) * (K + 8), ks, 0, nk, nk, krem, lane, acc);
      } else {
        for (int t0 = 0; t0 < nk; t0 += tps) {
          const int t1 = min(nk, t0 + tps), e0 = t0 * 128, len = min(K, t1 * 128) - e0;
          MxTile<1> ring[kMxAhead];
          mx_ring_fill<1, KS>(ring, cb, sb, ks, t0, t1, nk, krem, lane);
          if (ENT) mx_stage_ent<false>(hs, (const uint64_t*)p.h, K, e0, len, stride, nt, n0 + m0, p.status);
          else mx_stage(hs, (const uint16_t*)p.h, K, e0, len, stride, nt, row_of);
          mx_ring_run<1, KS>(ring, cb, sb, hs + min(col, nt - 1) * stride, ks, t0, t1, nk, krem, lane, acc);
        }
      }
      if (ENT) mx_reduce_buf<1, KS>(acc, strip, ks, lane, red);
      else mx_reduce<1, KS>(acc, strip, ks, lane);
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
  };
  switch (mx_slices(n, K)) {
    case 1: blocks(std::integral_constant<int, 1>{}); break;
    case 2: blocks(std::integral_constant<int, 2>{}); break;
    default: blocks(std::integral_constant<int, 4>{}); break;
  }
}

template <int KS, int YDT>
__global__ __launch_bounds__(256) void mx_down(FfnArgs p) { dn_body<KS, YDT, false>(p, blockIdx.x, nullptr); }

// Both projections in one grid: n_gu gate/up workgroups (one wave per strip), then the
// down workgroups (KSD waves per strip).
template <int KSD, int YDT>
__global__ __launch_bounds__(256) void mx_ffn1(FfnArgs p, int n_gu) {
  __shared__ f32x4 red[3 * 64];
  if ((int)blockIdx.x < n_gu) gu_body<1, true>(p, blockIdx.x, red);
  else dn_body<KSD, YDT, true>(p, blockIdx.x - n_gu, red);
}

__global__ __launch_bounds__(256) void mx_ent_clear(uint64_t* ent, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    mx_coh_store64(ent + i, 0);
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
  hipLaunchKernelGGL(mx_gateup<KS>, grid, dim3(256), mx_stage_bytes(p.d), stream, p);
}

template <int KS, int YDT>
void launch_dn(const FfnArgs& p, int experts, hipStream_t stream) {
  const dim3 grid(experts * (p.d / (16 * (4 / KS))));
  hipLaunchKernelGGL((mx_down<KS, YDT>), grid, dim3(256), mx_stage_bytes(p.f), stream, p);
}

template <int YDT>
void launch_dn_ks(const FfnArgs& p, int experts, hipStream_t stream) {
  switch (mx_ks(experts, p.d)) {
    case 1: launch_dn<1, YDT>(p, experts, stream); break;
    case 2: launch_dn<2, YDT>(p, experts, stream); break;
    default: launch_dn<4, YDT>(p, experts, stream); break;
  }
}

template <int KSD>
void launch_one(const FfnArgs& p, int y_dtype, dim3 grid, size_t lds, hipStream_t stream, int n_gu) {
  if (y_dtype == MOE_F32) hipLaunchKernelGGL((mx_ffn1<KSD, MOE_F32>), grid, dim3(256), lds, stream, p, n_gu);
  else hipLaunchKernelGGL((mx_ffn1<KSD, MOE_BF16>), grid, dim3(256), lds, stream, p, n_gu);
}

}  // namespace

bool ffn_mx_supported(int d, int f) {
  // strips of 16 rows grouped 4/KS per workgroup (d, f multiples of 64 cover every KS);
  // staged rows must fit the LDS (64 KB per workgroup)
  return d % 64 == 0 && f % 64 == 0 && std::max(mx_stage_bytes(d), mx_stage_bytes(f)) <= 65536;
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

// One launch only where gate/up has a wave per strip (min(E, T k) * f >= 65536, e.g. from
// T = 6 at top 6 and f = 2048): with fewer strips the split-strip bodies hold 3 workgroups
// per CU and the clearing launch is not paid back (T = 2 and 4 at d = 4096, f = 2048: 3%
// slower), so those calls take the two launches.
int launch_ffn_mx_one(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts) {
  if (experts <= 0) return MOE_OK;
  if (mx_ks(experts, p.f) != 1) return launch_ffn_mx(p, y_dtype, stream, experts);
  const long n = (long)T * p.k * p.f / 2;  // h entries, one per two units of a row
  hipLaunchKernelGGL(mx_ent_clear, dim3((unsigned)std::min<long>(1024, (n + 1023) / 1024)), dim3(256), 0,
                     stream, (uint64_t*)p.h, n);
  MOE_LAUNCH_CHECK();
  const int ksd = mx_ks(experts, p.d);
  const int n_gu = experts * (p.f / 64);
  const int n_dn = experts * (p.d / (16 * (4 / ksd)));
  const dim3 grid(n_gu + n_dn);
  const size_t lds = std::max(mx_stage_bytes(p.d), mx_stage_bytes(p.f));
  switch (ksd) {
    case 1: launch_one<1>(p, y_dtype, grid, lds, stream, n_gu); break;
    case 2: launch_one<2>(p, y_dtype, grid, lds, stream, n_gu); break;
    default: launch_one<4>(p, y_dtype, grid, lds, stream, n_gu); break;
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
