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
#include "mx_dev.h"

namespace moe {
namespace {

// Token rows staged per pass.  Each pass streams the expert's weights again, and an expert
// has at most T rows; 4 rows (32.8 KB at d = 4096) keep 4 workgroups per CU.  Above 16 tokens
// (where experts with more rows go to the grouped GEMM) this kernel's experts have up to 16
// rows, and 6 rows per pass (49 KB, 3 workgroups per CU) pay for the lost workgroup: d = 4096,
// f = 2048, top 6, FFN at Zipf 0.2: T = 32 270 -> 263 us, T = 64 421 -> 398 us; Zipf 1: T = 32
// 193 -> 179 us, T = 64 217 -> 199 us.  Up to 16 tokens the fourth workgroup is worth more at
// Zipf 0.2 (T = 12: 132 against 138 us, T = 16: 163 against 170), though not when skewed
// (Zipf 1, T = 16: 119 against 97).  launch_ffn_mx_few takes those calls.
constexpr int kMxNTL = 4, kMxNTLWide = 6;
constexpr int kMxAhead = 4;  // tiles in flight per wave

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

// nt rows of h (K units each, entries of rows row0 ..) into LDS at row stride K + 8, once
// every entry carries the tag: each thread loads its entries (eight in flight) and writes the
// values, and the workgroup repeats until no thread found an untagged one.
__device__ __forceinline__ void mx_stage_ent(uint16_t* lds, const uint64_t* hent, int K, int nt,
                                             int row0, int32_t* status) {
  const int ne = K >> 1, n = nt * ne;
  const uint64_t* src = hent + (size_t)row0 * ne;
  uint32_t* dst = (uint32_t*)lds;
  __syncthreads();  // the previous pass's readers are done
  for (unsigned polls = 1;; ++polls) {
    int stale = 0;
    for (int c0 = 0; c0 < n; c0 += 8 * 256) {
      uint64_t v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = mx_coh_load64(src + min(c0 + r * 256 + (int)threadIdx.x, n - 1));
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int c = c0 + r * 256 + threadIdx.x;
        if (c < n) {
          const int t = c / ne, q = c - t * ne;
          stale |= (uint32_t)(v[r] >> 32) != kMxTag;
          dst[t * ((K + 8) >> 1) + q] = (uint32_t)v[r];
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
template <int KS, bool ENT, int NTL>
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
  for (int m0 = 0; m0 < n; m0 += NTL) {
    const int nt = min(NTL, n - m0);
    MxTile<2> ring[kMxAhead];
    mx_ring_fill<2, KS>(ring, cb, sb, ks, nk, krem, lane);
    mx_stage(xs, (const uint16_t*)p.x, K, nt, [&](int t) { return p.perm[n0 + m0 + t] / p.k; });
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    mx_ring_run<2, KS>(ring, cb, sb, xs + min(col, nt - 1) * (K + 8), ks, nk, krem, lane, acc);
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
}

template <int KS, int NTL>
__global__ __launch_bounds__(256) void mx_gateup(FfnArgs p) { gu_body<KS, false, NTL>(p, blockIdx.x, nullptr); }

// Down: workgroup = 4/KS strips of 16 output channels of one expert.  ENT: h read from the
// tagged entries, partial sums through red.
template <int KS, int YDT, bool ENT, int NTL>
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
  for (int m0 = 0; m0 < n; m0 += NTL) {
    const int nt = min(NTL, n - m0);
    MxTile<1> ring[kMxAhead];
    mx_ring_fill<1, KS>(ring, cb, sb, ks, nk, krem, lane);
    if (ENT) mx_stage_ent(hs, (const uint64_t*)p.h, K, nt, n0 + m0, p.status);
    else mx_stage(hs, (const uint16_t*)p.h, K, nt, [&](int t) { return n0 + m0 + t; });
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    mx_ring_run<1, KS>(ring, cb, sb, hs + min(col, nt - 1) * (K + 8), ks, nk, krem, lane, acc);
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
}

template <int KS, int YDT, int NTL>
__global__ __launch_bounds__(256) void mx_down(FfnArgs p) { dn_body<KS, YDT, false, NTL>(p, blockIdx.x, nullptr); }

// Both projections in one grid: n_gu gate/up workgroups (one wave per strip), then the
// down workgroups (KSD waves per strip).
template <int KSD, int YDT, int NTL>
__global__ __launch_bounds__(256) void mx_ffn1(FfnArgs p, int n_gu) {
  __shared__ f32x4 red[3 * 64];
  if ((int)blockIdx.x < n_gu) gu_body<1, true, NTL>(p, blockIdx.x, red);
  else dn_body<KSD, YDT, true, NTL>(p, blockIdx.x - n_gu, red);
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

template <int KS, int NTL>
void launch_gu(const FfnArgs& p, int experts, hipStream_t stream) {
  const dim3 grid(experts * (p.f / (16 * (4 / KS))));
  hipLaunchKernelGGL((mx_gateup<KS, NTL>), grid, dim3(256), (size_t)NTL * (p.d + 8) * 2, stream, p);
}

template <int KS, int YDT, int NTL>
void launch_dn(const FfnArgs& p, int experts, hipStream_t stream) {
  const dim3 grid(experts * (p.d / (16 * (4 / KS))));
  hipLaunchKernelGGL((mx_down<KS, YDT, NTL>), grid, dim3(256), (size_t)NTL * (p.f + 8) * 2, stream, p);
}

template <int YDT, int NTL>
void launch_dn_ks(const FfnArgs& p, int experts, hipStream_t stream) {
  switch (mx_ks(experts, p.d)) {
    case 1: launch_dn<1, YDT, NTL>(p, experts, stream); break;
    case 2: launch_dn<2, YDT, NTL>(p, experts, stream); break;
    default: launch_dn<4, YDT, NTL>(p, experts, stream); break;
  }
}

template <int NTL>
void launch_two(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts) {
  switch (mx_ks(experts, p.f)) {
    case 1: launch_gu<1, NTL>(p, experts, stream); break;
    case 2: launch_gu<2, NTL>(p, experts, stream); break;
    default: launch_gu<4, NTL>(p, experts, stream); break;
  }
  if (hipPeekAtLastError() != hipSuccess) return;
  if (y_dtype == MOE_F32) launch_dn_ks<MOE_F32, NTL>(p, experts, stream);
  else launch_dn_ks<MOE_BF16, NTL>(p, experts, stream);
}

template <int KSD, int NTL>
void launch_one(const FfnArgs& p, int y_dtype, dim3 grid, size_t lds, hipStream_t stream, int n_gu) {
  if (y_dtype == MOE_F32) hipLaunchKernelGGL((mx_ffn1<KSD, MOE_F32, NTL>), grid, dim3(256), lds, stream, p, n_gu);
  else hipLaunchKernelGGL((mx_ffn1<KSD, MOE_BF16, NTL>), grid, dim3(256), lds, stream, p, n_gu);
}

}  // namespace

bool ffn_mx_supported(int d, int f) {
  // strips of 16 rows grouped 4/KS per workgroup (d, f multiples of 64 cover every KS);
  // staged rows must fit the LDS (64 KB per workgroup)
  return d % 64 == 0 && f % 64 == 0 && (size_t)kMxNTL * (std::max(d, f) + 8) * 2 <= 65536;
}

int launch_ffn_mx(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts) {
  if (experts <= 0) return MOE_OK;
  launch_two<kMxNTL>(p, y_dtype, stream, experts);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// The experts with at most 16 rows of a call above 16 tokens: 6 token rows per pass where
// they fit the LDS, else 4.
int launch_ffn_mx_few(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts) {
  if (experts <= 0) return MOE_OK;
  if ((size_t)kMxNTLWide * (std::max(p.d, p.f) + 8) * 2 <= 65536)
    launch_two<kMxNTLWide>(p, y_dtype, stream, experts);
  else
    launch_two<kMxNTL>(p, y_dtype, stream, experts);
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
  const size_t lds = (size_t)kMxNTL * (std::max(p.d, p.f) + 8) * 2;
  switch (ksd) {
    case 1: launch_one<1, kMxNTL>(p, y_dtype, grid, lds, stream, n_gu); break;
    case 2: launch_one<2, kMxNTL>(p, y_dtype, grid, lds, stream, n_gu); break;
    default: launch_one<4, kMxNTL>(p, y_dtype, grid, lds, stream, n_gu); break;
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
