// MXFP4 weight tiles on the matrix cores, shared by the weight-streaming kernels and the
// one-launch single-token layer (so both take the same products in the same order).
//
// Each R x K matrix of an entry is stored in tiles of 16 rows x 128 elements (1 KB of codes,
// 64 scale bytes); slot l = 16 q + i of a tile holds the 16 code bytes and the scale byte of
// row i, elements 32 q .. 32 q + 31 (element 2j in the low nibble of code byte j).  One
// 16-byte load per lane brings a tile, and lane l then holds exactly what the B operand of
// v_mfma_f32_16x16x32_bf16 wants for four consecutive products: column i (weight row),
// reduction group q, 8 elements each.  Codes are expanded to bf16 in registers with
// v_cvt_scalef32_pk_bf16_fp4 (exact for E8M0 scales).
#pragma once

#include "common.h"

namespace moe {

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

}  // namespace moe
