// Arguments and helpers shared by the expert FFN kernels (fp32, GEMV and GEMM paths).
//
// For every active expert e and its grouped rows p in [offsets[e], offsets[e+1]):
//   h = SiLU(x[perm[p]/k] W_gate^T) * (x[perm[p]/k] W_up^T),   y_perm[p] = h W_down^T
// with the weights of e read from the cache entry at arena + expert_slot[e] * stride,
// laid out [W_gate f x d][W_up f x d][W_down d x f] (contraction index contiguous).
#pragma once

#include "common.h"

namespace moe {

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
  int nmin = 1, nmax = 0x7fffffff;  // only experts with nmin <= rows <= nmax are processed
  int items = 0x7fffffff;           // work items of a grid-stride launch (set by its launcher)
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
  const int n = p.offsets[e + 1] - p.offsets[e];
  return n > 0 && n >= p.nmin && n <= p.nmax && (!p.mask || p.mask[e]);
}

// The a-th active expert in ascending id order, or -1; called by one full wave.
__device__ __forceinline__ int nth_active_expert(const FfnArgs& p, int a) {
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

int num_cus();  // compute units of the current device (256 if it cannot be read)

// Launchers (argument checks are done by moe_expert_ffn).  Each returns MOE_OK or MOE_EHIP.
// `experts`: grid size in experts (an upper bound on the experts the row filter admits);
// `parts`: 1 = gate/up kernel, 2 = down kernel, 3 = both.
int launch_ffn_gemv(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts,
                    int parts);
// `rounds` > 0: at most that many full rounds of resident workgroups, each looping over
// (expert, row block) items; 0: one workgroup per item.
int launch_ffn_dot(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts, int parts,
                   int rounds = 0);
bool ffn_dot_supported(int d, int f);  // row lengths the dot-product path handles
// MXFP4 weights (codes expanded in registers, products on the matrix cores)
int launch_ffn_mx(const FfnArgs& p, int y_dtype, hipStream_t stream, int experts);
bool ffn_mx_supported(int d, int f);  // shapes the weight-streaming MXFP4 kernels handle
// `experts` > 0: at most that many experts pass the row filter (bounds the grid).
int launch_ffn_mx_gemm(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts = 0);
bool ffn_gemm_supported(long long T, int k, int d, int f);
int launch_ffn_gemm(const FfnArgs& p, int y_dtype, hipStream_t stream);

}  // namespace moe
