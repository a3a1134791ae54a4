// Grouping tokens by expert: histogram, exclusive scan and a stable permutation.
//
// The T*k flat assignments a = t*k + j are counting-sorted by expert id.  The
// order inside an expert is the stable (t, j) order, so results are
// deterministic: LDS atomics only count, they never decide a position.
//
// Work is cut into chunks of kChunk assignments, one workgroup (4 waves) per
// chunk and kChunk/4 consecutive assignments per wave:
//   hist  : per-chunk expert counts (LDS atomics) -> ws[chunk][E]
//   scan  : one workgroup; counts, offsets, and for each (chunk, expert) the
//           first output position of that chunk's items -> ws (in place)
//   rank  : per-wave counts of the chunk give each wave its base per expert;
//           inside a wave, 64 items at a time, an item's rank among equal ids
//           comes from ballots over the id bits (equal-id lane mask) and a
//           popcount of the lower lanes; the last lane of each id group
//           advances the wave's running base.
// When everything fits one chunk (decode), a single fused launch does it all; for a
// handful of tokens moe_route_permute routes and groups in one launch (route_group_tiny).
#include "common.h"
#include "route_dev.h"

using namespace moe;

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;           // assignments per workgroup
constexpr int kPerWave = kChunk / 4;   // 256 per wave, 4 steps of 64
constexpr int kRoutePermuteMaxT = 16;  // tokens routed inside the fused launch (2 per wave)
constexpr int kTinyThreads = 512;      // its workgroup: 8 waves

__device__ __forceinline__ int id_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// Exclusive scan over v[0..n) (n <= 1024) held one per thread of a 1024-thread
// block, or four per thread of a 256-thread block; returns the exclusive prefix
// of this thread's value and the total through *total (LDS).
template <int NT>
__device__ int block_exclusive_scan(int v, int* s_wave, int* s_total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int c = s_wave[w];
      s_wave[w] = run;
      run += c;
    }
    *s_total = run;
  }
  __syncthreads();
  return s_wave[wave] + x - v;
}

__global__ __launch_bounds__(kThreads) void permute_hist(const int32_t* __restrict__ ids, int A,
                                                         int E, int32_t* __restrict__ ws,
                                                         int32_t* status) {
  __shared__ int h[kMaxE];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  bool bad = false;
#pragma unroll
  for (int q = 0; q < kChunk / kThreads; ++q) {
    const int a = base + q * kThreads + threadIdx.x;
    if (a < A) {
      const int id = ids[a];
      if (id >= 0 && id < E) atomicAdd(&h[id], 1);
      else bad = true;
    }
  }
  if (bad) set_status(status, MOE_ERANGE);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) ws[(size_t)blockIdx.x * E + e] = h[e];
}

// One 1024-thread workgroup.  In: ws[b][e] = count of expert e in chunk b.
// Out: counts, offsets, ws[b][e] = first position of chunk b's items of e.
__global__ __launch_bounds__(1024) void permute_scan(int nchunk, int E, int32_t* __restrict__ ws,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int s_wave[16];
  __shared__ int s_total;
  constexpr int kU = 8;  // chunk counts in flight per thread (independent loads)
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nchunk; b0 += kU) {
      int c[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) c[q] = b0 + q < nchunk ? ws[(size_t)(b0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        if (b0 + q < nchunk) ws[(size_t)(b0 + q) * E + e] = run;
        run += c[q];
      }
    }
  }
  const int off = block_exclusive_scan<1024>(e < E ? run : 0, s_wave, &s_total);
  if (e < E) {
    counts[e] = run;
    offsets[e] = off;
    for (int b0 = 0; b0 < nchunk; b0 += kU) {
      int c[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) c[q] = b0 + q < nchunk ? ws[(size_t)(b0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < kU; ++q)
        if (b0 + q < nchunk) ws[(size_t)(b0 + q) * E + e] = c[q] + off;
    }
  }
  if (e == 0) offsets[E] = s_total;
}

// Per chunk: stable ranks and scatter.  FUSED: single chunk, computes counts
// and offsets itself (ws unused).
template <bool FUSED>
__device__ __forceinline__ void permute_block(const int32_t* __restrict__ ids, int A, int E,
                                              const int32_t* __restrict__ ws,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int32_t* status) {
  __shared__ int wb[4][kMaxE];
  __shared__ int s_wave[4];
  __shared__ int s_total;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    wb[0][e] = 0; wb[1][e] = 0; wb[2][e] = 0; wb[3][e] = 0;
  }
  __syncthreads();
  const int base = blockIdx.x * kChunk + wave * kPerWave;
  int myid[kPerWave / 64];
  bool bad = false;
#pragma unroll
  for (int s = 0; s < kPerWave / 64; ++s) {
    const int a = base + s * 64 + lane;
    int id = -1;
    if (a < A) {
      id = ids[a];
      if (id < 0 || id >= E) { bad = true; id = -1; }
    }
    myid[s] = id;
    if (id >= 0) atomicAdd(&wb[wave][id], 1);
  }
  if (bad) set_status(status, MOE_ERANGE);
  __syncthreads();
  if (FUSED) {
    // counts and offsets from the per-wave counts; E <= 1024 = 4 experts per thread.
    int c[4], tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = threadIdx.x * 4 + q;
      c[q] = e < E ? wb[0][e] + wb[1][e] + wb[2][e] + wb[3][e] : 0;
      tot += c[q];
    }
    int run = block_exclusive_scan<kThreads>(tot, s_wave, &s_total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = threadIdx.x * 4 + q;
      if (e < E) {
        counts[e] = c[q];
        offsets[e] = run;
        int r = run;
        for (int w = 0; w < 4; ++w) {
          const int cw = wb[w][e];
          wb[w][e] = r;
          r += cw;
        }
      }
      run += c[q];
    }
    if (threadIdx.x == 0) offsets[E] = s_total;
  } else {
    for (int e = threadIdx.x; e < E; e += kThreads) {
      int r = ws[(size_t)blockIdx.x * E + e];
      for (int w = 0; w < 4; ++w) {
        const int cw = wb[w][e];
        wb[w][e] = r;
        r += cw;
      }
    }
  }
  __syncthreads();
  const int nb = id_bits(E);
#pragma unroll
  for (int s = 0; s < kPerWave / 64; ++s) {
    const int a = base + s * 64 + lane;
    const int id = myid[s];
    const bool valid = id >= 0;
    unsigned long long eq = __ballot(valid);
    for (int b = 0; b < nb; ++b) {
      const bool bit = valid && ((id >> b) & 1);
      const unsigned long long m = __ballot(bit);
      eq &= bit ? m : ~m;
    }
    if (valid) {
      const int p = wb[wave][id] + __popcll(eq & lanemask_lt(lane));
      perm[p] = a;
      inv[a] = p;
      if ((eq >> lane) == 1ull) wb[wave][id] += __popcll(eq);
    }
  }
}

template <bool FUSED>
__global__ __launch_bounds__(kThreads) void permute_rank(const int32_t* __restrict__ ids, int A,
                                                         int E, const int32_t* __restrict__ ws,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv,
                                                         int32_t* status) {
  permute_block<FUSED>(ids, A, E, ws, counts, offsets, perm, inv, status);
}

// Routing and grouping of a few tokens (T <= 16, so T*k <= 256) in one workgroup of 8
// waves: wave w routes tokens w and w + 8 (route_dev.h), keeping the ids in LDS as well;
// then assignment a's position is its stable rank, the number of assignments b with
// (id_b, b) < (id_a, a), and expert e's count and offset are the numbers of ids equal to and
// below e, each counted straight from the ids in LDS (every wave reads the same id at once,
// a broadcast).  With so few assignments this is shorter than the histogram, scan and
// ballot ranking of permute_block, which pays barriers and shuffle chains whatever the size.
template <int NPL>
__global__ __launch_bounds__(kTinyThreads) void route_group_tiny(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t s_ids[kRoutePermuteMaxT * kMaxK];
  const int wave = threadIdx.x >> 6;
  unsigned long long key[2][NPL];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = wave + 8 * i;
    if (t < T) route_keys<NPL>(logits + (size_t)t * E, E, key[i]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = wave + 8 * i;
    if (t < T) route_pick<NPL>(key[i], k, ids + (size_t)t * k, w + (size_t)t * k, s_ids + t * k);
  }
  __syncthreads();
  const int A = T * k;
  for (int a = threadIdx.x; a < A; a += kTinyThreads) {
    const int id = s_ids[a];
    int r = 0;
    for (int b = 0; b < A; ++b) {
      const int ib = s_ids[b];
      r += (ib < id) | ((ib == id) & (b < a));
    }
    perm[r] = a;
    inv[a] = r;
  }
  for (int e = threadIdx.x; e <= E; e += kTinyThreads) {
    int c = 0, below = 0;
    for (int b = 0; b < A; ++b) {
      const int ib = s_ids[b];
      c += ib == e;
      below += ib < e;
    }
    if (e < E) counts[e] = c;
    offsets[e] = below;  // offsets[E] = A
  }
}

}  // namespace

extern "C" size_t moe_permute_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return 256;
  const long long A = (long long)T * k;
  const long long nchunk = (A + kChunk - 1) / kChunk;
  return (size_t)(((nchunk * E * 4) + 255) / 256 * 256);
}

extern "C" int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                           size_t ws_bytes, int32_t* status, hipStream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || k <= 0 || k > kMaxK || k > E) return MOE_EINVAL;
  if ((long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (!counts || !offsets) return MOE_EINVAL;
  const int A = T * k;
  if (A > 0 && (!topk_ids || !perm || !inv)) return MOE_EINVAL;
  const int nchunk = (A + kChunk - 1) / kChunk;
  if (nchunk <= 1) {
    hipLaunchKernelGGL(permute_rank<true>, dim3(1), dim3(kThreads), 0, stream, topk_ids, A, E,
                       (const int32_t*)nullptr, counts, offsets, perm, inv, status);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  if (!ws || ws_bytes < moe_permute_workspace_bytes(T, k, E)) return MOE_EINVAL;
  int32_t* w = (int32_t*)ws;
  hipLaunchKernelGGL(permute_hist, dim3(nchunk), dim3(kThreads), 0, stream, topk_ids, A, E, w, status);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(1024), 0, stream, nchunk, E, w, counts, offsets);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(permute_rank<false>, dim3(nchunk), dim3(kThreads), 0, stream, topk_ids, A, E,
                     (const int32_t*)w, counts, offsets, perm, inv, status);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int moe_route_permute(const float* logits, int T, int E, int k, int32_t* topk_ids,
                                 float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                                 int32_t* inv, void* ws, size_t ws_bytes, int32_t* status,
                                 hipStream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || k <= 0 || k > kMaxK || k > E) return MOE_EINVAL;
  if ((long long)T * E >= (1ll << 31) || (long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (!counts || !offsets) return MOE_EINVAL;
  if (T > kRoutePermuteMaxT) {
    int rc = moe_route(logits, T, E, k, topk_ids, topk_w, stream);
    if (rc == MOE_OK) rc = moe_permute(topk_ids, T, k, E, counts, offsets, perm, inv, ws, ws_bytes, status, stream);
    return rc;
  }
  if (T > 0 && (!logits || !topk_ids || !topk_w || !perm || !inv)) return MOE_EINVAL;
  const dim3 g(1), b(kTinyThreads);
  if (E <= 64)
    hipLaunchKernelGGL(route_group_tiny<1>, g, b, 0, stream, logits, T, E, k, topk_ids, topk_w, counts, offsets, perm, inv);
  else if (E <= 128)
    hipLaunchKernelGGL(route_group_tiny<2>, g, b, 0, stream, logits, T, E, k, topk_ids, topk_w, counts, offsets, perm, inv);
  else if (E <= 256)
    hipLaunchKernelGGL(route_group_tiny<4>, g, b, 0, stream, logits, T, E, k, topk_ids, topk_w, counts, offsets, perm, inv);
  else if (E <= 512)
    hipLaunchKernelGGL(route_group_tiny<8>, g, b, 0, stream, logits, T, E, k, topk_ids, topk_w, counts, offsets, perm, inv);
  else
    hipLaunchKernelGGL(route_group_tiny<16>, g, b, 0, stream, logits, T, E, k, topk_ids, topk_w, counts, offsets, perm, inv);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
