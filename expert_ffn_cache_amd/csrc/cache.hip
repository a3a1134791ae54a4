// Global LRU cache of whole (layer, expert) entries, miss fills and
// double-buffered layer streaming.
//
// FreeToken pages: decode keeps a shared LRU expert cache across layers and
// tokens, so recent routing decides what stays resident (llama page, "Official
// project overview"; RTX-4090 page, "How the MoE memory hierarchy works");
// entries are complete (layer, expert) pairs under one logical mapping (same
// RTX-4090 section); misses are moved over PCIe into the GPU cache (benchmark
// page, runtime-tier table); prefill moves the next layer's experts while the
// current layer computes (benchmark page, "How FreeToken serves large MoE
// models"); control data stays on the device so routing-dependent decisions
// remain graph-compatible (benchmark page, feature cards).  Misses are filled either by
// host-issued copies of the records read back after the lookup, or entirely on the device
// by a copy kernel that reads the pinned pool over PCIe, so a decode step including its
// misses can be captured and replayed as one graph.
//
// The lookup runs as one 1024-thread workgroup, entirely on device tables:
//   requested-set flags in LDS -> |U| (barrier count) -> capacity check ->
//   hit detection through slot_of -> (stamp << 13 | slot) keys of all slots in
//   LDS with hit slots pushed to the end -> bitonic sort -> the i-th miss
//   (ascending id, block scan) takes the i-th smallest key -> table updates,
//   fill records, counters, clock.
#include <algorithm>

#include "common.h"

using namespace moe;

namespace {

constexpr int kCacheThreads = 1024;
constexpr int kMaxSlots = 4096;  // keys of all slots live in LDS (32 KB)
constexpr int kSlotBits = 13;

__global__ __launch_bounds__(256) void cache_init_kernel(moe_cache_t c) {
  const long long nkeys = (long long)c.L * c.E;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < nkeys; i += stride)
    c.slot_of[i] = -1;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < c.S; i += stride) {
    c.key_of[i] = -1;
    c.stamp[i] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x < 4) c.stats[threadIdx.x] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *c.clock = 0;
    *c.status = 0;
  }
}

// Ascending bitonic sort of keys[0 .. npow) in LDS by the whole workgroup (npow a power of
// two); ends with a barrier.
__device__ void bitonic_sort_lds(unsigned long long* keys, int npow) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < (npow >> 1); i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const unsigned long long x = keys[lo], y = keys[hi];
        if ((x > y) == asc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
    }
  }
  __syncthreads();
}

// SPLIT: only the first q* misses (ascending id) are filled, q* minimising
// max(q * host_mbps, (m - q) * pcie_mbps) over q = 0..m with ties to the larger q (the two
// paths' times for m misses of equal size, in integers); the others are left to the host
// (host_mask = 1), take no slot and are not inserted.
template <bool SPLIT>
__global__ __launch_bounds__(kCacheThreads) void lru_lookup_update(moe_cache_t c, int layer,
                                                                   const int32_t* __restrict__ ids,
                                                                   int A, int32_t* __restrict__ expert_slot,
                                                                   moe_fill_t* __restrict__ fills,
                                                                   int32_t* __restrict__ n_fills,
                                                                   int pcie_mbps, int host_mbps,
                                                                   uint8_t* __restrict__ host_mask) {
  __shared__ unsigned long long keys[kMaxSlots];
  __shared__ int req[kMaxE];       // 1 = requested
  __shared__ int miss_list[kMaxE];
  __shared__ int s_wave[16];
  __shared__ int s_err;
  __shared__ int s_q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = c.E, S = c.S;
  const long long t = *c.clock + 1;  // read before any thread can update the clock
  if (tid < E) req[tid] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  for (int a = tid; a < A; a += kCacheThreads) {
    const int id = ids[a];
    if (id >= 0 && id < E) req[id] = 1;
    else s_err = 1;
  }
  __syncthreads();
  const bool want = tid < E && req[tid];
  int slot = -1;
  if (want) {
    slot = c.slot_of[(size_t)layer * E + tid];
    if (slot >= S) s_err = 1;  // corrupted table
  }
  const int nU = __syncthreads_count(want);
  if (s_err || nU > S) {
    if (tid == 0) {
      set_status(c.status, s_err ? MOE_ERANGE : MOE_ECAPACITY);
      *n_fills = 0;
    }
    return;
  }
  const bool hit = want && slot >= 0;
  const bool miss = want && slot < 0;
  // keys of every slot; slots hit in this call sort after all candidates
  int npow = 64;
  while (npow < S) npow <<= 1;
  for (int s = tid; s < npow; s += kCacheThreads)
    keys[s] = s < S ? ((unsigned long long)c.stamp[s] << kSlotBits) | (unsigned)s : ~0ull;
  __syncthreads();
  if (hit) keys[slot] = ~0ull;
  // miss ranks in ascending expert id (one expert per thread)
  const unsigned long long mb = __ballot(miss);
  if (lane == 0) s_wave[wave] = __popcll(mb);
  __syncthreads();
  int before = 0, nmiss = 0;
  for (int w = 0; w < kCacheThreads / 64; ++w) {
    before += w < wave ? s_wave[w] : 0;
    nmiss += s_wave[w];
  }
  const int my_rank = before + __popcll(mb & lanemask_lt(lane));
  if (miss) miss_list[my_rank] = tid;
  int q = nmiss;  // misses filled in this call
  if (SPLIT) {
    if (tid == 0) {
      long long best_t = -1;
      int best_q = 0;
      for (int qq = 0; qq <= nmiss; ++qq) {
        const long long tt = max((long long)qq * host_mbps, (long long)(nmiss - qq) * pcie_mbps);
        if (best_t < 0 || tt <= best_t) {
          best_q = qq;
          best_t = tt;
        }
      }
      s_q = best_q;
    }
    __syncthreads();
    q = s_q;
  }
  const bool to_host = miss && my_rank >= q;
  bitonic_sort_lds(keys, npow);
  if (tid < q) {
    const int s = (int)(keys[tid] & ((1u << kSlotBits) - 1));
    const int e = miss_list[tid];
    const int old = c.key_of[s];
    const int key = layer * E + e;
    if (old >= 0) c.slot_of[old] = -1;
    c.key_of[s] = key;
    c.slot_of[key] = s;
    c.stamp[s] = t;
    fills[tid] = moe_fill_t{s, layer, e, old};
    expert_slot[e] = s;
  }
  if (tid < E) {
    if (hit) {
      c.stamp[slot] = t;
      expert_slot[tid] = slot;
    } else if (!miss || to_host) {
      expert_slot[tid] = -1;
    }
    if (SPLIT) host_mask[tid] = to_host;
  }
  if (tid == 0) {
    *c.clock = t;
    *n_fills = q;
    c.stats[0] += nU;
    c.stats[1] += nU - nmiss;
    c.stats[2] += nmiss;
    c.stats[3] += (long long)q * (long long)c.entry_bytes;
  }
}

// Device-driven miss fills: the record count and the records are read on the device (as the
// lookup left them), and each missed entry is copied from the pinned host pool, which the
// GPU reads directly over PCIe, into its arena slot.  The grid is fixed, so the launch does
// not depend on the count.  64 workgroups with 8 independent 16-byte loads per thread
// (2 MB in flight) keep the host link saturated while leaving most CUs to other work.
constexpr int kFillBlocks = 64, kFillThreads = 256, kFillUnroll = 8;

__global__ __launch_bounds__(kFillThreads) void fill_from_pool(moe_cache_t c,
                                                               const moe_fill_t* __restrict__ fills,
                                                               const int32_t* __restrict__ n_fills,
                                                               int max_fills) {
  const int n = *n_fills;
  if (n < 0 || n > max_fills) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(c.status, MOE_ERANGE);
    return;
  }
  const size_t n16 = c.entry_bytes / 16;
  constexpr size_t per_iter = (size_t)kFillThreads * kFillUnroll;
  const size_t iters = (n16 + per_iter - 1) / per_iter;
  const size_t total = (size_t)n * iters;
  const u32x4* pool = (const u32x4*)c.host_pool;
  u32x4* arena = (u32x4*)c.arena;
  for (size_t w = blockIdx.x; w < total; w += gridDim.x) {
    const int i = (int)(w / iters);
    const size_t it = w - (size_t)i * iters;
    const moe_fill_t f = fills[i];
    if (f.slot < 0 || f.slot >= c.S || f.layer < 0 || f.layer >= c.L || f.expert < 0 ||
        f.expert >= c.E || (long long)f.layer * c.E + f.expert >= c.pool_entries) {
      if (it == 0 && threadIdx.x == 0) set_status(c.status, MOE_ERANGE);
      continue;
    }
    const u32x4* src = pool + ((size_t)f.layer * c.E + f.expert) * n16;
    u32x4* dst = arena + (size_t)f.slot * n16;
    const size_t base = it * per_iter + threadIdx.x;
    u32x4 v[kFillUnroll];
#pragma unroll
    for (int q = 0; q < kFillUnroll; ++q) {
      const size_t j = base + (size_t)q * kFillThreads;
      if (j < n16) v[q] = src[j];
    }
#pragma unroll
    for (int q = 0; q < kFillUnroll; ++q) {
      const size_t j = base + (size_t)q * kFillThreads;
      if (j < n16) dst[j] = v[q];
    }
  }
}

// Hit / miss masks of the last lookup: requested experts (expert_slot >= 0) split by whether
// a fill record names them.  One workgroup; E <= 1024.
__global__ __launch_bounds__(kMaxE) void fill_masks_kernel(const int32_t* __restrict__ expert_slot,
                                                           const moe_fill_t* __restrict__ fills,
                                                           const int32_t* __restrict__ n_fills, int E,
                                                           uint8_t* __restrict__ hit_mask,
                                                           uint8_t* __restrict__ miss_mask,
                                                           int32_t* __restrict__ status) {
  __shared__ uint8_t missed[kMaxE];
  const int tid = threadIdx.x;
  if (tid < E) missed[tid] = 0;
  __syncthreads();
  const int n = *n_fills;
  if (n < 0 || n > E) {
    if (tid == 0) set_status(status, MOE_ERANGE);
    if (tid < E) hit_mask[tid] = miss_mask[tid] = 0;
    return;
  }
  if (tid < n) {
    const int e = fills[tid].expert;
    if (e >= 0 && e < E) missed[e] = 1;
    else set_status(status, MOE_ERANGE);
  }
  __syncthreads();
  if (tid < E) {
    const bool req = expert_slot[tid] >= 0;
    hit_mask[tid] = req && !missed[tid];
    miss_mask[tid] = req && missed[tid];
  }
}

// Elastic resize.  Tables: the survivors are the min(S_new, resident) entries with the
// largest stamps (ties to the lower old slot), found by sorting (2^50 - 1 - stamp, slot)
// keys; they go to new slots 0..n-1 in ascending old-slot order (block scan of survivor
// flags) with their stamps; clock and counters carry over.  The new tables were cleared by
// cache_init_kernel just before.  One workgroup; old S <= 4096.
constexpr long long kStampLimit = 1ll << 50;  // clock values stay far below this

__global__ __launch_bounds__(kCacheThreads) void resize_tables(moe_cache_t o, moe_cache_t n) {
  __shared__ unsigned long long keys[kMaxSlots];
  __shared__ int keep[kMaxSlots];
  __shared__ int s_wave[kCacheThreads / 64];
  __shared__ int s_nres;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = o.S;
  int npow = 64;
  while (npow < S) npow <<= 1;
  if (tid == 0) s_nres = 0;
  for (int s = tid; s < npow; s += kCacheThreads) {
    const bool used = s < S && o.key_of[s] >= 0;
    keys[s] = used ? ((unsigned long long)(kStampLimit - 1 - o.stamp[s]) << kSlotBits) | (unsigned)s
                   : ~0ull;
    if (s < S) keep[s] = 0;
  }
  bitonic_sort_lds(keys, npow);
  // resident count = position of the first empty key (all occupied keys sort before it)
  for (int i = tid; i < npow; i += kCacheThreads)
    if (keys[i] != ~0ull && (i + 1 == npow || keys[i + 1] == ~0ull)) s_nres = i + 1;
  __syncthreads();
  const int nkeep = min(s_nres, n.S);
  for (int i = tid; i < nkeep; i += kCacheThreads) keep[(int)(keys[i] & ((1u << kSlotBits) - 1))] = 1;
  __syncthreads();
  // new index of each kept slot = number of kept slots before it (4 slots per thread)
  int c = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s = tid * 4 + q;
    c += s < S ? keep[s] : 0;
  }
  int x = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  int j = base + x - c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s = tid * 4 + q;
    if (s < S && keep[s]) {
      const int key = o.key_of[s];
      n.key_of[j] = key;
      n.stamp[j] = o.stamp[s];
      n.slot_of[key] = j;
      ++j;
    }
  }
  if (tid == 0) {
    *n.clock = *o.clock;
    for (int i = 0; i < 4; ++i) n.stats[i] = o.stats[i];
  }
}

// Copies the arena entry of every occupied new slot from its old slot.
__global__ __launch_bounds__(kFillThreads) void resize_copy(moe_cache_t o, moe_cache_t n) {
  const size_t n16 = n.entry_bytes / 16;
  constexpr size_t per_iter = (size_t)kFillThreads * kFillUnroll;
  const size_t iters = (n16 + per_iter - 1) / per_iter;
  const size_t total = (size_t)n.S * iters;
  const u32x4* src_arena = (const u32x4*)o.arena;
  u32x4* dst_arena = (u32x4*)n.arena;
  for (size_t w = blockIdx.x; w < total; w += gridDim.x) {
    const int j = (int)(w / iters);
    const size_t it = w - (size_t)j * iters;
    const int key = n.key_of[j];
    if (key < 0) continue;
    const int s = o.slot_of[key];
    const u32x4* src = src_arena + (size_t)s * n16;
    u32x4* dst = dst_arena + (size_t)j * n16;
    const size_t b = it * per_iter + threadIdx.x;
    u32x4 v[kFillUnroll];
#pragma unroll
    for (int q = 0; q < kFillUnroll; ++q) {
      const size_t i = b + (size_t)q * kFillThreads;
      if (i < n16) v[q] = src[i];
    }
#pragma unroll
    for (int q = 0; q < kFillUnroll; ++q) {
      const size_t i = b + (size_t)q * kFillThreads;
      if (i < n16) dst[i] = v[q];
    }
  }
}

bool cache_ok(const moe_cache_t* c) {
  return c && c->L > 0 && c->E > 0 && c->E <= kMaxE && c->S > 0 && c->S <= kMaxSlots &&
         (long long)c->L * c->E < (1ll << 31) && c->entry_bytes > 0 && c->slot_of && c->key_of &&
         c->stamp && c->clock && c->stats && c->status;
}

}  // namespace

extern "C" int cache_init(const moe_cache_t* cache, hipStream_t stream) {
  if (!cache_ok(cache)) return MOE_EINVAL;
  const long long n = std::max<long long>((long long)cache->L * cache->E, cache->S);
  const int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(cache_init_kernel, dim3(blocks), dim3(256), 0, stream, *cache);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int cache_lookup_update(const moe_cache_t* cache, int layer, const int32_t* topk_ids,
                                   int T, int k, int32_t* expert_slot, moe_fill_t* fills,
                                   int32_t* n_fills, hipStream_t stream) {
  if (!cache_ok(cache)) return MOE_EINVAL;
  if (layer < 0 || layer >= cache->L) return MOE_ERANGE;
  if (T < 0 || k <= 0 || k > kMaxK || k > cache->E) return MOE_EINVAL;
  if ((long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (!expert_slot || !fills || !n_fills || (T > 0 && !topk_ids)) return MOE_EINVAL;
  hipLaunchKernelGGL(lru_lookup_update<false>, dim3(1), dim3(kCacheThreads), 0, stream, *cache,
                     layer, topk_ids, T * k, expert_slot, fills, n_fills, 0, 0, (uint8_t*)nullptr);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int cache_lookup_update_split(const moe_cache_t* cache, int layer,
                                         const int32_t* topk_ids, int T, int k, int pcie_mbps,
                                         int host_mbps, int32_t* expert_slot, moe_fill_t* fills,
                                         int32_t* n_fills, uint8_t* host_mask, hipStream_t stream) {
  if (!cache_ok(cache)) return MOE_EINVAL;
  if (layer < 0 || layer >= cache->L) return MOE_ERANGE;
  if (T < 0 || k <= 0 || k > kMaxK || k > cache->E) return MOE_EINVAL;
  if ((long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (pcie_mbps < 0 || host_mbps < 0 || (long long)pcie_mbps + host_mbps == 0) return MOE_EINVAL;
  if (!expert_slot || !fills || !n_fills || !host_mask || (T > 0 && !topk_ids)) return MOE_EINVAL;
  hipLaunchKernelGGL(lru_lookup_update<true>, dim3(1), dim3(kCacheThreads), 0, stream, *cache,
                     layer, topk_ids, T * k, expert_slot, fills, n_fills, pcie_mbps, host_mbps,
                     host_mask);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int cache_fill(const moe_cache_t* cache, const moe_fill_t* fills_host, int n_fills,
                          hipStream_t copy_stream) {
  if (!cache || !cache->arena || !cache->host_pool || cache->S <= 0 || cache->L <= 0 ||
      cache->E <= 0 || cache->entry_bytes == 0)
    return MOE_EINVAL;
  if (n_fills < 0 || (n_fills > 0 && !fills_host)) return MOE_EINVAL;
  for (int i = 0; i < n_fills; ++i) {
    const moe_fill_t& f = fills_host[i];
    if (f.slot < 0 || f.slot >= cache->S || f.layer < 0 || f.layer >= cache->L || f.expert < 0 ||
        f.expert >= cache->E || (long long)f.layer * cache->E + f.expert >= cache->pool_entries)
      return MOE_ERANGE;
  }
  const size_t eb = cache->entry_bytes;
  const char* pool = (const char*)cache->host_pool;
  char* arena = (char*)cache->arena;
  int i = 0;
  while (i < n_fills) {
    const long long src0 = (long long)fills_host[i].layer * cache->E + fills_host[i].expert;
    const int dst0 = fills_host[i].slot;
    int run = 1;
    while (i + run < n_fills) {
      const moe_fill_t& g = fills_host[i + run];
      if ((long long)g.layer * cache->E + g.expert != src0 + run || g.slot != dst0 + run) break;
      ++run;
    }
    MOE_HIP_CHECK(hipMemcpyAsync(arena + (size_t)dst0 * eb, pool + (size_t)src0 * eb,
                                 (size_t)run * eb, hipMemcpyHostToDevice, copy_stream));
    i += run;
  }
  return MOE_OK;
}

extern "C" int cache_fill_device(const moe_cache_t* cache, const moe_fill_t* fills,
                                 const int32_t* n_fills, int max_fills, hipStream_t stream) {
  if (!cache || !cache->arena || !cache->host_pool || !cache->status || cache->S <= 0 ||
      cache->L <= 0 || cache->E <= 0 || (long long)cache->L * cache->E >= (1ll << 31))
    return MOE_EINVAL;
  if (cache->entry_bytes == 0 || cache->entry_bytes % 16 != 0 || !moe_aligned16(cache->arena) ||
      !moe_aligned16(cache->host_pool))
    return MOE_EINVAL;
  if (!fills || !n_fills || max_fills < 0) return MOE_EINVAL;
  if (max_fills == 0) return MOE_OK;
  hipLaunchKernelGGL(fill_from_pool, dim3(kFillBlocks), dim3(kFillThreads), 0, stream, *cache,
                     fills, n_fills, max_fills);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int cache_fill_masks(const int32_t* expert_slot, const moe_fill_t* fills,
                                const int32_t* n_fills, int E, uint8_t* hit_mask,
                                uint8_t* miss_mask, int32_t* status, hipStream_t stream) {
  if (E <= 0 || E > kMaxE) return MOE_EINVAL;
  if (!expert_slot || !fills || !n_fills || !hit_mask || !miss_mask) return MOE_EINVAL;
  hipLaunchKernelGGL(fill_masks_kernel, dim3(1), dim3(kMaxE), 0, stream, expert_slot, fills,
                     n_fills, E, hit_mask, miss_mask, status);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int cache_resize(const moe_cache_t* old_cache, const moe_cache_t* new_cache,
                            hipStream_t stream) {
  if (!cache_ok(old_cache) || !cache_ok(new_cache)) return MOE_EINVAL;
  const moe_cache_t& o = *old_cache;
  const moe_cache_t& n = *new_cache;
  if (o.L != n.L || o.E != n.E || o.entry_bytes != n.entry_bytes) return MOE_EINVAL;
  if (!o.arena || !n.arena || o.entry_bytes % 16 != 0 || !moe_aligned16(o.arena) ||
      !moe_aligned16(n.arena))
    return MOE_EINVAL;
  const uintptr_t oa = (uintptr_t)o.arena, na = (uintptr_t)n.arena;
  if (oa < na + (uintptr_t)n.S * n.entry_bytes && na < oa + (uintptr_t)o.S * o.entry_bytes)
    return MOE_EINVAL;  // arenas overlap
  if (o.slot_of == n.slot_of || o.key_of == n.key_of || o.stamp == n.stamp) return MOE_EINVAL;
  const long long nt = std::max<long long>((long long)n.L * n.E, n.S);
  const int blocks = (int)std::min<long long>((nt + 255) / 256, 4096);
  hipLaunchKernelGGL(cache_init_kernel, dim3(blocks), dim3(256), 0, stream, n);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(resize_tables, dim3(1), dim3(kCacheThreads), 0, stream, o, n);
  MOE_LAUNCH_CHECK();
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  hipLaunchKernelGGL(resize_copy, dim3(4 * cus), dim3(kFillThreads), 0, stream, o, n);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int layer_stream_prefetch(const void* host_src, void* dst, size_t bytes, int n_chunks,
                                     hipStream_t copy_stream, hipEvent_t wait_before,
                                     hipEvent_t done) {
  if (!host_src || !dst || n_chunks <= 0) return MOE_EINVAL;
  if (wait_before) MOE_HIP_CHECK(hipStreamWaitEvent(copy_stream, wait_before, 0));
  const size_t chunk = (bytes + (size_t)n_chunks - 1) / (size_t)n_chunks;
  for (size_t off = 0; off < bytes; off += chunk) {
    const size_t n = std::min(chunk, bytes - off);
    MOE_HIP_CHECK(hipMemcpyAsync((char*)dst + off, (const char*)host_src + off, n,
                                 hipMemcpyHostToDevice, copy_stream));
  }
  if (done) MOE_HIP_CHECK(hipEventRecord(done, copy_stream));
  return MOE_OK;
}
