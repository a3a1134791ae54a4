// One token through a routed-MoE layer in a single launch: top-k softmax routing, the k
// selected experts' SwiGLU FFNs and the gate-weighted combine (bf16 or MXFP4 weights).
//
// A one-token decode step reads k whole experts (302 MB at k = 6, d = 4096, f = 2048) and
// does next to no arithmetic on them, so its time is the weight stream plus whatever stops
// that stream.  Run as separate launches (routing, gate/up, down, combine) it stops at every
// boundary: each launch pays its ramp and its tail, and the routing and combine launches move
// almost no bytes at all.  Here one grid of G workgroups, all resident at once, walks a fixed
// list of work items (workgroup b takes items b, b + G, b + 2G, ...):
//   gate/up item (j, b): the units u of block b of the j-th selected expert,
//       h_j[u] = SiLU(x . W_gate_j[u]) * (x . W_up_j[u])      (fp32 sums, h rounded to bf16)
//   down item b: the output channels o of block b,
//       out[o] = sum_j w_j * (h_j . W_down_j[o])               (j ascending, fp32)
// and every workgroup routes the token itself first (the logits are only 4E bytes), so no
// launch waits for another.  Gate/up items come first in the list.  A down item needs all of
// h, so a workgroup's first down item issues its weight loads and only then waits, once per
// workgroup, until all of h is there; the weight stream runs on through the change of phase.
//
// Cross-workgroup traffic stays cheap on this chip: the eight L2 caches are not coherent
// with one another, and the fences that would make ordinary stores visible across them
// (write back or invalidate a whole L2) cost more than the layer when hundreds of workgroups
// issue them, as does a device-scope atomic per work item on one counter (each is
// serialised at the memory side), and so does waiting for stores to be acknowledged before
// raising a flag.  So every h value carries its own flag: each UPW-unit group of h is one
// 8-byte device-coherent store of the values and the launch's epoch (single-copy atomic),
// and a reader loads the entries device-coherently and takes them once every epoch
// matches.  The epoch word at the head of the workspace is one less than the launch's
// epoch; workgroup 0 advances it once it has seen every entry of this launch (so every
// workgroup has read it), and nothing is reset between calls or graph replays.  The wait
// ends once every workgroup has run its gate/up items, which needs the G workgroups to be
// resident together: G is within the occupancy bound for this kernel on an otherwise idle
// GPU.  The wait is bounded all the same (MOE_ETIMEOUT), so calls that share the GPU with
// another launch that never yields fail rather than hang.
//
// The dot products are those of the multi-token weight-streaming kernels (lane l takes the
// 16-byte chunks l, l + 64, ... of a row; packed bf16 products with fp32 accumulation; one
// cross-lane sum per row) in the same order, so `out` is bit-identical to routing, grouping,
// the expert FFN with fp32 outputs and the combine run as separate calls.
#include <algorithm>

#include "ffn_args.h"
#include "mx_dev.h"
#include "route_dev.h"
#include "wave.h"

using namespace moe;

namespace {

constexpr int kTokThreads = 256;     // four waves
constexpr int kTokDownCh = 4;        // output channels per down item, one per wave
constexpr size_t kTokHdrBytes = 256;  // the epoch word, then padding
constexpr unsigned kTokSpinLimit = 1u << 18;  // polls of h (well over a second)

struct TokArgs {
  const float* logits;  // [E] fp32, or nullptr: ids and weights are read from topk_ids / topk_w
  const uint16_t* x;    // [d] bf16
  int E, k, d, f;
  const int32_t* expert_slot;
  const char* arena;
  size_t stride;
  const int32_t* slot_key;
  int key_base;
  int32_t* topk_ids;
  float* topk_w;
  uint32_t* epoch_word;
  uint64_t* hent;  // h entries: UPW units of h (bf16, low half first) | launch epoch << 32
  float* out;     // [d] fp32
  int32_t* status;
  int n_gu, n_items;
};

// Device-coherent 32-bit accesses (relaxed atomics at device scope: served past the
// per-XCD L2 caches, so other XCDs see them without any cache maintenance).
__device__ __forceinline__ uint32_t coh_load(const uint32_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(uint32_t* a, uint32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t coh_load64(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store64(uint64_t* a, uint64_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// acc + a . b over 8 bf16 pairs, four packed products in element order (the pairs taken
// with shufflevector, as the multi-token kernels take them).
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
  const bf16x8 x = as_bf16x8(a), y = as_bf16x8(b);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                        __builtin_shufflevector(y, y, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                        __builtin_shufflevector(y, y, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                        __builtin_shufflevector(y, y, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                        __builtin_shufflevector(y, y, 6, 7), acc, false);
  return acc;
}

// Wave index as a scalar, so row addresses built from it stay in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* q) {
  const uint64_t v = (uint64_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// Byte offset of lane chunk i of a row of nck 16-byte chunks: chunk lane + 64 i, clamped to
// the last one (a lane past the row re-reads it and leaves it out of its sums), so that every
// load of a row is issued without a per-lane branch.
__device__ __forceinline__ uint32_t chunk_off(int i, int nck) {
  return (uint32_t)min((int)(threadIdx.x & 63) + 64 * i, nck - 1) * 16u;
}

__device__ __forceinline__ u32x4 ldrow(const void* row, uint32_t off) {
  return ldg16_nt((const char*)row + off);
}

// Lane chunk i of a row staged in LDS, or zeros for a lane past the row (a select, not a
// branch: every product below is taken by every lane, so no load is left pending on a path
// that skips it).
__device__ __forceinline__ u32x4 lds_chunk(const uint16_t* row, int i, int nck) {
  const u32x4 v = *(const u32x4*)((const char*)row + chunk_off(i, nck));
  const bool in = (int)(threadIdx.x & 63) + 64 * i < nck;
  return u32x4{in ? v[0] : 0u, in ? v[1] : 0u, in ? v[2] : 0u, in ? v[3] : 0u};
}

// Gate/up item: UPW units per wave of the a-th selected expert; lane 0 stores the wave's
// h values with the launch's epoch in one device-coherent 8-byte entry.
template <int NCHD, int UPW>
__device__ __forceinline__ void gateup_item(const TokArgs& p, const uint16_t* xs,
                                            const char* const* ent, int item, uint32_t epoch) {
  constexpr int UPB = 4 * UPW;
  const int nub = p.f / UPB;
  const int a = item / nub, ub = item - a * nub;
  const int wave = wave_id();
  const int d = p.d, nck = d >> 3;
  const char* e = uniform_ptr(ent[a]);
  const int u0 = ub * UPB + wave * UPW;
  u32x4 wg[UPW][NCHD], wu[UPW][NCHD];
  if (e) {
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
      const uint16_t* pg = (const uint16_t*)e + (size_t)(u0 + uu) * d;
      const uint16_t* pu = pg + (size_t)p.f * d;
#pragma unroll
      for (int i = 0; i < NCHD; ++i) {
        wg[uu][i] = ldrow(pg, chunk_off(i, nck));
        wu[uu][i] = ldrow(pu, chunk_off(i, nck));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of what follows
  if (!e) return;
  float g[UPW], u[UPW];
#pragma unroll
  for (int uu = 0; uu < UPW; ++uu) g[uu] = u[uu] = 0.f;
#pragma unroll
  for (int i = 0; i < NCHD; ++i) {
    const u32x4 xv = lds_chunk(xs, i, nck);
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
      g[uu] = dot8(xv, wg[uu][i], g[uu]);
      u[uu] = dot8(xv, wu[uu][i], u[uu]);
    }
  }
  uint16_t hv[UPW];
#pragma unroll
  for (int uu = 0; uu < UPW; ++uu) hv[uu] = f32_to_bf16(silu(wave_sum_f32(g[uu])) * wave_sum_f32(u[uu]));
  if ((threadIdx.x & 63) == 0) {
    uint32_t v = hv[0];
    if (UPW == 2) v |= (uint32_t)hv[UPW - 1] << 16;
    coh_store64(p.hent + ((size_t)a * p.f + u0) / UPW, (uint64_t)v | ((uint64_t)epoch << 32));
  }
}

// Stages all k rows of h in LDS once every entry carries this launch's epoch: each thread
// loads its entries (eight in flight at a time) and writes the values; the workgroup repeats
// until no thread found a stale entry.  Returns false on giving up.
template <int UPW>
__device__ __forceinline__ bool stage_h(const TokArgs& p, uint16_t* hs, uint32_t epoch) {
  const int n = p.k * p.f / UPW;
  for (unsigned polls = 0; polls < kTokSpinLimit; ++polls) {
    int stale = 0;
    for (int q0 = 0; q0 < n; q0 += 8 * kTokThreads) {
      uint64_t v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        v[r] = coh_load64(p.hent + min(q0 + r * kTokThreads + (int)threadIdx.x, n - 1));
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int q = q0 + r * kTokThreads + threadIdx.x;
        if (q < n) {
          stale |= (uint32_t)(v[r] >> 32) != epoch;
          if (UPW == 2) ((uint32_t*)hs)[q] = (uint32_t)v[r];
          else hs[q] = (uint16_t)v[r];
        }
      }
    }
    if (!__syncthreads_or(stale)) return true;
    __builtin_amdgcn_s_sleep(8);
  }
  return false;
}

template <int UPW>
__device__ __forceinline__ void wait_and_stage_h(const TokArgs& p, uint16_t* hs, uint32_t epoch) {
  if (!stage_h<UPW>(p, hs, epoch) && threadIdx.x == 0) set_status(p.status, MOE_ETIMEOUT);
}

// Entries of the selected experts j0 .. j0 + JG - 1 (nullptr past k or for a missing
// entry), in scalar registers.  The same pointers decide both which rows are loaded and
// which are multiplied, so no load is left pending on a path that skips its use.
template <int JG>
__device__ __forceinline__ void down_entries(const TokArgs& p, const char* const* ent, int j0,
                                             const char* (&e)[JG]) {
#pragma unroll
  for (int jj = 0; jj < JG; ++jj) e[jj] = j0 + jj < p.k ? uniform_ptr(ent[j0 + jj]) : nullptr;
}

// Down rows of output channel o of those experts into registers.
template <int NCHF, int JG>
__device__ __forceinline__ void down_load(const TokArgs& p, const char* const (&e)[JG], int o,
                                          u32x4 (&wv)[JG][NCHF]) {
  const int nck = p.f >> 3;
#pragma unroll
  for (int jj = 0; jj < JG; ++jj) {
    if (e[jj]) {
      const char* row = e[jj] + (2 * (size_t)p.f * p.d + (size_t)o * p.f) * 2;
#pragma unroll
      for (int i = 0; i < NCHF; ++i) wv[jj][i] = ldrow(row, chunk_off(i, nck));
    }
  }
}

// acc after adding w_j * (h_j . W_down_j[o]) for those experts, j ascending.
template <int NCHF, int JG>
__device__ __forceinline__ float down_dot(const TokArgs& p, const uint16_t* hs,
                                          const char* const (&e)[JG], const float* wj, int j0,
                                          const u32x4 (&wv)[JG][NCHF], float acc) {
  const int f = p.f, nck = f >> 3;
#pragma unroll
  for (int jj = 0; jj < JG; ++jj) {
    if (e[jj]) {
      const int j = j0 + jj;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NCHF; ++i) s = dot8(lds_chunk(hs + j * f, i, nck), wv[jj][i], s);
      acc = fmaf(wj[j], wave_sum_f32(s), acc);
    }
  }
  return acc;
}

// Down item: wave w takes output channel 4b + w for all k experts, JG experts' rows at a
// time in registers (one group when k <= JG); the first group's loads are in flight before
// any wait for h.
template <int NCHF, int JG, int UPW>
__device__ __forceinline__ void down_item(const TokArgs& p, uint16_t* hs, const char* const* ent,
                                          const float* wj, int b, bool staged, uint32_t epoch) {
  const int o = b * kTokDownCh + wave_id();
  u32x4 wv[JG][NCHF];
  const char* e[JG];
  down_entries<JG>(p, ent, 0, e);
  down_load<NCHF, JG>(p, e, o, wv);
  __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of what follows
  if (!staged) wait_and_stage_h<UPW>(p, hs, epoch);
  float acc = down_dot<NCHF, JG>(p, hs, e, wj, 0, wv, 0.f);
  for (int j0 = JG; j0 < p.k; j0 += JG) {
    down_entries<JG>(p, ent, j0, e);
    down_load<NCHF, JG>(p, e, o, wv);
    acc = down_dot<NCHF, JG>(p, hs, e, wj, j0, wv, acc);
  }
  if ((threadIdx.x & 63) == 0) p.out[o] = acc;
}

// Shared memory of a workgroup besides the dynamic x / h rows.
struct TokShared {
  int32_t id[kMaxK];
  float w[kMaxK];
  const char* ent[kMaxK];
  uint32_t epoch;
};

// Every workgroup's start: wave 0 reads the epoch word, routes the token (or takes the given
// ids and weights) and looks up the k entries, while waves 1..3 stage x in LDS (NCHD:
// 16-byte chunks per lane of a row, d <= 512 * NCHD).  Returns this launch's epoch.
template <int NPL, int NCHD>
__device__ __forceinline__ uint32_t tok_prologue(const TokArgs& p, uint16_t* xs, TokShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = p.k;
  if (wave == 0) {
    uint32_t epoch = 0;
    if (tid == 0) epoch = coh_load(p.epoch_word) + 1u;  // this launch's epoch
    if (p.logits) {
      unsigned long long key[NPL];
      route_keys<NPL>(p.logits, p.E, key);
      route_pick<NPL>(key, k, sh.id, sh.w, nullptr);
    } else if (lane < k) {
      sh.id[lane] = p.topk_ids[lane];
      sh.w[lane] = p.topk_w[lane];
    }
    if (lane < k) {  // the wave reads back its own LDS writes in order
      const int e = sh.id[lane];
      const char* ent = nullptr;
      if (e >= 0 && e < p.E) {
        const int s = p.expert_slot ? p.expert_slot[e] : e;
        if (s >= 0 && (!p.slot_key || p.slot_key[s] == p.key_base + e))
          ent = p.arena + (size_t)s * p.stride;
      }
      if (!ent) set_status(p.status, MOE_ERANGE);
      sh.ent[lane] = ent;
      if (blockIdx.x == 0 && p.logits) {
        if (p.topk_ids) p.topk_ids[lane] = e;
        if (p.topk_w) p.topk_w[lane] = sh.w[lane];
      }
    }
    if (tid == 0) sh.epoch = epoch;
  } else {
    // every load in flight before the first LDS write
    constexpr int XR = (NCHD * 64 + kTokThreads - 65) / (kTokThreads - 64);
    const int nck = p.d >> 3;
    u32x4 xv[XR];
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      const int q = tid - 64 + r * (kTokThreads - 64);
      if (q < nck) xv[r] = ldg16(p.x + (size_t)q * 8);
    }
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      const int q = tid - 64 + r * (kTokThreads - 64);
      if (q < nck) *(u32x4*)&xs[q * 8] = xv[r];
    }
  }
  __syncthreads();
  return sh.epoch;
}

// Workgroup 0's last step: every workgroup has a gate/up item and read the epoch word before
// storing its h; once all of h is of this launch, advance the word for the next one.
template <int UPW>
__device__ __forceinline__ void tok_epilogue(const TokArgs& p, uint16_t* hs, uint32_t epoch,
                                             bool staged) {
  if (blockIdx.x != 0) return;
  if (!staged) wait_and_stage_h<UPW>(p, hs, epoch);
  if (threadIdx.x == 0) coh_store(p.epoch_word, epoch);
}

// bf16 weights.  NPL: logits per lane in the routing wave (E <= 64 * NPL); NCHD / NCHF:
// 16-byte chunks per lane of a gate/up row (d <= 512 * NCHD) and of a down row
// (f <= 512 * NCHF); UPW: units per wave in a gate/up item; JG: experts per register group in
// a down item.
template <int NPL, int NCHD, int UPW, int NCHF, int JG>
__global__ __launch_bounds__(kTokThreads) __attribute__((amdgpu_waves_per_eu(NCHF == 4 && JG <= 6 ? 2 : 1)))
void decode_token(TokArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // x [d], then h [k][f]
  __shared__ TokShared sh;
  uint16_t* xs = lds;
  uint16_t* hs = lds + p.d;
  const uint32_t epoch = tok_prologue<NPL, NCHD>(p, xs, sh);
  // Items b, b + G, ...: the gate/up ones (below n_gu) first, then the down ones.
  const int G = gridDim.x;
  int item = blockIdx.x;
  for (; item < p.n_gu; item += G) gateup_item<NCHD, UPW>(p, xs, sh.ent, item, epoch);
  bool staged = false;
  for (; item < p.n_items; item += G) {
    down_item<NCHF, JG, UPW>(p, hs, sh.ent, sh.w, item - p.n_gu, staged, epoch);
    staged = true;
  }
  tok_epilogue<UPW>(p, hs, epoch, staged);
}

// ------------------------------------------------------------------ MXFP4 weights
// Entry: [codes W_gate][codes W_up][codes W_down][scales W_gate][scales W_up][scales W_down],
// tiles of 16 rows x 128 elements (mx_dev.h).  Both item kinds give a 16-row strip to the
// workgroup's four waves, wave ks taking tiles ks, ks + 4, ... (all of them in flight at
// once) and the partial sums meeting in LDS: the split and order of the weight-streaming
// MXFP4 kernels for one token, so the results are theirs bit for bit.

// Tile kt of a strip (NMAT matrices), loaded whatever kt and the lane, so that every load of
// a present expert is issued and used on every path: a tile past the strip (kt >= nk) reads
// the strip's last tile and a lane past a short last tile its row's first block (both in
// bounds); such values are zeroed where they are used (mx_tile_use).
template <int NMAT>
__device__ __forceinline__ void mx_tile_any(MxTile<NMAT>& t, const uint8_t* const (&cb)[NMAT],
                                            const uint8_t* const (&sb)[NMAT], int kt, int nk,
                                            int krem, int lane) {
  const int q = lane >> 4;
  const int kc = min(kt, nk - 1);
  const bool ok = kt < nk && (kc != nk - 1 || krem == 0 || q < krem);
  const int l = ok ? lane : (lane & 15);
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    t.c[m] = ldg16_nt(cb[m] + (size_t)kc * 1024 + l * 16);
    t.s[m] = ldg_u8(sb[m] + (size_t)kc * 64 + l);
  }
}

// acc[m] += the token row x tile kt of matrix m, with the tile's missing blocks as zeros (a
// tile past the strip adds exact zeros).  xk: the activations (x or h_j) of the strip's row.
template <int NMAT>
__device__ __forceinline__ void mx_tile_use(const MxTile<NMAT>& t, const uint16_t* xk, int kt,
                                            int nk, int krem, int lane, f32x4 (&acc)[NMAT]) {
  const int q = lane >> 4;
  const int kc = min(kt, nk - 1);
  const bool ok = kt < nk && (kc != nk - 1 || krem == 0 || q < krem);
  MxTile<NMAT> u;
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    u.c[m] = ok ? t.c[m] : u32x4{0u, 0u, 0u, 0u};
    u.s[m] = ok ? t.s[m] : 0u;
  }
  mx_tile_mma<NMAT>(u, xk + kc * 128 + (ok ? 32 * q : 0), acc);
}

// Gate/up item (a, rt): units 16 rt .. 16 rt + 15 of the a-th selected expert.  GT: tiles
// per wave per matrix (d <= 512 * GT).
template <int GT>
__device__ __forceinline__ void mx_gateup_item(const TokArgs& p, const uint16_t* xs,
                                               const char* const* ent, int item, uint32_t epoch) {
  const int nbg = p.f / 16;
  const int a = item / nbg, rt = item - a * nbg;
  const int lane = threadIdx.x & 63, ks = wave_id();
  const int K = p.d, nk = (K + 127) >> 7, krem = (K & 127) >> 5;
  const uint8_t* W = (const uint8_t*)uniform_ptr(ent[a]);
  MxTile<2> t[GT];
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (W) {
    const size_t fd = (size_t)p.f * K;
    const uint8_t* const cb[2] = {W + (size_t)rt * 8 * K, W + fd / 2 + (size_t)rt * 8 * K};
    const uint8_t* const sb[2] = {W + 3 * fd / 2 + (size_t)rt * (K / 2),
                                  W + 3 * fd / 2 + fd / 32 + (size_t)rt * (K / 2)};
#pragma unroll
    for (int r = 0; r < GT; ++r) mx_tile_any<2>(t[r], cb, sb, ks + 4 * r, nk, krem, lane);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of what follows
#pragma unroll
    for (int r = 0; r < GT; ++r) mx_tile_use<2>(t[r], xs, ks + 4 * r, nk, krem, lane, acc);
  }
  mx_reduce<2, 4>(acc, 0, ks, lane);
  // lane l < 16 of wave 0 holds the token's row of unit 16 rt + l
  if (W && ks == 0 && lane < 16) {
    const uint16_t hv = f32_to_bf16(silu(acc[0][0]) * acc[1][0]);
    coh_store64(p.hent + (size_t)a * p.f + 16 * rt + lane, (uint64_t)hv | ((uint64_t)epoch << 32));
  }
  __syncthreads();  // the partial sums are read before the next item's waves store theirs
}

// Down item rt: output channels 16 rt .. 16 rt + 15, all k experts (KMAX >= k), every
// expert's tiles in flight before any wait for h; out = sum_j w_j y_j, j ascending.  DT:
// tiles per wave per expert (f <= 512 * DT).
template <int DT, int KMAX>
__device__ __forceinline__ void mx_down_item(const TokArgs& p, uint16_t* hs,
                                             const char* const* ent, const float* wj, int rt,
                                             bool staged, uint32_t epoch) {
  const int lane = threadIdx.x & 63, ks = wave_id();
  const int K = p.f, nk = (K + 127) >> 7, krem = (K & 127) >> 5;
  const size_t fd = (size_t)K * p.d;
  const uint8_t* W[KMAX];  // one pointer decides both loading and multiplying an expert
  MxTile<1> t[KMAX][DT];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    W[j] = j < p.k ? (const uint8_t*)uniform_ptr(ent[j]) : nullptr;
    if (W[j]) {
      const uint8_t* const cb[1] = {W[j] + fd + (size_t)rt * 8 * K};
      const uint8_t* const sb[1] = {W[j] + 3 * fd / 2 + 2 * (fd / 32) + (size_t)rt * (K / 2)};
#pragma unroll
      for (int r = 0; r < DT; ++r) mx_tile_any<1>(t[j][r], cb, sb, ks + 4 * r, nk, krem, lane);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of what follows
  if (!staged) wait_and_stage_h<1>(p, hs, epoch);
  float o = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < p.k) {
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if (W[j]) {
#pragma unroll
        for (int r = 0; r < DT; ++r) mx_tile_use<1>(t[j][r], hs + j * K, ks + 4 * r, nk, krem, lane, acc);
      }
      mx_reduce<1, 4>(acc, 0, ks, lane);
      if (W[j]) o = fmaf(wj[j], acc[0][0], o);
      __syncthreads();  // the partial sums are read before the next expert's are stored
    }
  }
  if (ks == 0 && lane < 16) p.out[16 * rt + lane] = o;
}

template <int NPL, int KMAX>
__global__ __launch_bounds__(kTokThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_token_mx(TokArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // x [d], then h [k][f]
  __shared__ TokShared sh;
  uint16_t* xs = lds;
  uint16_t* hs = lds + p.d;
  const uint32_t epoch = tok_prologue<NPL, 8>(p, xs, sh);
  const int G = gridDim.x;
  int item = blockIdx.x;
  for (; item < p.n_gu; item += G) mx_gateup_item<8>(p, xs, sh.ent, item, epoch);
  bool staged = false;
  for (; item < p.n_items; item += G) {
    mx_down_item<4, KMAX>(p, hs, sh.ent, sh.w, item - p.n_gu, staged, epoch);
    staged = true;
  }
  tok_epilogue<1>(p, hs, epoch, staged);
}

// Grid: two workgroups per compute unit where the occupancy allows (eight waves, each with
// 24-32 KB of weight loads in flight, keep HBM busy; at d = 4096, f = 2048, k = 6 the bf16
// items then divide evenly, 3 gate/up and 2 down per workgroup), and no more workgroups than
// gate/up items (each must store some of h before workgroup 0 may advance the epoch).
template <typename K>
int launch_grid(K kern, const TokArgs& p, size_t lds, hipStream_t stream) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kTokThreads, lds) != hipSuccess ||
      occ <= 0)
    occ = 1;
  const int grid = std::min(p.n_gu, std::min(occ, 2) * num_cus());
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kTokThreads), lds, stream, p);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

template <int NPL, int NCHD, int UPW, int NCHF, int JG>
int launch_token(const TokArgs& p, size_t lds, hipStream_t stream) {
  return launch_grid(decode_token<NPL, NCHD, UPW, NCHF, JG>, p, lds, stream);
}

template <int NPL>
int launch_token_mx(TokArgs p, size_t lds, hipStream_t stream) {
  p.n_gu = p.k * (p.f / 16);
  p.n_items = p.n_gu + p.d / 16;
  if (p.k <= 6) return launch_grid(decode_token_mx<NPL, 6>, p, lds, stream);
  return launch_grid(decode_token_mx<NPL, 8>, p, lds, stream);
}

// MXFP4 shapes the one-launch kernel takes: gate/up strips of d <= 4096 and down strips of
// f <= 2048 held whole in registers, k <= 8.
bool token_mx_supported(int k, int d, int f) { return d <= 4096 && f <= 2048 && k <= 8; }

template <int NPL, int NCHD, int UPW>
int launch_token_f(TokArgs p, size_t lds, hipStream_t stream) {
  p.n_gu = p.k * (p.f / (4 * UPW));
  p.n_items = p.n_gu + p.d / kTokDownCh;
  if (p.f > 2048) return launch_token<NPL, NCHD, UPW, 16, 2>(p, lds, stream);
  if (p.k <= 4) return launch_token<NPL, NCHD, UPW, 4, 4>(p, lds, stream);
  if (p.k <= 6) return launch_token<NPL, NCHD, UPW, 4, 6>(p, lds, stream);
  return launch_token<NPL, NCHD, UPW, 4, 8>(p, lds, stream);
}

template <int NPL>
int launch_token_d(const TokArgs& p, size_t lds, hipStream_t stream) {
  if (p.d <= 4096) return launch_token_f<NPL, 8, 2>(p, lds, stream);
  return launch_token_f<NPL, 16, 1>(p, lds, stream);
}

}  // namespace

extern "C" size_t moe_decode_token_workspace_bytes(int k, int f) {
  if (k <= 0 || f <= 0) return kTokHdrBytes;
  return kTokHdrBytes + (size_t)k * f * 8;  // an 8-byte entry per unit at most (UPW = 1)
}

extern "C" int moe_decode_token(const float* logits, const void* x, int E, int k, int d, int f,
                                const int32_t* expert_slot, const void* arena, size_t entry_stride,
                                int w_dtype, const int32_t* slot_key, int key_base,
                                int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                float* out, int32_t* status, hipStream_t stream) {
  if (E <= 0 || E > kMaxE || k <= 0 || k > kMaxK || k > E) return MOE_EINVAL;
  if (d <= 0 || f <= 0 || d % 64 != 0 || f % 64 != 0) return MOE_EINVAL;
  const bool mx = w_dtype == MOE_MXFP4;
  if (w_dtype != MOE_BF16 && !mx) return MOE_EUNSUPPORTED;
  if (d > 8192 || f > 8192 || ((size_t)d + (size_t)k * f) * 2 > 65536) return MOE_EUNSUPPORTED;
  if (mx && !token_mx_supported(k, d, f)) return MOE_EUNSUPPORTED;
  if (entry_stride < moe_entry_bytes(d, f, w_dtype) || entry_stride % 16 != 0) return MOE_EINVAL;
  if (!x || !arena || !ws || !out) return MOE_EINVAL;
  if (!logits && (!topk_ids || !topk_w)) return MOE_EINVAL;
  if (!moe_aligned16(x) || !moe_aligned16(arena) || !moe_aligned16(ws) || !moe_aligned16(out))
    return MOE_EINVAL;
  if (ws_bytes < moe_decode_token_workspace_bytes(k, f)) return MOE_EINVAL;
  TokArgs p{};
  p.logits = logits;
  p.x = (const uint16_t*)x;
  p.E = E;
  p.k = k;
  p.d = d;
  p.f = f;
  p.expert_slot = expert_slot;
  p.arena = (const char*)arena;
  p.stride = entry_stride;
  p.slot_key = slot_key;
  p.key_base = key_base;
  p.topk_ids = topk_ids;
  p.topk_w = topk_w;
  p.epoch_word = (uint32_t*)ws;
  p.hent = (uint64_t*)((char*)ws + kTokHdrBytes);
  p.out = out;
  p.status = status;
  const size_t lds = ((size_t)d + (size_t)k * f) * 2;
  if (mx) return E <= 256 ? launch_token_mx<4>(p, lds, stream) : launch_token_mx<16>(p, lds, stream);
  if (E <= 256) return launch_token_d<4>(p, lds, stream);
  return launch_token_d<16>(p, lds, stream);
}
