// Expert SwiGLU FFNs over tokens grouped by expert: the C entry point and the fp32 path.
//
// For every active expert e and its grouped rows p in [offsets[e], offsets[e+1]):
//   h = SiLU(x[perm[p]/k] W_gate^T) * (x[perm[p]/k] W_up^T),   y_perm[p] = h W_down^T
// (the GPU runs the experts it holds on the tokens routed to them: FreeToken
// RTX-4090 page, component table; SwiGLU form and no biases are a reading).
//
// Paths by weight type:
//  * fp32 (MOE_F32 weights): plain fp32 FMA loops in this file; small shapes only.
//  * GEMV (bf16, decode-shaped counts, a few tokens per expert): weight streaming from
//    HBM into registers; up to 8 tokens per call with packed bf16 dot products and whole
//    1 KB row loads (ffn_dot.hip), above that split by rows per expert between those and
//    MFMA (ffn_gemv.hip).
//  * GEMM (bf16, prefill-shaped counts): LDS-tiled grouped GEMM with direct global->LDS
//    loads and persistent XCD-aware workgroups, ffn_gemm.hip.
//  * MXFP4 weights (bf16 activations): codes expanded to bf16 in registers and multiplied
//    on the matrix cores against staged token rows: weight streaming for decode-shaped
//    counts (ffn_mx.hip), a grouped GEMM for prefill-shaped ones (ffn_mx_gemm.hip).
// Both bf16 paths fuse SiLU(g)*u into the gate/up epilogue and write h once as bf16.
#include <algorithm>
#include <mutex>

#include "ffn_args.h"

using namespace moe;

namespace moe {
// Both MXFP4 projections in one launch after a small clearing kernel (ffn_mx.hip); p.h is a
// workspace of T*k*f/2 eight-byte entries (T * k * f * 4 bytes).
int launch_ffn_mx_one(const FfnArgs& p, int T, int y_dtype, hipStream_t stream, int experts);
}  // namespace moe

namespace {

constexpr int kDotMaxT = 8;     // up to this many tokens per call every expert takes the dot path
constexpr int kDotMaxRows = 4;  // rows per expert the dot path takes when splitting
// MXFP4: tokens per call of the one-launch form; above twice as many, the most rows an expert
// may have on the weight-streaming path
constexpr int kMxMaxRows = 16;
// AUTO path: bf16 experts take the grouped GEMM above this many rows per expert on average
// (T*k / E), MXFP4 experts above kMxGemmMinRowsPerExpert (their streaming path, with the row
// split above, stays ahead to about 5 rows per expert at Zipf 0.2 and beyond 8 when skewed).
constexpr long long kGemmMinRowsPerExpert = 2, kMxGemmMinRowsPerExpert = 8;
// Rounds of resident workgroups in the row-split dot-product launches (each loops over items).
constexpr int kDotSplitRounds = 2;

// ------------------------------------------------------------------ fp32 path
__global__ __launch_bounds__(64) void f32_gateup(FfnArgs p) {
  const int e = blockIdx.x;
  if (!active(p, e)) return;
  const char* w = entry_of(p, e);
  if (!w) return;
  const int i = blockIdx.y * 64 + threadIdx.x;
  const float* wg = (const float*)w + (size_t)i * p.d;
  const float* wu = wg + (size_t)p.f * p.d;
  const float* X = (const float*)p.x;
  float* H = (float*)p.h;
  for (int q = p.offsets[e]; q < p.offsets[e + 1]; ++q) {
    const float* xr = X + (size_t)(p.perm[q] / p.k) * p.d;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < p.d; ++c) {
      g = fmaf(xr[c], wg[c], g);
      u = fmaf(xr[c], wu[c], u);
    }
    H[(size_t)q * p.f + i] = g / (1.0f + expf(-g)) * u;
  }
}

__global__ __launch_bounds__(64) void f32_down(FfnArgs p) {
  const int e = blockIdx.x;
  if (!active(p, e)) return;
  const char* w = entry_of(p, e);
  if (!w) return;
  const int o = blockIdx.y * 64 + threadIdx.x;
  const float* wd = (const float*)w + 2 * (size_t)p.f * p.d + (size_t)o * p.f;
  const float* H = (const float*)p.h;
  float* Y = (float*)p.y;
  for (int q = p.offsets[e]; q < p.offsets[e + 1]; ++q) {
    const float* hr = H + (size_t)q * p.f;
    float s = 0.f;
    for (int i = 0; i < p.f; ++i) s = fmaf(hr[i], wd[i], s);
    Y[(size_t)q * p.d + o] = s;
  }
}

}  // namespace

extern "C" size_t moe_entry_bytes(int d, int f, int w_dtype) {
  if (d <= 0 || f <= 0) return 0;
  const size_t fd = (size_t)d * f;
  switch (w_dtype) {
    case MOE_F32: return 3 * fd * 4;
    case MOE_BF16: return 3 * fd * 2;
    case MOE_MXFP4: return 3 * fd / 2 + 3 * (fd / 32);
    default: return 0;
  }
}

// The SwiGLU intermediate h, T*k rows of f units: what every path needs at least.
static size_t ffn_h_bytes(int T, int k, int f, int act_dtype) {
  return (size_t)T * k * f * (act_dtype == MOE_F32 ? 4 : 2);
}

// Up to kMxMaxRows tokens with bf16 activations, room for h as tagged 8-byte entries (4 bytes
// per unit), which lets MXFP4 calls run both projections in one launch.
extern "C" size_t moe_expert_ffn_workspace_bytes(int T, int k, int f, int act_dtype) {
  if (T <= 0 || k <= 0 || f <= 0) return 256;
  const size_t el = act_dtype == MOE_F32 ? 4 : T <= kMxMaxRows ? 4 : 2;
  return ((size_t)T * k * f * el + 255) / 256 * 256;
}

extern "C" int moe_expert_ffn(const void* x, int act_dtype, const int32_t* perm,
                              const int32_t* offsets, int T, int k, int E, int d, int f,
                              const int32_t* expert_slot, const void* arena, size_t entry_stride,
                              int w_dtype, const uint8_t* expert_mask, const int32_t* slot_key,
                              int key_base, void* ws, size_t ws_bytes, void* y_perm, int y_dtype,
                              int path, int32_t* status, hipStream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || k <= 0 || k > kMaxK || k > E) return MOE_EINVAL;
  if (d <= 0 || f <= 0 || d % 64 != 0 || f % 64 != 0) return MOE_EINVAL;
  if ((long long)T * k >= (1ll << 31)) return MOE_EINVAL;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM) return MOE_EINVAL;
  const bool f32 = w_dtype == MOE_F32, mx = w_dtype == MOE_MXFP4;
  if (f32) {
    if (act_dtype != MOE_F32 || y_dtype != MOE_F32) return MOE_EUNSUPPORTED;
  } else if (w_dtype == MOE_BF16 || mx) {
    if (act_dtype != MOE_BF16 || (y_dtype != MOE_F32 && y_dtype != MOE_BF16)) return MOE_EUNSUPPORTED;
  } else {
    return MOE_EUNSUPPORTED;
  }
  const bool bf16_gemm_fits = ffn_gemm_supported(T, k, d, f);
  if (w_dtype == MOE_BF16 && path == MOE_PATH_GEMM && !bf16_gemm_fits) return MOE_EUNSUPPORTED;
  const size_t need = mx ? moe_entry_bytes(d, f, w_dtype) : 3 * (size_t)d * f * (f32 ? 4 : 2);
  if (entry_stride < need || entry_stride % 16 != 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !perm || !offsets || !arena || !ws || !y_perm) return MOE_EINVAL;
  if (!moe_aligned16(x) || !moe_aligned16(arena) || !moe_aligned16(ws) || !moe_aligned16(y_perm))
    return MOE_EINVAL;
  if (ws_bytes < ffn_h_bytes(T, k, f, act_dtype)) return MOE_EINVAL;

  FfnArgs p{x, perm, offsets, k, E, d, f, expert_slot, (const char*)arena, entry_stride,
            expert_mask, slot_key, key_base, ws, y_perm, status};
  if (f32) {
    hipLaunchKernelGGL(f32_gateup, dim3(E, f / 64), dim3(64), 0, stream, p);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(f32_down, dim3(E, d / 64), dim3(64), 0, stream, p);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  if (mx) {
    const bool gemm = path == MOE_PATH_GEMM ||
                      (path == MOE_PATH_AUTO && (long long)T * k > kMxGemmMinRowsPerExpert * E) ||
                      !ffn_mx_supported(d, f);
    if (gemm) return launch_ffn_mx_gemm(p, T, y_dtype, stream);
    const int A = T * k, experts = std::min(E, A);
    // Up to kMxMaxRows tokens, with room for h as tagged entries, gate/up and down run in one
    // launch where gate/up has a wave per strip: the down workgroups of an expert start as soon
    // as its h is complete, while other experts' gate/up workgroups still stream (d = 4096,
    // f = 2048, top 6: T = 8 97 vs 102 µs at Zipf 0.2, 74 vs 76 at Zipf 1; T = 13 and T = 16
    // at Zipf 1 12% faster; bit-identical).
    if (T <= kMxMaxRows && ws_bytes >= (size_t)A * f * 4) return launch_ffn_mx_one(p, T, y_dtype, stream, experts);
    // An expert has at most T rows (a token picks it once).  The weight-streaming MXFP4
    // kernels stream an expert's weights once for up to 16 rows (once per 16 rows beyond).  Up
    // to 2 * kMxMaxRows tokens every expert stays there (at most two streams; d = 4096, f = 2048,
    // top 6, Zipf 1: T = 24 150 -> 112 us, T = 32 153 -> 129 us against sending the experts above
    // 16 rows to the grouped GEMM; Zipf 0.2 2% faster); above that, experts with more than kMxMaxRows rows go
    // to the grouped GEMM, which streams them once per 64 or 256 rows and pays a fixed start-up
    // per workgroup instead (at T = 64, Zipf 1, moving that split to 32 rows costs 33%: the
    // streaming launch that runs first grows while the GEMM still waits behind it).  At most
    // A / (kMxMaxRows + 1) experts have more rows.
    if (T <= 2 * kMxMaxRows) return launch_ffn_mx(p, y_dtype, stream, experts);
    FfnArgs few = p, many = p;
    few.nmax = kMxMaxRows;
    many.nmin = kMxMaxRows + 1;
    int rc = launch_ffn_mx(few, y_dtype, stream, experts);
    if (rc == MOE_OK) rc = launch_ffn_mx_gemm(many, T, y_dtype, stream, std::max(1, A / (kMxMaxRows + 1)));
    return rc;
  }
  // bf16: the grouped GEMM from more than 2 rows per expert on average (measured crossover
  // near 2 at Zipf 0.2; with skewed routing the GEMM wins from fewer tokens still, as its
  // 256-row tiles read a hot expert's weights once per 256 rows).  Past the GEMM's size limit
  // the weight-streaming kernels (64-bit offsets) take the call.
  if (path == MOE_PATH_AUTO)
    path = (long long)T * k <= kGemmMinRowsPerExpert * E || !bf16_gemm_fits ? MOE_PATH_GEMV : MOE_PATH_GEMM;
  if (path == MOE_PATH_GEMM) return launch_ffn_gemm(p, y_dtype, stream);
  const int A = T * k, experts = std::min(E, A);
  if (!ffn_dot_supported(d, f)) return launch_ffn_gemv(p, T, y_dtype, stream, experts, 3);
  // One token: k experts give only ~2 rounds of workgroups; one persistent round of looping
  // workgroups trims the second round's tail (about 1.5% of the layer).
  if (T <= kDotMaxT) return launch_ffn_dot(p, y_dtype, stream, experts, 3, T == 1 ? 1 : 0);
  // More tokens: split the experts by rows (counted on the device), up to the GEMM switch.
  // Up to kDotMaxRows rows the dot-product kernels stream an expert's weights once at full
  // rate; above that the MFMA kernels take the expert (their cost per row is far lower).  At most
  // A / (kDotMaxRows + 1) experts have more rows, which bounds the second grid.  The first
  // class has no host-side bound below min(E, A) experts, most of them absent when routing
  // is skewed, so its launches are capped grids of looping workgroups: an absent item costs
  // one lookup per workgroup instead of one per (expert, row block).
  FfnArgs few = p, many = p;
  few.nmax = kDotMaxRows;
  many.nmin = kDotMaxRows + 1;
  const int many_max = std::min(E, A / (kDotMaxRows + 1));
  int rc = launch_ffn_dot(few, y_dtype, stream, experts, 1, kDotSplitRounds);
  if (rc == MOE_OK) rc = launch_ffn_gemv(many, T, y_dtype, stream, many_max, 1);
  if (rc == MOE_OK) rc = launch_ffn_dot(few, y_dtype, stream, experts, 2, kDotSplitRounds);
  if (rc == MOE_OK) rc = launch_ffn_gemv(many, T, y_dtype, stream, many_max, 2);
  return rc;
}

// ---------------------------------------------------------------- no-allocation variant
// The SwiGLU intermediate of moe_expert_ffn_noalloc lives in this file-scope device array:
// every GPU the library runs on holds its own copy from module load to process end.  In host
// code the name `scratch` is only a host-side stand-in, so its device address is looked up
// once per device (with that device current) and only that address is ever passed on.
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of this device's scratch array, or nullptr if it cannot be obtained.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t moe_expert_ffn_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int moe_expert_ffn_noalloc(const void* x, int act_dtype, const int32_t* perm,
                                      const int32_t* offsets, int T, int k, int E, int d, int f,
                                      const int32_t* expert_slot, const void* arena,
                                      size_t entry_stride, int w_dtype, const uint8_t* expert_mask,
                                      const int32_t* slot_key, int key_base, void* y_perm,
                                      int y_dtype, int path, int32_t* status, hipStream_t stream) {
  if (T < 0 || k <= 0 || f <= 0) return MOE_EINVAL;
  if (ffn_h_bytes(T, k, f, act_dtype) > kScratchBytes) return MOE_ETOOBIG;
  void* ws = scratch_ptr();
  if (!ws) return MOE_EHIP;
  return moe_expert_ffn(x, act_dtype, perm, offsets, T, k, E, d, f, expert_slot, arena,
                        entry_stride, w_dtype, expert_mask, slot_key, key_base, ws, kScratchBytes,
                        y_perm, y_dtype, path, status, stream);
}
