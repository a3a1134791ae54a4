// Measurement helpers: achievable HBM read bandwidth, and a plain copy of
// known size used to scale hardware byte counters.
#include <algorithm>

#include "common.h"

using namespace moe;

namespace {

constexpr int kProbeBlocks = 4096;

// Each thread keeps 8 independent 16-byte loads in flight per iteration; full chunks are
// loaded without per-load bounds checks so the loads issue back to back.  The loads are
// non-temporal, as for any data streamed once (plain loads of the same stream stay near
// 6.3 TB/s on MI355X, non-temporal ones reach about 7.1 TB/s).
__global__ __launch_bounds__(256) void hbm_read(const u32x4* __restrict__ src, size_t n16,
                                                uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t chunk = (size_t)256 * 8;
  const size_t stride = (size_t)gridDim.x * chunk;
  for (size_t base = (size_t)blockIdx.x * chunk; base < n16; base += stride) {
    const size_t i = base + threadIdx.x;
    if (base + chunk <= n16) {
      u32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = __builtin_nontemporal_load(&src[i + q * 256]);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc ^= v[q][0] ^ v[q][1] ^ v[q][2] ^ v[q][3];
    } else {
      for (int q = 0; q < 8; ++q)
        if (i + q * 256 < n16) {
          const u32x4 v = src[i + q * 256];
          acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

__global__ __launch_bounds__(256) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes % 16 != 0 || !moe_aligned16(src)) return MOE_EINVAL;
  if (bytes == 0) return MOE_OK;
  const size_t n16 = bytes / 16;
  const int blocks = (int)std::min<size_t>(kProbeBlocks, (n16 + 2047) / 2048);
  hipLaunchKernelGGL(hbm_read, dim3(blocks), dim3(256), 0, stream, (const u32x4*)src, n16, sink);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int moe_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes % 16 != 0 || !moe_aligned16(src) || !moe_aligned16(dst)) return MOE_EINVAL;
  if (bytes == 0) return MOE_OK;
  const size_t n16 = bytes / 16;
  const int blocks = (int)std::min<size_t>(kProbeBlocks, (n16 + 255) / 256);
  hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst, n16);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, size or limit)";
    case MOE_EUNSUPPORTED: return "unsupported dtype combination";
    case MOE_EHIP: return "HIP launch or copy failed";
    case MOE_ECAPACITY: return "more unique experts requested than cache slots";
    case MOE_ERANGE: return "id, layer or slot out of range, or stale cache slot";
    case MOE_ETOOBIG: return "request larger than a fixed library limit (no-allocation scratch)";
    case MOE_ETIMEOUT: return "a bounded device wait gave up";
    default: return "unknown status";
  }
}

extern "C" int moe_abi_version(void) { return 3; }
