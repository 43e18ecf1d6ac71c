// Read-bandwidth probe for gfx950: how fast the memory system streams a
// buffer into the CUs, the practical ceiling the decode pass is measured
// against beside the HBM peak.  Three access forms: one contiguous sweep
// with the default cache policy, the same with non-temporal loads, and
// tiles of a given size read whole in a given (e.g. shuffled) order with
// non-temporal loads -- the access of a block-table walk over a pool of
// randomly placed blocks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;

// Folds what a thread read into a value the compiler must keep: a store
// happens only for a pattern no buffer of this probe holds, so the loads stay
// and almost nothing is written.
__device__ __forceinline__ void keep(uint32_t acc, uint32_t* sink) {
  if (acc == 0x9E3779B9u) sink[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void read_sweep_kernel(const u32x4* buf, int64_t n16,
                                                                   uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  // four loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = NT ? __builtin_nontemporal_load(buf + i + u * stride) : buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(buf + i) : buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  keep(acc, sink);
}

// Each wave reads whole tiles: tile order[t] of tile_bytes (a multiple of
// 1 KiB), one 1 KiB row per load instruction, all of a tile's loads issued
// before any is used.
__global__ __launch_bounds__(kProbeThreads) void read_tiles_kernel(const char* buf, const int32_t* order,
                                                                   int64_t tiles, int64_t tile_bytes,
                                                                   int64_t num_tiles, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
  const int64_t waves = ((int64_t)gridDim.x * kProbeThreads) >> 6;
  const int rows = (int)(tile_bytes / 1024);
  uint32_t acc = 0;
  for (int64_t t = wave; t < tiles; t += waves) {
    int64_t id = order[t];
    id = id < 0 ? 0 : (id >= num_tiles ? num_tiles - 1 : id);
    const u32x4* p = reinterpret_cast<const u32x4*>(buf + id * tile_bytes) + lane;
    for (int r0 = 0; r0 < rows; r0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = r0 + r < rows ? __builtin_nontemporal_load(p + (r0 + r) * 64) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < 8; ++r) acc ^= v[r].x ^ v[r].y ^ v[r].z ^ v[r].w;
    }
  }
  keep(acc, sink);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, int mode, const int32_t* order,
                             int64_t tile_bytes, int64_t tiles, uint32_t* sink, int grid,
                             hipStream_t stream) {
  const dim3 g(grid), b(kProbeThreads);
  if (mode == 0)
    hipLaunchKernelGGL(read_sweep_kernel<false>, g, b, 0, stream, static_cast<const u32x4*>(buf), bytes / 16, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(read_sweep_kernel<true>, g, b, 0, stream, static_cast<const u32x4*>(buf), bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_tiles_kernel, g, b, 0, stream, static_cast<const char*>(buf), order, tiles, tile_bytes,
                       bytes / tile_bytes, sink);
  return hipGetLastError();
}

}  // namespace pkv
