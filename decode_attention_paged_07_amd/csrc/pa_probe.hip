// HBM read-bandwidth probes for gfx950: the ceilings a purely streaming
// kernel and a tile-gathering kernel reach on this device, reported beside
// the decode kernels' bandwidth.
//
// Each lane reads 16-byte words with non-temporal loads (every byte once, as
// the decode kernels do with K and V), eight independent loads in flight per
// lane per iteration, in a grid-stride walk so one wave instruction covers
// 1 KiB contiguous. The XOR of everything read is compared with a constant so
// the loads cannot be dropped; the sink is written only on that (practically
// impossible) match.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

constexpr int kProbeUnroll = 8;

__global__ void __launch_bounds__(256)
pa_read_probe_kernel(const u32x4p* __restrict__ buf, uint64_t words, unsigned* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4p acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < words; i += kProbeUnroll * stride) {
    u32x4p v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < words; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

// Gather probe: wave w reads whole tiles ids[w], ids[w + W], ... (W waves in
// the grid), DEPTH tiles in flight before any is consumed. A tile is WPL KiB;
// lane l reads 16-byte words l, l+64, ... of it. Ids are clamped into the pool.
// The wave index is made wave-uniform so the ids are scalar loads: a vector
// load of the next id would join the tile loads' in-order count, and each
// step would wait one extra memory latency for it before issuing its tiles.
template <int WPL, int DEPTH>
__global__ void __launch_bounds__(256)
pa_gather_probe_kernel(const u32x4p* __restrict__ pool, uint64_t pool_tiles, const int32_t* __restrict__ ids,
                       int num_tiles, unsigned* __restrict__ sink) {
  constexpr int kWords = WPL * 64;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = gridDim.x * 4;
  u32x4p acc = {0u, 0u, 0u, 0u};
  for (int i = wave; i < num_tiles; i += W * DEPTH) {
    u32x4p v[DEPTH][WPL];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int t = i + d * W;
      if (t < num_tiles) {
        uint64_t id = (uint32_t)ids[t];
        id = id < pool_tiles ? id : pool_tiles - 1;
        const u32x4p* base = pool + id * kWords;
#pragma unroll
        for (int w = 0; w < WPL; ++w) v[d][w] = __builtin_nontemporal_load(base + lane + 64 * w);
      } else {
#pragma unroll
        for (int w = 0; w < WPL; ++w) v[d][w] = u32x4p{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int w = 0; w < WPL; ++w) acc ^= v[d][w];
  }
  const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

template <int WPL>
static void launch_gather(const void* pool, uint64_t pool_tiles, const int32_t* ids, int num_tiles, int depth,
                          int workgroups, unsigned* sink, hipStream_t stream) {
  const auto* p = static_cast<const u32x4p*>(pool);
  if (depth == 1)
    hipLaunchKernelGGL((pa_gather_probe_kernel<WPL, 1>), dim3(workgroups), dim3(256), 0, stream, p, pool_tiles, ids,
                       num_tiles, sink);
  else
    hipLaunchKernelGGL((pa_gather_probe_kernel<WPL, 2>), dim3(workgroups), dim3(256), 0, stream, p, pool_tiles, ids,
                       num_tiles, sink);
}

hipError_t launch_gather_probe(const void* pool, uint64_t pool_bytes, int tile_bytes, const int32_t* ids,
                               int num_tiles, int depth, int workgroups, unsigned* sink, hipStream_t stream) {
  const uint64_t pool_tiles = pool_bytes / (uint64_t)tile_bytes;
  switch (tile_bytes) {
    case 1024: launch_gather<1>(pool, pool_tiles, ids, num_tiles, depth, workgroups, sink, stream); break;
    case 2048: launch_gather<2>(pool, pool_tiles, ids, num_tiles, depth, workgroups, sink, stream); break;
    case 4096: launch_gather<4>(pool, pool_tiles, ids, num_tiles, depth, workgroups, sink, stream); break;
    case 8192: launch_gather<8>(pool, pool_tiles, ids, num_tiles, depth, workgroups, sink, stream); break;
    case 18432: launch_gather<18>(pool, pool_tiles, ids, num_tiles, depth, workgroups, sink, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, uint64_t bytes, int workgroups, unsigned* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(pa_read_probe_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4p*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
