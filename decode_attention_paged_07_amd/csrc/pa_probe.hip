// HBM read-bandwidth probe for gfx950: the ceiling a purely streaming kernel
// reaches on this device, reported beside the decode kernels' bandwidth.
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

hipError_t launch_read_probe(const void* buf, uint64_t bytes, int workgroups, unsigned* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(pa_read_probe_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4p*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
