// Plain streaming read of a device buffer (libqlora_probe.so): the read
// ceiling that memory-bound kernels are compared with at their own size.
#include <hip/hip_runtime.h>

#include "../../include/qlora_read_probe.h"

namespace {

// Grid-stride walk, four independent 16-byte loads in flight per lane.  The
// XOR of everything read is compared with a constant so the loads stay.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * stride < n16 ? p[i + u * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

extern "C" int qlora_read_probe(const void* src, int64_t bytes, int grid, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > 65536 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}
