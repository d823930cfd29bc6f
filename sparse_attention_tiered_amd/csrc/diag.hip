// Diagnostic: a plain streaming read of a device buffer, to measure the
// practical HBM read ceiling on the same run as the decode kernels.  Not part
// of the decode step.
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

__global__ __launch_bounds__(256) void k_read_stream(const u32x4* __restrict__ p, size_t n,
                                                     unsigned* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) acc ^= p[i];
  // the sink is written only if the xor happens to hit a fixed value, so the
  // loads cannot be removed
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = 1u;
}

hipError_t launch_read_stream(const void* buf, size_t bytes, unsigned* sink, hipStream_t s) {
  // 2048 workgroups: measured best for a grid-stride stream on MI355X
  hipLaunchKernelGGL(k_read_stream, dim3(2048), dim3(256), 0, s,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace spin
