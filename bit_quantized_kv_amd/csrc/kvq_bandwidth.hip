// kvq_bandwidth.hip -- a plain streaming-read kernel, the practical HBM read
// ceiling that the decode kernel's bandwidth is compared with.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

// Grid-stride read of n16 16-byte vectors, consecutive lanes on consecutive
// vectors; the XOR of everything read decides one conditional store, so no
// load can be dropped.  (A variant with four loads a grid-stride apart in
// flight per thread measured slower.)
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ a, int64_t n16,
                                                          uint32_t* sink) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) acc ^= ld_global<u32x4_t>(a + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = 1u;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, stream, (const u32x4_t*)buf, bytes / 16,
                     sink);
  return hipGetLastError();
}

}  // namespace kvq
