// Streaming-read ceiling kernel (measurement aid, not part of the method):
// every 16-byte word of a buffer is loaded once, non-temporally, with U loads
// in flight per lane over a grid-stride loop sized to fill the chip.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;
constexpr int kProbeGrid = 16384;
constexpr uint32_t kSentinel = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                                     size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
       i += stride * kProbeLoads) {
    uint4 v[kProbeLoads];
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u) {
      const size_t j = i + (size_t)u * stride;
      v[u] = j < n16 ? load16_stream(p + j) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kSentinel) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
  const unsigned grid = (unsigned)(need < (size_t)kProbeGrid ? need : (size_t)kProbeGrid);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace prhs
