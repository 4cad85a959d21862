// Streaming-read probe for gfx950: reads a device buffer once, front to back,
// with 16-byte non-temporal loads spread over every CU (grid-stride, eight
// loads in flight per lane), and folds the data into one word per wave so the
// loads stay live. Its rate is a measured HBM read ceiling on this device, the
// figure the gathers (which read whole 256-byte rows non-temporally) are set
// against beside the nominal peak.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* p, long long n16, uint32_t* sink) {
  const long long stride = static_cast<long long>(gridDim.x) * kProbeThreads;
  long long i = static_cast<long long>(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load16_stream(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = load16_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane_id() == 0) sink[(static_cast<long long>(blockIdx.x) * kProbeThreads + threadIdx.x) / kWave] = acc;
}

int stream_read_blocks() { return 256 * 8; }

hipError_t launch_stream_read(const void* p, long long n16, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_read_blocks()), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(p), n16, sink);
  return hipGetLastError();
}

}  // namespace tsa
