// Streaming-read probe for gfx950: reads a device buffer once with 16-byte
// non-temporal loads, every workgroup sweeping its own contiguous chunk
// (kProbeUnroll loads in flight per lane, each wave-load 1 KiB contiguous),
// and folds the data into one word per wave so the loads stay live. Its
// rate is a measured HBM read ceiling on this device, the figure the
// gathers (which read whole 256-byte rows non-temporally) are set against
// beside the nominal peak. Contiguous per-workgroup chunks measured faster
// than a grid-stride sweep of the whole buffer (7.1 vs 6.5 TB/s over 8 GiB).
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr int kProbeBlocks = 8192;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* p, long long n16, uint32_t* sink) {
  constexpr long long kTile = static_cast<long long>(kProbeThreads) * kProbeUnroll;
  // chunks are whole tiles; the last chunks may be short or empty
  const long long chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const long long per = (chunk + kTile - 1) / kTile * kTile;
  const long long lo = min(n16, static_cast<long long>(blockIdx.x) * per);
  const long long hi = min(n16, lo + per);
  uint32_t acc = 0;
  long long i = lo + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < hi; i += kTile) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load16_stream(p + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kProbeThreads) {
    const uint4 v = load16_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane_id() == 0) sink[(static_cast<long long>(blockIdx.x) * kProbeThreads + threadIdx.x) / kWave] = acc;
}

int stream_read_blocks() { return kProbeBlocks; }
int stream_read_waves_per_block() { return kProbeThreads / kWave; }

hipError_t launch_stream_read(const void* p, long long n16, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(p), n16, sink);
  return hipGetLastError();
}

}  // namespace tsa
