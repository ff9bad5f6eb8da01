// Read-bandwidth probe: a measurement aid, not part of the computation.
//
// Streams a buffer once with the access pattern of the decode scan's key
// loads (16-byte loads, each wave covering 1 KB contiguous per load, eight
// loads in flight per lane, a grid of 2048 four-wave workgroups striding over
// the buffer) and does nothing with the data but fold it into one word per
// wave, so the loads cannot be dropped.  Its duration gives the read rate
// this GPU reaches for such a stream, the practical ceiling that the
// HBM-bound kernels are compared against next to the published peak.
#include "../../include/li.h"
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeBlocks = 2048;
static_assert(kProbeBlocks * (kProbeThreads / 64) == LI_READ_PROBE_SINK_WORDS, "one sink word per wave");

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const i32x4* __restrict__ p, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t step = (int64_t)kProbeThreads * kProbeUnroll;
  int64_t i = (int64_t)blockIdx.x * step + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * step;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < n16; i += stride) {
    i32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = p[i + u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  }
  for (int u = 0; u < kProbeUnroll; ++u) {
    const int64_t j = i + u * kProbeThreads;
    if (j < n16) {
      const i32x4 v = p[j];
      acc ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  return launch_kernel(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0u, stream,
                       reinterpret_cast<const i32x4*>(p), bytes / 16, sink);
}

}  // namespace li
