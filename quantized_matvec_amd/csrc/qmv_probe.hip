// Streaming-read probe: a plain 128-bit read over a large buffer, the
// measured read ceiling that the bandwidth-bound kernels are compared with.
#include <algorithm>

#include "qmv_launch.hpp"

namespace qmv {

constexpr int kProbeThreads = 256;

// Every 16-byte chunk is read once (grid-stride, consecutive lanes on
// consecutive chunks); a wave XORs its words together and one lane folds
// the result into *sink with an atomic, so the loads cannot be dropped.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                                    int64_t n16,
                                                                    uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d);
  if ((threadIdx.x & 63) == 0 && acc != 0) atomicXor(sink, acc);
}

hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  int64_t grid = 4 * (int64_t)device_cu_count();
  grid = std::min<int64_t>(grid, (n16 + kProbeThreads - 1) / kProbeThreads);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, st,
                     static_cast<const uint4 *>(p), n16, sink);
  return hipGetLastError();
}

}  // namespace qmv
