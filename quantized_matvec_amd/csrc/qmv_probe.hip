// Streaming-read probe: a plain 128-bit read over a large buffer, the
// measured read ceiling that the bandwidth-bound kernels are compared with.
#include <algorithm>

#include "qmv_launch.hpp"

namespace qmv {

constexpr int kProbeThreads = 256;

constexpr int kProbeMaxGrid = 1024;  // workgroups, one sink word each

// Every 16-byte chunk is read once (grid-stride, consecutive lanes on
// consecutive chunks); the workgroup XORs its words together and XORs the
// result into its own sink word (a plain read-modify-write: no atomics, which
// would serialise on one address at the end of the pass).
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                                    int64_t n16,
                                                                    uint32_t *__restrict__ sink) {
  __shared__ uint32_t part[kProbeThreads / 64];
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
    for (int i = 0; i < kProbeThreads / 64; ++i) w ^= part[i];
    sink[blockIdx.x] ^= w;
  }
}

// Up to 32 MB every thread reads one chunk (all loads in flight at once,
// which reads a buffer of that size fastest; at most 8192 workgroups, one
// sink word each); beyond, at most 1024 workgroups stride over the buffer
// (the faster form for gigabytes).
constexpr int64_t kProbeOnePassChunks = int64_t(1) << 21;

hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  int64_t grid = std::min<int64_t>(4 * (int64_t)device_cu_count(), kProbeMaxGrid);
  if (n16 <= kProbeOnePassChunks) grid = n16;  // then divided by the threads per workgroup
  grid = std::min<int64_t>(grid, (n16 + kProbeThreads - 1) / kProbeThreads);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, st,
                     static_cast<const uint4 *>(p), n16, sink);
  return hipGetLastError();
}

}  // namespace qmv
