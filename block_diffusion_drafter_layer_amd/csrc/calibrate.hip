// A plain device copy with the memory access shape of the weight streams:
// 16-byte vector loads and stores, one contiguous kilobyte per wave
// instruction, four independent loads in flight per lane. It is the
// reference whose hardware byte counters calibrate the traffic figures of
// the other kernels (the counters' scale depends on the request sizes, so
// the reference must issue the same kind of requests).
#include "common.h"
#include "launch.h"

namespace dfl {

__global__ void __launch_bounds__(256)
copy_bytes(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256 * 4;
  for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + 256 * u < n16 ? src[i + 256 * u] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 256 * u < n16) dst[i + 256 * u] = v[u];
  }
}

hipError_t launch_copy_bytes(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t blocks = std::min<size_t>(4096, (n16 + 1023) / 1024);
  if (!blocks) return hipSuccess;
  hipLaunchKernelGGL(copy_bytes, dim3((unsigned)blocks), dim3(256), 0, st, (u32x4*)dst,
                     (const u32x4*)src, n16);
  return hipGetLastError();
}

}  // namespace dfl
