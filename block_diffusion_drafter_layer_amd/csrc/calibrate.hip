// Measurement references (not part of the method).
//
// copy_bytes: a plain device copy with the memory access shape of the weight
// streams: 16-byte vector loads and stores, one contiguous kilobyte per wave
// instruction, four independent loads in flight per lane. It is the
// reference whose hardware byte counters calibrate the traffic figures of
// the other kernels (the counters' scale depends on the request sizes, so
// the reference must issue the same kind of requests).
//
// read_bytes: the read ceiling of the weight streams' own access pattern -
// the streaming GEMM's loads without its arithmetic: one workgroup per CU,
// four waves, each streaming 512-byte pieces of 16 rows of 8 KB straight
// into a ring of three 8 KB LDS slots per wave with the non-temporal hint,
// two slots in flight. Nothing is computed; a word of each slot is folded
// into a value that is stored only if it equals an impossible constant.
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

constexpr int kReadRing = 3;
constexpr int kReadRow = 8192;    // bytes per row
constexpr int kReadTile = 16;     // rows per tile
constexpr int kReadPiece = 512;   // bytes of a row per load instruction pair

__global__ void __launch_bounds__(256)
read_bytes(const uint8_t* __restrict__ src, size_t rows, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][kReadRing][kReadTile * kReadPiece];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t gw = (size_t)blockIdx.x * 4 + w, W = (size_t)gridDim.x * 4;
  constexpr int kPieces = kReadRow / kReadPiece;
  const size_t items = rows / kReadTile * kPieces;
  const size_t n_items = gw < items ? (items - gw + W - 1) / W : 0;
  auto issue = [&](size_t t) {
    const size_t it = gw + t * W;
    const size_t tile = it / kPieces, piece = it % kPieces;
    uint8_t* slot = &ring[w][t % kReadRing][0];
    const int hi = lane >> 5, pos = lane & 31;
#pragma unroll
    for (int q = 0; q < kReadTile / 2; ++q) {
      const size_t r = tile * kReadTile + 2 * q + hi;
      dma16_nt(src + r * kReadRow + piece * kReadPiece + pos * 16, slot + q * 1024);
    }
  };
  const size_t pre = n_items < kReadRing - 1 ? n_items : kReadRing - 1;
  for (size_t t = 0; t < pre; ++t) issue(t);
  uint32_t acc = 0;
  for (size_t t = 0; t < n_items; ++t) {
    if (t + kReadRing - 1 < n_items) {
      issue(t + kReadRing - 1);
      __builtin_amdgcn_s_waitcnt(((8 * (kReadRing - 1)) & 15) | (((8 * (kReadRing - 1)) >> 4) << 14) | 0xF70);
    } else {
      __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    }
    acc ^= *reinterpret_cast<volatile uint32_t*>(&ring[w][t % kReadRing][lane * 4]);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // no load still writing the ring at exit
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 255] = acc;
}

hipError_t launch_read_bytes(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t rows = bytes / kReadRow;
  if (!rows) return hipSuccess;
  hipLaunchKernelGGL(read_bytes, dim3(256), dim3(256), 0, st, (const uint8_t*)src, rows, sink);
  return hipGetLastError();
}

}  // namespace dfl
