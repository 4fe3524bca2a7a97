// Read-only HBM stream: the floor that a weight-streaming kernel is measured
// against.  It reads a buffer once, 16 bytes per lane and eight loads in
// flight per lane, folds the words into one XOR per lane and stores nothing
// unless that XOR hits one fixed value (a data-dependent store keeps the
// loads alive).  It is no step of the FP8 path; the decode-batch GEMM and the
// MXFP8 linear, which stream a cold weight once per call, are timed against
// it on the same buffers.
#include <algorithm>

#include "common.hpp"

namespace mx {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;
constexpr uint32_t kStreamMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
  constexpr int64_t kBlockVec = int64_t(kStreamThreads) * kStreamUnroll;
  uint32_t acc = 0;
  for (int64_t base = int64_t(blockIdx.x) * kBlockVec + threadIdx.x; base < n16;
       base += int64_t(gridDim.x) * kBlockVec) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = base + int64_t(u) * kStreamThreads;
      v[u] = i < n16 ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kStreamMagic) sink[0] = acc;
}

}  // namespace

// One pass over `bytes` (a multiple of 16) at `src`: 32 KiB per workgroup,
// at most 2048 workgroups (8 per compute unit), the rest by grid stride.
mx_status launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return MX_OK;
  constexpr int64_t kBlockVec = int64_t(kStreamThreads) * kStreamUnroll;
  const int64_t blocks = std::min<int64_t>((n16 + kBlockVec - 1) / kBlockVec, 2048);
  stream_read_kernel<<<static_cast<unsigned>(blocks), kStreamThreads, 0, stream>>>(static_cast<const uint4*>(src), n16,
                                                                                   sink);
  return launch_status("mx_stream_read");
}

}  // namespace mx
