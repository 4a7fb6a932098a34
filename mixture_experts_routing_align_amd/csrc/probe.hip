// Plain streaming-read kernel: the HBM read rate one launch reaches on a
// buffer of a given size, with none of the layer's work.  The layer kernels'
// weight-stream bandwidth is reported beside it, so a gap between the two is
// the layer's own cost and not the memory system's.
//
// The buffer is cut into 16 KB tiles (kUnroll 16-byte loads per thread, each
// load instruction of a wave covering 1 KB in one piece); workgroup b reads
// tiles b, b + blocks, ... with all of a tile's loads issued before any is
// used.  What it read is folded with XOR so the loads cannot be dropped, and
// each wave writes one 32-bit word.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t tile = (size_t)kThreads * kUnroll;
  uint32_t acc = 0;
  for (size_t t0 = (size_t)blockIdx.x * tile; t0 < n16; t0 += (size_t)gridDim.x * tile) {
    if (t0 + tile <= n16) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[t0 + u * kThreads + threadIdx.x];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {
      for (int u = 0; u < kUnroll; ++u) {
        const size_t i = t0 + u * kThreads + threadIdx.x;
        if (i < n16) {
          const uint4 v = src[i];
          acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
      }
    }
  }
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  stream_read_kernel<<<blocks, kThreads, 0, stream>>>(static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
