// Plain streaming-read kernel: the HBM read rate one launch reaches on a
// buffer of a given size, with none of the layer's work.  The layer kernels'
// weight-stream bandwidth is reported beside it, so a gap between the two is
// the layer's own cost and not the memory system's.
//
// Each thread issues kUnroll independent 16-byte loads per round over a
// grid-stride walk (consecutive lanes on consecutive 16-byte pieces), folds
// what it read with XOR so the loads cannot be dropped, and each wave writes
// one 32-bit word.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
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
