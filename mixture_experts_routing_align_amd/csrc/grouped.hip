// Public launchers of the grouped projections (kernels in grouped_impl.h, one
// translation unit per weight type and projection) and the weight tiling kernel.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mma_common.h"
#include "moe_internal.h"

namespace moe {

// defined in grouped_{gu,down}_{fp8,bf16,fp4}.hip
hipError_t launch_gate_up_fp8(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s);
hipError_t launch_gate_up_bf16(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s);
hipError_t launch_down_fp8(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s);
hipError_t launch_down_bf16(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s);
hipError_t launch_gate_up_fp4(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s);
hipError_t launch_down_fp4(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s);

namespace {

constexpr int kKC = 128;
constexpr int kWaveCols = 16;
constexpr int kMaxRowCap = 128;

__host__ __device__ constexpr int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Tiled weight layout: for each expert, 16-row tiles; inside a tile, 128-deep
// chunks (K zero-padded to a multiple of 128); inside a chunk, 1 KB fragments
// in which lane l of a wave finds, at byte 16*l, the 16 bytes it feeds the
// matrix core: row 16*t + l%16 at the k of k_of_step for quad l/16.
// MXFP4 (esz 0, K a multiple of 128): a chunk is 1 KB in two 512-byte halves;
// in half h lane l finds at byte 8*l the 8 bytes (16 codes) of row
// 16*t + l%16 at k = 128c + 64h + 16q .. +15, q = l/16, as they lie in the
// row-major row, so each 64-deep half of a tile is contiguous.
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                           int N, int K, int esz, size_t units) {
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte unit of the tiled output
  if (u >= units) return;
  if (esz == 0) {
    const size_t per_expert = (size_t)N * K / 2 / 16;
    const size_t e = u / per_expert;
    const size_t r = u % per_expert;
    const size_t block = r / 64;        // (tile, chunk) fragment of 1 KB
    const int within = (int)(r % 64);   // 16-byte unit inside it: lanes l0, l0 + 1 of half h
    const int h = within / 32, l0 = 2 * (within % 32);
    const int t = (int)(block / (K / kKC)), c = (int)(block % (K / kKC));
    uint2 out[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int l = l0 + i;
      const int row = t * kWaveCols + (l & 15), qd = l >> 4;
      out[i] = *reinterpret_cast<const uint2*>(src + (e * N + row) * (size_t)(K / 2) + c * (kKC / 2) + 32 * h + 8 * qd);
    }
    reinterpret_cast<uint4*>(dst)[u] = uint4{out[0].x, out[0].y, out[1].x, out[1].y};
    return;
  }
  const int kp = round_up(K, kKC);
  const size_t per_expert = (size_t)N * kp * esz / 16;
  const size_t e = u / per_expert;
  const size_t r = u % per_expert;
  const int per_chunk = kWaveCols * kKC * esz / 16;  // units in one tile chunk
  const size_t block = r / per_chunk;
  const int within = (int)(r % per_chunk);
  const int j = within / 64, l = within % 64;
  const int t = (int)(block / (kp / kKC)), c = (int)(block % (kp / kKC));
  const int row = t * kWaveCols + (l & 15), qd = l >> 4;
  const int kk = c * kKC + (esz == 1 ? j * 64 + qd * 16 : j * 32 + qd * 8);
  uint4 v = {0u, 0u, 0u, 0u};
  if (kk < K) v = *reinterpret_cast<const uint4*>(src + ((e * N + row) * (size_t)K + kk) * esz);
  reinterpret_cast<uint4*>(dst)[u] = v;
}

}  // namespace

int grouped_rows_per_pass(int64_t M) {
  int r = 4;
  while (r < M && r < kMaxRowCap) r <<= 1;
  return r;
}

int grouped_step_rows(int64_t M) { return std::min(grouped_rows_per_pass(M), 16); }

// an expert holds at most M rows when ids are distinct within a token (with
// repeated ids it can hold more, and gets more passes)
int grouped_passes(int64_t M) {
  const int r = grouped_step_rows(M);
  return (int)std::max<int64_t>(1, (M + r - 1) / r);
}

hipError_t launch_grouped_gate_up(const GroupedArgs& a, int fmt, bool tiled, hipStream_t s) {
  if (grouped_wide(fmt, a, true)) return launch_wide_gate_up(fmt, a, tiled, s);
  const int rowcap = grouped_step_rows(a.M);
  if (fmt == kFmtFP4) return launch_gate_up_fp4(a, rowcap, tiled, s);
  return fmt == kFmtFP8 ? launch_gate_up_fp8(a, rowcap, tiled, s) : launch_gate_up_bf16(a, rowcap, tiled, s);
}

hipError_t launch_grouped_down(const GroupedArgs& a, int fmt, bool tiled, hipStream_t s) {
  if (grouped_wide(fmt, a, false)) return launch_wide_down(fmt, a, tiled, s);
  const int rowcap = grouped_step_rows(a.M);
  if (fmt == kFmtFP4) return launch_down_fp4(a, rowcap, tiled, s);
  return fmt == kFmtFP8 ? launch_down_fp8(a, rowcap, tiled, s) : launch_down_bf16(a, rowcap, tiled, s);
}

size_t tiled_weight_bytes(int fmt, int64_t E, int N, int K) {
  const size_t elems = (size_t)E * N * round_up(K, kKC);
  return fmt == kFmtFP4 ? elems / 2 : elems * (fmt == kFmtFP8 ? 1 : 2);
}

hipError_t launch_tile_weights(const void* src, void* dst, int fmt, int64_t E, int N, int K, hipStream_t s) {
  const size_t units = tiled_weight_bytes(fmt, E, N, K) / 16;
  const size_t blocks = (units + 255) / 256;
  const int esz = fmt == kFmtFP4 ? 0 : (fmt == kFmtFP8 ? 1 : 2);
  hipLaunchKernelGGL(tile_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst), N, K, esz, units);
  return hipGetLastError();
}

}  // namespace moe
