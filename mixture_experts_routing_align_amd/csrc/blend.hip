// Top-k blend for gfx950.
//
// out[t, h] = bf16( sum_{k=0..top_k-1, in order} w[t,k] * expert_out[token_to_perm[t*top_k+k], h]
//                   + gate_t * sh_out[t, h] )
// Restated from metrale fp8_moe_grouped.rs (moe_weighted_sum_blend_fp8_grouped:
// expert outputs are rows of sorted positions reached through token_to_perm; the
// shared expert's output is added ungated when no gate is given, and scaled by
// gate_t = sigmoid(x[t] . g) when its gate vector g is given) and nbxtensor
// moe_decode_vec.py (moe_part_reduce_kernel: the top-k sum in a constant order so
// the combine is deterministic).  The accumulation is a float32 fused
// multiply-add chain over k starting from 0, then + sh_out (ungated) or a fused
// multiply-add of gate_t and sh_out, then one round-to-nearest-even to bf16.  A token's bits depend only on its own inputs.
//
// Layout: one thread owns 4 consecutive hidden columns (16-byte loads of each
// expert row, an 8-byte store); grid = (ceil(H / 1024), min(M, 65535)), the
// y blocks striding over the tokens.  The expert rows a
// token reads are each contiguous, so every load is coalesced.
#include <hip/hip_runtime.h>

#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

using mma::bf16_rne_out;

__global__ __launch_bounds__(256) void blend_kernel(uint16_t* __restrict__ out,
                                                    const float* __restrict__ expert_out,
                                                    const float* __restrict__ w,
                                                    const int32_t* __restrict__ perm,
                                                    const float* __restrict__ sh_out,
                                                    const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ sh_gate, int M, int H,
                                                    int top_k) {
  __shared__ float red[256];
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  const bool gated = sh_out != nullptr && sh_gate != nullptr;
  for (int t = blockIdx.y; t < M; t += gridDim.y) {
  const float gate = gated ? mma::shared_gate256(x + (size_t)t * H, sh_gate, H, red) : 1.f;
  if (h >= H) continue;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  const size_t slot0 = (size_t)t * top_k;
  // kKB slots at a time: their positions and weights, then their rows, all
  // requested before the first is used; summed in k order
  constexpr int kKB = 8;
  for (int k0 = 0; k0 < top_k; k0 += kKB) {
    int pk[kKB];
    float wk[kKB];
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      const int k = min(k0 + j, top_k - 1);
      pk[j] = k0 + j < top_k ? perm[slot0 + k] : -1;
      wk[j] = w[slot0 + k];
    }
    float4 y[kKB];
#pragma unroll
    for (int j = 0; j < kKB; ++j)
      y[j] = *reinterpret_cast<const float4*>(expert_out + (size_t)(pk[j] < 0 ? 0 : pk[j]) * H + h);
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      if (pk[j] < 0) continue;
      a0 = fmaf(wk[j], y[j].x, a0);
      a1 = fmaf(wk[j], y[j].y, a1);
      a2 = fmaf(wk[j], y[j].z, a2);
      a3 = fmaf(wk[j], y[j].w, a3);
    }
  }
  if (sh_out != nullptr) {
    const float4 s = *reinterpret_cast<const float4*>(sh_out + (size_t)t * H + h);
    if (gated) {
      a0 = fmaf(gate, s.x, a0);
      a1 = fmaf(gate, s.y, a1);
      a2 = fmaf(gate, s.z, a2);
      a3 = fmaf(gate, s.w, a3);
    } else {
      a0 += s.x;
      a1 += s.y;
      a2 += s.z;
      a3 += s.w;
    }
  }
  uint2 packed;
  packed.x = bf16_rne_out(a0) | (bf16_rne_out(a1) << 16);
  packed.y = bf16_rne_out(a2) | (bf16_rne_out(a3) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * H + h) = packed;
  }
}

}  // namespace

hipError_t launch_blend(uint16_t* out, const float* expert_out, const float* w, const int32_t* perm,
                        const float* sh_out, const void* x, const void* sh_gate, int M, int H, int top_k,
                        hipStream_t s) {
  const dim3 grid((H / 4 + 255) / 256, M < 65535 ? M : 65535);
  hipLaunchKernelGGL(blend_kernel, grid, dim3(256), 0, s, out, expert_out, w, perm, sh_out,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(sh_gate), M, H, top_k);
  return hipGetLastError();
}

}  // namespace moe
