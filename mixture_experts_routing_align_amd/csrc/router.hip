// Per-row router for gfx950: the step before the path (metrale
// forward_nvfp4_grouped_decode.rs, the decode layer's admission predicate: a
// BF16 softmax gate with no correction bias, computed by a router GEMV over
// the batch rows and a per-row top-k softmax, whose indices and weights feed
// the sort).
//
//   logits[t, e] = sum_h W[e, h] x[t, h]          (bf16 in, float32 accumulation)
//   ids[t, :]    = the top_k largest logits of row t, larger first, equal
//                  logits to the lower expert
//   wts[t, j]    = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the chosen i
//                  (the full softmax renormalised over its top k)
//
// Two launches.  The GEMV is a matrix-core tile product: a workgroup owns 16
// experts x 16 tokens (v_mfma_f32_16x16x32_bf16, weights as the A operand,
// tokens as B), its 16 waves split H in 128-deep rounds with both operands
// loaded straight from global memory, and their partial tiles are summed in a
// fixed order, so the logits do not depend on timing.
// The selection is one wave per token: each lane holds the logits of experts
// lane, lane + 64, ...; top_k rounds of a wave arg-max (ties to the lower
// expert) pick the experts, lane j keeps the j-th pick, and the softmax over
// the picks is one more wave reduction; the reductions run on the DPP lane
// crossbar.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace mma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;                            // experts (and tokens) per wave tile
constexpr int kLanesMax = MOE_MAX_EXPERTS / 64;      // logits per lane in the selection
constexpr int kKWaves = 16;                          // waves sharing one logits tile, split over H

// grid (ceil(E / 16), ceil(M / 16)) x kKWaves waves: every wave of a
// workgroup works on the same 16 experts x 16 tokens, wave w on the 128-deep
// rounds w, w + kKWaves, ... of H (the next round's loads go out before this
// one is multiplied); the waves' partial tiles meet in LDS and are summed in
// wave order.  Rows past E or M read the last row and store nothing.
__global__ __launch_bounds__(kKWaves * 64) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ w, int M, int H,
                                                                    int E, float* __restrict__ logits) {
  __shared__ f32x4 part[kKWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int et = blockIdx.x, tt = blockIdx.y;
  const int q = lane >> 4, r16 = lane & 15;
  const uint16_t* wr = w + (size_t)min(et * kTile + r16, E - 1) * H;
  const uint16_t* xr = x + (size_t)min(tt * kTile + r16, M - 1) * H;
  const int rounds = (H + 127) / 128;
  auto load = [&](int r, uint4 (&a)[4], uint4 (&b)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // lane's 8 consecutive k of step s (H is a multiple of 8: all in range or none)
      const int k = 128 * r + 32 * s + 8 * q;
      const int kk = min(k, H - 8);
      a[s] = *reinterpret_cast<const uint4*>(wr + kk);
      b[s] = *reinterpret_cast<const uint4*>(xr + kk);
      if (k >= H) a[s] = uint4{0u, 0u, 0u, 0u};
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint4 a[4], b[4], na[4], nb[4];
  if (wave < rounds) load(wave, a, b);
  for (int r = wave; r < rounds; r += kKWaves) {
    if (r + kKWaves < rounds) load(r + kKWaves, na, nb);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (128 * r + 32 * s < H) acc = mfma(as_bf16x8(a[s]), as_bf16x8(b[s]), acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = na[s];
      b[s] = nb[s];
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x < 256) {
    const int l = threadIdx.x & 63, i = threadIdx.x >> 6;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kKWaves; ++v) sum += part[v][l][i];
    const int t = tt * kTile + (l & 15), e = et * kTile + 4 * (l >> 4) + i;
    if (t < M && e < E) logits[(size_t)t * E + e] = sum;
  }
}

// (v, i) beats (ov, oi): larger logit, or equal logit and lower expert; i < 0: none
__device__ __forceinline__ bool beats(float ov, int oi, float v, int i) {
  return oi >= 0 && (i < 0 || ov > v || (ov == v && oi < i));
}

// Wave-wide reductions on the DPP lane crossbar (no LDS round trip): within
// quads (lane xor 1, xor 2), then the half-row and row mirrors, then the row
// broadcasts of lanes 15 and 31, which leave the whole wave's result in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = __int_as_float(dpp<CTRL, ROW_MASK>(__float_as_int(v)));
  const int oi = dpp<CTRL, ROW_MASK>(i);
  if (beats(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}
// the wave's best (value, expert), uniform across lanes
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<0xB1, 0xF>(v, i);   // quad_perm [1, 0, 3, 2]
  best_step<0x4E, 0xF>(v, i);   // quad_perm [2, 3, 0, 1]
  best_step<0x141, 0xF>(v, i);  // row_half_mirror
  best_step<0x140, 0xF>(v, i);  // row_mirror
  best_step<0x142, 0xA>(v, i);  // row_bcast:15 into rows 1 and 3
  best_step<0x143, 0xC>(v, i);  // row_bcast:31 into rows 2 and 3
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}
// the wave's sum, uniform across lanes (a fixed order)
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(dpp<0xB1, 0xF>(__float_as_int(v)));
  v += __int_as_float(dpp<0x4E, 0xF>(__float_as_int(v)));
  v += __int_as_float(dpp<0x141, 0xF>(__float_as_int(v)));
  v += __int_as_float(dpp<0x140, 0xF>(__float_as_int(v)));
  const float b15 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += b15;
  const float b31 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  v += b31;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// one wave per token
template <typename IdT>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(const float* __restrict__ logits, int M, int E,
                                                               int top_k, IdT* __restrict__ ids,
                                                               float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= M) return;
  const float* row = logits + (size_t)t * E;
  const int nent = (E + 63) / 64;
  float v[kLanesMax];
  uint32_t taken = 0;  // bit i: expert lane + 64 i chosen already, or past E
#pragma unroll
  for (int i = 0; i < kLanesMax; ++i) {
    if (i >= nent) break;
    const int e = lane + 64 * i;
    v[i] = row[min(e, E - 1)];  // all loads in flight at once; entries past E are marked taken
    if (e >= E) taken |= 1u << i;
  }
  float mine_v = 0.f, top = 0.f;
  int mine_i = 0;
  for (int k = 0; k < top_k; ++k) {
    // this lane's best untaken expert (ascending expert order, so ties keep the lower)
    float bv = 0.f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < kLanesMax; ++i) {
      if (i >= nent) break;  // uniform: only the entries E needs
      if (!((taken >> i) & 1u) && beats(v[i], lane + 64 * i, bv, bi)) {
        bv = v[i];
        bi = lane + 64 * i;
      }
    }
    wave_best(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (k == 0) top = bv;
    if (lane == k) {
      mine_v = bv;
      mine_i = bi;
    }
  }
  const float p = lane < top_k ? expf(mine_v - top) : 0.f;
  const float sum = wave_sum(p);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = (IdT)mine_i;
    wts[(size_t)t * top_k + lane] = p / sum;
  }
}

}  // namespace

hipError_t launch_router(const void* x, const void* w, int M, int H, int E, int top_k, float* logits, void* ids,
                         bool ids64, float* wts, hipStream_t s) {
  const dim3 g1((E + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  hipLaunchKernelGGL(router_logits_kernel, g1, dim3(kKWaves * 64), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w), M, H, E, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((M + kWaves - 1) / kWaves);
  if (ids64)
    hipLaunchKernelGGL(router_topk_kernel<int64_t>, g2, dim3(kThreads), 0, s, logits, M, E, top_k,
                       static_cast<int64_t*>(ids), wts);
  else
    hipLaunchKernelGGL(router_topk_kernel<int32_t>, g2, dim3(kThreads), 0, s, logits, M, E, top_k,
                       static_cast<int32_t*>(ids), wts);
  return hipGetLastError();
}

}  // namespace moe
