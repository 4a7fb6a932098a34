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
// Two launches: the logits, a workgroup per 16 experts x 16 tokens whose 16
// waves split H in interleaved 128-deep rounds with both operands loaded
// straight from global memory, partial tiles summed in wave order; then the
// selection, one wave per token.  (Handing the logits to the last workgroup
// of the first launch instead, through a counter, measured slower: the
// hand-off's dependent memory round trips cost more than the launch.)
// The tile product is on the matrix cores (v_mfma_f32_16x16x32_bf16, weights as
// the A operand, tokens as B) with a fixed summation order, so the logits do not
// depend on timing.
// The selection is one wave per token: each lane holds the logits of experts
// lane, lane + 64, ... (loaded at once), as 64-bit keys that order them the
// way the choice does; top_k rounds of a wave maximum pick the experts, lane j
// keeps the j-th pick, and the softmax over the picks is one more wave
// reduction; the reductions run on the DPP lane crossbar.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace mma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;                            // experts (and tokens) per wave tile
constexpr int kLanesMax = MOE_MAX_EXPERTS / 64;      // most logits per lane in the selection
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

// A logit and its expert as one 64-bit key whose unsigned order is the
// choice's: the high word is the logit's bits made monotone (negative values
// inverted, positive ones with the sign bit set; -0 taken as +0, so equal
// logits compare equal), the low word the inverted expert, so equal logits go
// to the lower expert.  0 is below every key and marks an entry out of play.
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ bool key_above(uint32_t ah, uint32_t al, uint32_t bh, uint32_t bl) {
  return (((uint64_t)ah << 32) | al) > (((uint64_t)bh << 32) | bl);
}

// Wave-wide reductions on the DPP lane crossbar (no LDS round trip): within
// quads (lane xor 1, xor 2), then the half-row and row mirrors, then the row
// broadcasts of lanes 15 and 31, which leave the whole wave's result in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
// (a lane that the move does not write gets key 0, which never wins)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void max_step(uint32_t& h, uint32_t& l) {
  const uint32_t oh = __builtin_amdgcn_update_dpp(0u, h, CTRL, ROW_MASK, 0xF, false);
  const uint32_t ol = __builtin_amdgcn_update_dpp(0u, l, CTRL, ROW_MASK, 0xF, false);
  if (key_above(oh, ol, h, l)) {
    h = oh;
    l = ol;
  }
}
// the wave's largest key, uniform across lanes
__device__ __forceinline__ void wave_max(uint32_t& h, uint32_t& l) {
  max_step<0xB1, 0xF>(h, l);   // quad_perm [1, 0, 3, 2]
  max_step<0x4E, 0xF>(h, l);   // quad_perm [2, 3, 0, 1]
  max_step<0x141, 0xF>(h, l);  // row_half_mirror
  max_step<0x140, 0xF>(h, l);  // row_mirror
  max_step<0x142, 0xA>(h, l);  // row_bcast:15 into rows 1 and 3
  max_step<0x143, 0xC>(h, l);  // row_bcast:31 into rows 2 and 3
  h = __builtin_amdgcn_readlane(h, 63);
  l = __builtin_amdgcn_readlane(l, 63);
}
// the wave's sum, uniform across lanes (a fixed order)
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp<0xB1, 0xF>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x4E, 0xF>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x141, 0xF>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x140, 0xF>(__float_as_uint(v)));
  const float b15 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += b15;
  const float b31 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  v += b31;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One wave selects token t's top_k from its logits row: each lane holds the
// keys of experts lane, lane + 64, ... (NENT entries, a power of two at least
// ceil(E / 64), all loaded unconditionally, clamped into the row, so every load
// is in flight at once); top_k rounds of a wave maximum pick the experts, lane
// j keeps the j-th pick, and the softmax over the picks is one more wave
// reduction.
template <typename IdT, int NENT>
__device__ __forceinline__ void select_topk(const float* __restrict__ row, int t, int E, int top_k,
                                            IdT* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  float v[NENT];
  uint32_t kh[NENT], kl[NENT];  // entry i: expert lane + 64 i (key 0: chosen already, or past E)
#pragma unroll
  for (int i = 0; i < NENT; ++i) {
    const int e = lane + 64 * i;
    v[i] = row[min(e, E - 1)];  // all loads in flight at once
  }
#pragma unroll
  for (int i = 0; i < NENT; ++i) {
    const int e = lane + 64 * i;
    kh[i] = e < E ? order_bits(v[i]) : 0u;
    kl[i] = e < E ? ~(uint32_t)e : 0u;
  }
  float mine_v = 0.f, top = 0.f;
  int mine_i = 0;
  for (int k = 0; k < top_k; ++k) {
    // this lane's largest key, then the wave's
    uint32_t bh = kh[0], bl = kl[0];
#pragma unroll
    for (int i = 1; i < NENT; ++i)
      if (key_above(kh[i], kl[i], bh, bl)) {
        bh = kh[i];
        bl = kl[i];
      }
    wave_max(bh, bl);
    // the winner leaves play (the low word names one expert, so one entry matches)
#pragma unroll
    for (int i = 0; i < NENT; ++i)
      if (kl[i] == bl) kh[i] = kl[i] = 0u;
    const float bv = order_value(bh);
    if (k == 0) top = bv;
    if (lane == k) {
      mine_v = bv;
      mine_i = (int)~bl;
    }
  }
  const float p = lane < top_k ? expf(mine_v - top) : 0.f;
  const float sum = wave_sum(p);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = (IdT)mine_i;
    wts[(size_t)t * top_k + lane] = p / sum;
  }
}

// one wave per token
template <typename IdT, int NENT>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(const float* __restrict__ logits, int M, int E,
                                                               int top_k, IdT* __restrict__ ids,
                                                               float* __restrict__ wts) {
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= M) return;
  select_topk<IdT, NENT>(logits + (size_t)t * E, t, E, top_k, ids, wts);
}

}  // namespace

namespace {

// the selection's entries per lane for E experts: ceil(E / 64) rounded up to a
// power of two
template <typename F>
void with_nent(int E, F&& f) {
  static_assert(kLanesMax == 16, "entries per lane: 1, 2, 4, 8 or 16");
  if (E <= 64) f(std::integral_constant<int, 1>{});
  else if (E <= 128) f(std::integral_constant<int, 2>{});
  else if (E <= 256) f(std::integral_constant<int, 4>{});
  else if (E <= 512) f(std::integral_constant<int, 8>{});
  else f(std::integral_constant<int, 16>{});
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
  with_nent(E, [&](auto n) {
    constexpr int N = decltype(n)::value;
    if (ids64)
      hipLaunchKernelGGL((router_topk_kernel<int64_t, N>), g2, dim3(kThreads), 0, s, logits, M, E, top_k,
                         static_cast<int64_t*>(ids), wts);
    else
      hipLaunchKernelGGL((router_topk_kernel<int32_t, N>), g2, dim3(kThreads), 0, s, logits, M, E, top_k,
                         static_cast<int32_t*>(ids), wts);
  });
  return hipGetLastError();
}

}  // namespace moe
