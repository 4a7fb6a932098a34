// Grouped expert projections for gfx950: gate+up with SiLU, and down.
//
// What is computed (metrale fp8_moe_grouped.rs: module doc, and the gate+up and
// down launchers' docs; nbxtensor moe_decode_vec.py: the SwiGLU epilogue):
//   gate+up: act[p, c] = silu(g) * u, g = sum_k Wg[e][c][k] x[t][k],
//            u = sum_k Wu[e][c][k] x[t][k], for each sorted position p holding a
//            slot of active expert e (t = slot / top_k); the shared expert does
//            the same for every token t into sh_act[t, c].
//   down:    out[p, c] = sum_k Wd[e][c][k] act[p][k] (shared: rows are tokens).
// A workgroup owns one active expert (or one group of shared-expert rows) and a
// 64-column tile of the output, and applies each weight row it streams from HBM
// to every row routed to that expert, so each expert's weights are read once
// per pass.  Rows of the intermediates are sorted positions.
//
// gfx950 design (not the pages' CUDA geometry):
//  * Matrix cores: v_mfma_f32_16x16x32_bf16.  The weights are the A operand
//    (16 output columns per wave), the expert's rows the B operand (16-row
//    tiles, zero-padded).  FP8 e4m3 codes convert exactly to bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp8, scale 1); bf16 activations are exact, so the
//    only rounding is the float32 accumulation.  Each 128-deep FP8 scale block
//    is accumulated alone and then multiplied by its scale.  The down
//    projection's float32 input is split into bf16 hi + lo and both halves go
//    through the matrix core, so it keeps ~16 bits of the input's mantissa.
//  * Memory: each lane streams 16-byte (dwordx4) loads of its weight row; one
//    128-deep chunk ahead is kept in flight in registers while the current one
//    is multiplied.  The rows' activations for the current chunk are staged in
//    LDS once per workgroup (row stride padded by 16 bytes against bank
//    conflicts) and read as B operands by all four waves.
//  * Row invariance: a row's value depends only on its own inputs: every output
//    element is the same sequence of MFMA k-steps, scale FMAs and chunk sums
//    whatever tile, slot or pass the row occupies, and the number of rows per
//    pass comes from the shape class, never from the routing.
//  * Graph replay: the grid is (ceil(N/64), cap + shared row groups), sized from
//    shapes only; a workgroup past the device-side active count exits at once.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 wave64 per workgroup
constexpr int kWaveCols = 16;   // output columns per wave: one MFMA tile edge
constexpr int kTileCols = 64;   // output columns per workgroup
constexpr int kKC = 128;        // depth of one chunk (= one FP8 scale block)
constexpr int kLdsRow = kKC + 8;  // bf16 elements per staged row (+16 B pad)

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 8 FP8 e4m3 codes (two dwords, lowest byte first) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t d0, uint32_t d1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Element offset, inside a 128-deep chunk, of the 8 consecutive k a lane of
// quad q feeds to MFMA step s.  The A and B operands use the same map, so the
// k order inside one MFMA is a permutation the product does not see.
//  FP8: one 16-byte load holds 16 codes = steps s and s+1 (s even).
//  BF16: one 16-byte load holds 8 elements = one step.
template <bool FP8>
__device__ __forceinline__ int k_of_step(int s, int q) {
  return FP8 ? ((s >> 1) * 64 + q * 16 + (s & 1) * 8) : (s * 32 + q * 8);
}

template <bool FP8, bool GATE_UP, int RT>
__global__ __launch_bounds__(kThreads) void grouped_kernel(GroupedArgs p) {
  constexpr int NS = GATE_UP ? 2 : 1;   // weight streams (gate, up) or (down)
  constexpr int NX = GATE_UP ? 1 : 2;   // B planes: bf16 x, or bf16 hi + lo of act
  constexpr int ROWS = RT * 16;
  constexpr int WL = FP8 ? 2 : 4;       // 16-byte weight loads per lane per chunk
  constexpr int XL = GATE_UP ? RT : 2 * RT;  // 16-byte activation loads per thread per chunk
  constexpr int ESZ = FP8 ? 1 : 2;      // weight element bytes

  __shared__ __attribute__((aligned(16))) uint16_t xs[NX][ROWS][kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int by = blockIdx.y;

  // ---- which expert / rows this workgroup serves
  const bool routed = by < p.cap;
  int e = 0, rows, row_base, N, K;
  const char *W0, *W1 = nullptr;
  const float *S0 = nullptr, *S1 = nullptr;
  const char* X;
  float* OUT;
  if (routed) {
    if (by >= *p.active_count) return;
    e = p.active_experts[by];
    rows = p.expert_counts[e];
    row_base = p.expert_offsets[e];
    N = p.N;
    K = p.K;
    const size_t wstride = (size_t)N * K * ESZ;
    W0 = static_cast<const char*>(p.w0) + (size_t)e * wstride;
    if (GATE_UP) W1 = static_cast<const char*>(p.w1) + (size_t)e * wstride;
    if (FP8) {
      const size_t sstride = (size_t)(N / kFp8Block) * (K / kFp8Block);
      S0 = p.s0 + (size_t)e * sstride;
      if (GATE_UP) S1 = p.s1 + (size_t)e * sstride;
    }
    X = static_cast<const char*>(p.x);
    OUT = p.out;
  } else {
    const int g = by - p.cap;
    row_base = g * ROWS;
    rows = min(ROWS, p.M - row_base);
    N = p.sN;
    K = p.sK;
    W0 = static_cast<const char*>(p.sw0);
    W1 = static_cast<const char*>(p.sw1);
    S0 = p.ss0;
    S1 = p.ss1;
    X = static_cast<const char*>(p.sx);
    OUT = p.sout;
  }
  const int col0 = blockIdx.x * kTileCols;
  if (col0 >= N || rows <= 0) return;
  const int wcol = col0 + wave * kWaveCols;
  const bool wave_on = wcol < N;
  const int kblocks = K / kFp8Block;
  const float* S0w = FP8 ? S0 + (size_t)(wcol / kFp8Block) * kblocks : nullptr;
  const float* S1w = (FP8 && GATE_UP) ? S1 + (size_t)(wcol / kFp8Block) * kblocks : nullptr;
  // this lane's weight row (A operand row r16 of the wave's tile)
  const char* wrow0 = W0 + (size_t)(wcol + r16) * K * ESZ;
  const char* wrow1 = GATE_UP ? W1 + (size_t)(wcol + r16) * K * ESZ : nullptr;

  for (int r0 = 0; r0 < rows; r0 += ROWS) {
    const int nr = min(ROWS, rows - r0);
    const int nrt = (nr + 15) >> 4;

    // ---- activation rows this thread stages (source row index or -1)
    // gate+up: ROWS x 128 bf16 = 16 pieces of 16 B per row; down: 32 per row (fp32)
    constexpr int PIECES = GATE_UP ? 16 : 32;
    constexpr int ROW_STEP = kThreads / PIECES;
    const int piece = tid % PIECES, prow = tid / PIECES;
    int src[XL];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int r = prow + j * ROW_STEP;
      int s = -1;
      if (r < nr) {
        if (!routed)
          s = row_base + r0 + r;  // token
        else if (GATE_UP)
          s = p.sorted_token_ids[row_base + r0 + r] / p.top_k;  // token of the slot
        else
          s = row_base + r0 + r;  // sorted position
      }
      src[j] = s;
    }

    auto load_x = [&](uint4 (&xr)[XL], int k0) {
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        uint4 v = {0u, 0u, 0u, 0u};
        if (GATE_UP) {
          const int kk = k0 + piece * 8;
          if (src[j] >= 0 && kk < K)
            v = *reinterpret_cast<const uint4*>(X + ((size_t)src[j] * K + kk) * 2);
        } else {
          const int kk = k0 + piece * 4;
          if (src[j] >= 0 && kk < K)
            v = *reinterpret_cast<const uint4*>(X + ((size_t)src[j] * K + kk) * 4);
        }
        xr[j] = v;
      }
    };
    auto store_x = [&](const uint4 (&xr)[XL]) {
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        const int r = prow + j * ROW_STEP;
        if (GATE_UP) {
          *reinterpret_cast<uint4*>(&xs[0][r][piece * 8]) = xr[j];
        } else {
          const float f[4] = {__uint_as_float(xr[j].x), __uint_as_float(xr[j].y),
                              __uint_as_float(xr[j].z), __uint_as_float(xr[j].w)};
          uint16_t hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hi[i] = bf16_rne_bits(f[i]);
            lo[i] = bf16_rne_bits(f[i] - bf16_bits_to_f32(hi[i]));
          }
          uint2 h2, l2;
          h2.x = hi[0] | ((uint32_t)hi[1] << 16);
          h2.y = hi[2] | ((uint32_t)hi[3] << 16);
          l2.x = lo[0] | ((uint32_t)lo[1] << 16);
          l2.y = lo[2] | ((uint32_t)lo[3] << 16);
          *reinterpret_cast<uint2*>(&xs[0][r][piece * 4]) = h2;
          *reinterpret_cast<uint2*>(&xs[NX - 1][r][piece * 4]) = l2;
        }
      }
    };
    auto load_w = [&](uint4 (&wr)[NS][WL], int k0) {
#pragma unroll
      for (int j = 0; j < WL; ++j) {
        const int kk = k0 + k_of_step<FP8>(FP8 ? 2 * j : j, q);
        const bool ok = wave_on && kk < K;
        wr[0][j] = ok ? *reinterpret_cast<const uint4*>(wrow0 + (size_t)kk * ESZ) : uint4{0u, 0u, 0u, 0u};
        if (GATE_UP)
          wr[NS - 1][j] = ok ? *reinterpret_cast<const uint4*>(wrow1 + (size_t)kk * ESZ) : uint4{0u, 0u, 0u, 0u};
      }
    };

    f32x4 acc[NS][RT];
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[st][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 wcur[NS][WL], wnxt[NS][WL];
    uint4 xr[XL];
    load_w(wcur, 0);
    load_x(xr, 0);

    for (int k0 = 0; k0 < K; k0 += kKC) {
      __syncthreads();  // every wave is done reading the previous chunk
      store_x(xr);
      __syncthreads();
      const bool more = k0 + kKC < K;
      if (more) {
        load_w(wnxt, k0 + kKC);
        load_x(xr, k0 + kKC);
      }
      if (wave_on) {
        // A operands of the 4 k-steps of this chunk
        bf16x8 a[NS][4];
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (FP8) {
              const uint4 v = wcur[st][s >> 1];
              a[st][s] = (s & 1) ? fp8x8_to_bf16(v.z, v.w) : fp8x8_to_bf16(v.x, v.y);
            } else {
              a[st][s] = as_bf16x8(wcur[st][s]);
            }
          }
        float sc[NS];
        if (FP8) {
          sc[0] = S0w[k0 / kFp8Block];
          if (GATE_UP) sc[NS - 1] = S1w[k0 / kFp8Block];
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (rt < nrt) {
            bf16x8 b[NX][4];
#pragma unroll
            for (int x = 0; x < NX; ++x)
#pragma unroll
              for (int s = 0; s < 4; ++s)
                b[x][s] = as_bf16x8(
                    *reinterpret_cast<const uint4*>(&xs[x][rt * 16 + r16][k_of_step<FP8>(s, q)]));
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              if (FP8) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                  for (int x = 0; x < NX; ++x) t = mfma(a[st][s], b[x][s], t);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[st][rt][i] = fmaf(sc[st], t[i], acc[st][rt][i]);
              } else {
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                  for (int x = 0; x < NX; ++x) acc[st][rt] = mfma(a[st][s], b[x][s], acc[st][rt]);
              }
            }
          }
        }
      }
      if (more) {
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int j = 0; j < WL; ++j) wcur[st][j] = wnxt[st][j];
      }
    }

    // ---- epilogue: lane holds columns wcol + 4q .. +3 of tile row r16
    if (wave_on) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = rt * 16 + r16;
        if (rt < nrt && r < nr) {
          float4 v;
          if (GATE_UP) {
            const f32x4 g = acc[0][rt], u = acc[NS - 1][rt];
            v.x = g[0] / (1.0f + expf(-g[0])) * u[0];
            v.y = g[1] / (1.0f + expf(-g[1])) * u[1];
            v.z = g[2] / (1.0f + expf(-g[2])) * u[2];
            v.w = g[3] / (1.0f + expf(-g[3])) * u[3];
          } else {
            v.x = acc[0][rt][0];
            v.y = acc[0][rt][1];
            v.z = acc[0][rt][2];
            v.w = acc[0][rt][3];
          }
          *reinterpret_cast<float4*>(OUT + (size_t)(row_base + r0 + r) * N + wcol + 4 * q) = v;
        }
      }
    }
  }
}

template <bool FP8, bool GATE_UP>
hipError_t launch(const GroupedArgs& a, int rt, hipStream_t s) {
  const int nmax = (a.sw0 != nullptr && a.sN > a.N) ? a.sN : a.N;
  const int rows = rt * 16;
  const int shared_groups = a.sw0 != nullptr ? (a.M + rows - 1) / rows : 0;
  const dim3 grid((nmax + kTileCols - 1) / kTileCols, a.cap + shared_groups);
  const dim3 block(kThreads);
  switch (rt) {
    case 1: hipLaunchKernelGGL((grouped_kernel<FP8, GATE_UP, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((grouped_kernel<FP8, GATE_UP, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((grouped_kernel<FP8, GATE_UP, 4>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((grouped_kernel<FP8, GATE_UP, 8>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

int grouped_row_tiles(int64_t M, int top_k) {
  (void)top_k;
  // with ids distinct within a token an expert holds at most M rows
  if (M <= 16) return 1;
  if (M <= 32) return 2;
  if (M <= 64) return 4;
  return 8;
}

hipError_t launch_grouped_gate_up(const GroupedArgs& a, bool fp8, int row_tiles, hipStream_t s) {
  return fp8 ? launch<true, true>(a, row_tiles, s) : launch<false, true>(a, row_tiles, s);
}

hipError_t launch_grouped_down(const GroupedArgs& a, bool fp8, int row_tiles, hipStream_t s) {
  return fp8 ? launch<true, false>(a, row_tiles, s) : launch<false, false>(a, row_tiles, s);
}

}  // namespace moe
