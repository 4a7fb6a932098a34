// Wide-pass grouped projections for gfx950: every row an expert holds, 32 at
// a time, in one workgroup per (expert pass, column group), so an expert's
// weights are streamed once per column group per 32 rows instead of once per
// 16-row pass.  For layers whose experts hold many rows (verify and prefill
// widths); FP8 weights (block or row scales) or MXFP4, tiled or row-major.
//
// What is computed is the grouped projection of the pass kernels
// (grouped_impl.h; metrale fp8_moe_grouped.rs: the gate+up and down launchers;
// nbxtensor moe_decode_vec.py: the SwiGLU epilogue), with the same arithmetic
// for every output element:
//   gate+up: FP8: per 128-deep chunk c (one scale block), t = the chunk's 4
//            MFMA steps from zero, acc = fma(scale_c, t, acc), c ascending;
//            MXFP4: the codes decoded with their 32-deep block's power-of-two
//            scale (exact in bf16), every MFMA step straight into acc;
//            act = silu(g) * u
//   down:    per 64-deep half h, t = its 2 MFMA steps over bf16 hi then lo of
//            act, from zero; acc = acc + scale * t (FP8; MXFP4: acc + t), each
//            operation rounded, h ascending
// so a row has the same bits whichever kernel (or layer path) runs it.
//
// gfx950 design.  4 waves.  Each wave streams its own weight rows (16 gate
// and 16 up columns; or 4 x 16 rows of the down output) from HBM into a
// register ring (gate+up: 3 steps, 4 workgroups per compute unit at 128
// registers a lane; down: 4 steps, 3 workgroups per compute unit), 16-byte
// buffer loads, no LDS.  The rows' activations (bf16 x, or act split into
// bf16 hi + lo) are shared by the 4 waves through two LDS slots: each thread
// requests its pieces of the rows two steps ahead into registers and writes
// them to LDS one step ahead, with one barrier per step.  Rows and tiles past
// an expert's count or the output, and the steps that pad the depth to whole
// loop rounds, fetch nothing (buffer loads past the buffer's end return zeros)
// and change no stored output.  The shared expert's units are narrower than
// the routed ones (its depth S makes them longer), so that no unit holds the
// launch up.  No register spills.
#include <hip/hip_runtime.h>

#include <climits>

#include "align_device.h"
#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace wide_detail {

using namespace mma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// rows per pass: routed passes of an expert, shared-expert passes of tokens
constexpr int kGuRows = 32, kGuShRows = 32;              // gate+up
constexpr int kDnRows = 32, kDnShRows = 32;              // down
static_assert(kGuShRows <= kGuRows && kDnShRows <= kDnRows, "a shared pass fits the routed pass registers");
constexpr int kGuCols = kWaves * kWaveCols;              // gate+up columns per workgroup
constexpr int kDnTiles = 4;                              // down: 16-row output tiles per wave (at most 4)
constexpr int kDnOcc = 3;                                // down: workgroups per compute unit
constexpr int kDnCols = kWaves * kDnTiles * kWaveCols;   // down output rows (of H) per routed workgroup
constexpr int kDnShCols = kWaves * kWaveCols;            // per shared-expert workgroup (one tile per wave)
constexpr int kGuRing = 3;                               // gate+up: weight steps in the register ring (2 ahead)
constexpr int kMaxScaleBlocks = 128;                     // FP8 depth limit: 128 scale blocks
constexpr int kSL = kMaxScaleBlocks / 64;
constexpr int kXStride = kKC + kPad;                     // staged x row, bf16 elements (one chunk)
constexpr size_t kGuLds = (size_t)2 * kGuRows * kXStride * 2;    // two slots
// 16-byte row pieces each thread stages per step (rows u*16 + tid/16)
template <int RP>
constexpr int pieces_of() {
  static_assert(RP * 16 % kThreads == 0, "whole pieces per thread");
  return RP * 16 / kThreads;
}
// 16 bytes as a native vector: a register copy, where the uint4 struct would
// be copied through private memory
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Staged rows and the down weights are read with buffer loads: a load whose
// offset lies past the resource's size returns zeros and fetches nothing, so
// rows past an expert's count (and a wave's tiles past the output) cost no
// memory traffic and need no branch around their loads.
constexpr uint32_t kNoFetch = 0x80000000u;  // past every resource this file builds (each < 2^31 bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// MXFP4: copy n consecutive scale dwords (a workgroup's weight rows, K / 128
// dwords each) from src to LDS, every load of a round issued before its
// stores.  No barrier.
constexpr int kStageJ = 8, kStageRound = kStageJ * kThreads;
__device__ __forceinline__ void stage_scales(uint32_t* __restrict__ dst, const void* src, int n) {
  const __amdgpu_buffer_rsrc_t r = rsrc(src, (uint32_t)n * 4);
  for (int b0 = 0; b0 < n; b0 += kStageRound) {
    uint32_t v[kStageJ];
#pragma unroll
    for (int j = 0; j < kStageJ; ++j) v[j] = bload4(r, (uint32_t)(b0 + j * kThreads + (int)threadIdx.x) * 4);
#pragma unroll
    for (int j = 0; j < kStageJ; ++j) {
      const int i = b0 + j * kThreads + (int)threadIdx.x;
      if (i < n) dst[i] = v[j];
    }
  }
}

// Which pass routed item j is: the active experts in ascending order, each
// contributing ceil(count / RP) passes.  Every thread takes a run of active
// indices, a block scan of their pass counts places the runs, and the thread
// whose run holds pass j publishes (expert, first row, count, offset).
// e = -1: the routing has fewer passes.  Contains barriers.
struct Pass {
  int e, r0, count, offset;
};
template <int RP>
__device__ __forceinline__ Pass locate_pass(const GroupedArgs& p, int j, int* s_item) {
  constexpr int kPer = (MOE_MAX_EXPERTS + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  const int per = (p.cap + kThreads - 1) / kThreads;
  const int a0 = min(p.cap, tid * per);
  int ex[kPer], cn[kPer], np = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) ex[i] = (i < per && a0 + i < p.cap) ? p.active_experts[a0 + i] : -1;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    cn[i] = ex[i] >= 0 ? p.expert_counts[ex[i]] : 0;
    np += (cn[i] + RP - 1) / RP;
  }
  if (tid == 0) s_item[0] = -1;
  int base, unused_ex, total, unused_tot;
  align_dev::block_scan2<kWaves>(np, 0, s_item + 4, s_item + 4 + kWaves, base, unused_ex, total, unused_tot);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int npi = (cn[i] + RP - 1) / RP;
    if (j >= base && j < base + npi) {
      s_item[0] = ex[i];
      s_item[1] = (j - base) * RP;
      s_item[2] = cn[i];
      s_item[3] = p.expert_offsets[ex[i]];
    }
    base += npi;
  }
  __syncthreads();
  return Pass{s_item[0], s_item[1], s_item[2], s_item[3]};
}

// The routed gate+up grid by XCD lane: column c = a * ng + g (a: index in the
// active list, g: column group) belongs to lane c % 8, and lane l's units are
// its columns in ascending order, each column's passes one after another.
// Workgroup b of the routed part takes unit b / 8 of lane b % 8: workgroups
// are dealt to the XCDs round-robin by id, so every pass of one (expert,
// column group) runs on one XCD, next to the others in dispatch order, and
// reads the expert's weights through one L2; a lane's units past its count
// come after its real ones.  The thread whose run of active experts holds
// unit k publishes (expert, first row, count, offset, column group); e = -1:
// lane l has fewer units.  Contains barriers.
struct LaneUnit {
  int e, r0, count, offset, g;
};
template <int RP>
__device__ __forceinline__ LaneUnit locate_lane_unit(const GroupedArgs& p, int lane, int k, int ng, int* s_item) {
  constexpr int kPer = (MOE_MAX_EXPERTS + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  const int per = (p.cap + kThreads - 1) / kThreads;
  const int a0 = min(p.cap, tid * per);
  // the first column group of active expert a in this lane, and how many it has there
  auto g_first = [&](int a) { return (lane - (a * ng) % 8 + 8) % 8; };
  auto n_cols = [&](int a) {
    const int g0 = g_first(a);
    return g0 < ng ? (ng - 1 - g0) / 8 + 1 : 0;
  };
  int ex[kPer], cn[kPer], units = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) ex[i] = (i < per && a0 + i < p.cap) ? p.active_experts[a0 + i] : -1;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    cn[i] = ex[i] >= 0 ? p.expert_counts[ex[i]] : 0;
    units += (cn[i] + RP - 1) / RP * n_cols(a0 + i);
  }
  if (tid == 0) s_item[0] = -1;
  int base, unused_ex, total, unused_tot;
  align_dev::block_scan2<kWaves>(units, 0, s_item + 8, s_item + 8 + kWaves, base, unused_ex, total, unused_tot);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int np = (cn[i] + RP - 1) / RP, u = np * n_cols(a0 + i);
    if (k >= base && k < base + u) {
      const int rel = k - base;
      s_item[0] = ex[i];
      s_item[1] = rel % np * RP;
      s_item[2] = cn[i];
      s_item[3] = p.expert_offsets[ex[i]];
      s_item[4] = g_first(a0 + i) + 8 * (rel / np);
    }
    base += u;
  }
  __syncthreads();
  return LaneUnit{s_item[0], s_item[1], s_item[2], s_item[3], s_item[4]};
}

// the FP8 block scale of chunk c from the lane-indexed registers
__device__ __forceinline__ float block_scale(const float (&sr)[kSL], int c) {
  const float v = (kSL == 1 || c < 64) ? sr[0] : sr[kSL - 1];
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), c & 63));
}

// ------------------------------------------------------------------ gate+up --

// one 128-deep chunk: gate and up from the ring, x rows from LDS slot xb.
// Each MFMA step reads its x fragment once for both matrices and converts the
// codes where they are used (registers for 4 workgroups per compute unit);
// every sum still runs its 4 steps in order.
template <bool ROWS>
__device__ __forceinline__ void gu_chunk(const u32x4 (&w)[2][2], const uint16_t* __restrict__ xb, int nrt, int q,
                                         int r16, float sg, float su, const f32x4 (&rs)[2],
                                         f32x4 (&acc)[2][kGuRows / 16]) {
#pragma unroll
  for (int rt = 0; rt < kGuRows / 16; ++rt) {
    if (rt < nrt) {
      f32x4 t[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 b =
            as_bf16x8(*reinterpret_cast<const uint4*>(xb + (rt * 16 + r16) * kXStride + k_of_step<true>(s, q)));
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 v = w[st][s >> 1];
          t[st] = mfma((s & 1) ? fp8x8_to_bf16(v.z, v.w) : fp8x8_to_bf16(v.x, v.y), b, t[st]);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[st][rt][i] = fmaf(ROWS ? rs[st][i] : (st == 0 ? sg : su), t[st][i], acc[st][rt][i]);
    }
  }
}

// MXFP4: one 128-deep chunk, gate and up codes (half 0 in .x .y, half 1 in
// .z .w) with the rows' scale dwords (one E8M0 byte per 32-deep block), over
// NRT row tiles.  Each step's codes are decoded once for all row tiles; every
// sum takes the steps in order.
template <int NRT>
__device__ __forceinline__ void gu_chunk_fp4_tiles(const u32x4 (&w)[2], const uint32_t (&sc)[2],
                                                   const uint16_t* __restrict__ xb, int q, int r16,
                                                   f32x4 (&acc)[2][kGuRows / 16]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 a[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) a[st] = fp4x8_to_bf16(w[st][s], e8m0_at(sc[st], 16 * (s >> 1) + 8 * (q >> 1)));
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const bf16x8 b =
          as_bf16x8(*reinterpret_cast<const uint4*>(xb + (rt * 16 + r16) * kXStride + k_of_step<true>(s, q)));
#pragma unroll
      for (int st = 0; st < 2; ++st) acc[st][rt] = mfma(a[st], b, acc[st][rt]);
    }
  }
}
// the pass's row tiles (1 or 2) chosen once per chunk, so no branch splits a step
__device__ __forceinline__ void gu_chunk_fp4(const u32x4 (&w)[2], const uint32_t (&sc)[2],
                                             const uint16_t* __restrict__ xb, int nrt, int q, int r16,
                                             f32x4 (&acc)[2][kGuRows / 16]) {
  static_assert(kGuRows == 32, "one or two row tiles");
  if (nrt > 1)
    gu_chunk_fp4_tiles<2>(w, sc, xb, q, r16, acc);
  else
    gu_chunk_fp4_tiles<1>(w, sc, xb, q, r16, acc);
}

// Grid (1-D): the shared expert's (32-token pass, 64-column group) units, then
// the routed (pass, 64-column group) units in XCD lanes (locate_lane_unit); the
// grid covers 8 lanes of ceil(groups / 8) times the most passes any routing of
// n slots can need, and the units past a lane's count exit.
template <int FMT, bool ROWS, bool TILED>
__global__ __launch_bounds__(kThreads, 4) void wide_gate_up_kernel(GroupedArgs p) {
  constexpr bool FP4 = FMT == kFmtFP4;
  static_assert(!(FP4 && ROWS), "MXFP4 has block scales only");
  constexpr int kRows = kGuRows, kShRows = kGuShRows, kRT = kRows / 16, kPieces = pieces_of<kRows>();
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [2][kRows][kXStride]
  __shared__ int s_src[kRows];
  __shared__ int s_item[8 + 2 * kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;

  const int sng = p.sw0 != nullptr ? p.sN / kGuCols : 0;
  const int nshared = p.sgroups * sng;
  const bool routed = (int)blockIdx.x >= nshared;
  int g, e = 0, r0 = 0, nr, row_base;
  if (routed) {
    const int r = (int)blockIdx.x - nshared;
    const LaneUnit u = locate_lane_unit<kRows>(p, r % 8, r / 8, p.N / kGuCols, s_item);
    if (u.e < 0) return;
    g = u.g;
    e = u.e;
    r0 = u.r0;
    nr = min(kRows, u.count - r0);
    row_base = u.offset;
  } else {
    g = (int)blockIdx.x % sng;
    row_base = (int)blockIdx.x / sng * kShRows;
    nr = min(kShRows, p.M - row_base);
  }
  const int N = routed ? p.N : p.sN, K = routed ? p.K : p.sK;
  const int nch = K / kKC;
  const int wcol = g * kGuCols + wave * kWaveCols;

  const size_t wstride = FP4 ? (size_t)N * K / 2 : (size_t)N * K;  // bytes of one matrix
  const char* W0 = routed ? static_cast<const char*>(p.w0) + (size_t)e * wstride : static_cast<const char*>(p.sw0);
  const char* W1 = routed ? static_cast<const char*>(p.w1) + (size_t)e * wstride : static_cast<const char*>(p.sw1);
  const size_t sstride = FP4 ? (size_t)N * (K / kMxBlock) : ROWS ? (size_t)N : (size_t)(N / kFp8Block) * (K / kFp8Block);
  const size_t sbytes = FP4 ? sstride : sstride * 4;
  const char* S0 = routed ? static_cast<const char*>(p.s0) + (size_t)e * sbytes : static_cast<const char*>(p.ss0);
  const char* S1 = routed ? static_cast<const char*>(p.s1) + (size_t)e * sbytes : static_cast<const char*>(p.ss1);
  // the expert's gate and up [N, K] matrices as buffers; tiled: the wave's
  // 16-column tile is one run of chunk fragments (FP8: 2 KB, this lane's 16
  // bytes at 16 * lane of each 1 KB half; MXFP4: 1 KB, 8 bytes at 8 * lane of
  // each 512-byte half); row-major: the lane's row
  const __amdgpu_buffer_rsrc_t wrs0 = rsrc(W0, (uint32_t)wstride), wrs1 = rsrc(W1, (uint32_t)wstride);
  const uint32_t lo =
      FP4 ? (uint32_t)(TILED ? (size_t)(wcol / kWaveCols) * (K / 2) * kWaveCols + lane * 8
                             : (size_t)(wcol + r16) * (K / 2) + q * 8)
          : (uint32_t)(TILED ? (size_t)(wcol / kWaveCols) * K * kWaveCols + lane * 16 : (size_t)(wcol + r16) * K + q * 16);
  // MXFP4: the E8M0 scale bytes ([N, K / 32], one dword per row and chunk)
  // of the workgroup's 64 gate and 64 up rows, staged in LDS once behind the x
  // slots; each step reads the lane's row dword of the next chunk from there
  const int kd = K / kKC;
  uint32_t* const s_sc = reinterpret_cast<uint32_t*>(xs + 2 * kRows * kXStride);
  if constexpr (FP4) {
    const int n = kGuCols * kd;
    stage_scales(s_sc, S0 + (size_t)g * n * 4, n);
    stage_scales(s_sc + n, S1 + (size_t)g * n * 4, n);
  }
  const uint32_t* const sc_row0 = s_sc + (wave * kWaveCols + r16) * kd;
  const uint32_t* const sc_row1 = sc_row0 + kGuCols * kd;

  // the row sources: the token of each row
  if (tid < nr) s_src[tid] = routed ? p.sorted_token_ids[row_base + r0 + tid] / p.top_k : row_base + tid;

  // scales: per lane one 128x128 block of the wave's columns, or (ROWS) the
  // row scales of the lane's 4 output columns
  float sreg[2][kSL];
  f32x4 rs[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const float* sp = reinterpret_cast<const float*>(st == 0 ? S0 : S1);
    if constexpr (FP4) {
#pragma unroll
      for (int i = 0; i < kSL; ++i) sreg[st][i] = 0.f;
      rs[st] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if constexpr (ROWS) {
      rs[st] = *reinterpret_cast<const f32x4*>(sp + wcol + 4 * q);
#pragma unroll
      for (int i = 0; i < kSL; ++i) sreg[st][i] = 0.f;
    } else {
      const int kb = K / kFp8Block;
      const float* sw = sp + (size_t)(wcol / kFp8Block) * kb;
#pragma unroll
      for (int i = 0; i < kSL; ++i) sreg[st][i] = lane + 64 * i < kb ? sw[lane + 64 * i] : 0.f;
      rs[st] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __syncthreads();  // s_src

  // x [M, K] bf16 as a buffer; this thread's rows u*16 + prow, 16-byte piece
  // ppc of each chunk (rows past the count: no fetch, zeros)
  const __amdgpu_buffer_rsrc_t xrs =
      rsrc(routed ? p.x : p.sx, (uint32_t)((size_t)p.M * K * 2));
  const int prow = tid >> 4, ppc = tid & 15;
  uint32_t xo[kPieces];
#pragma unroll
  for (int u = 0; u < kPieces; ++u)
    xo[u] = u * 16 + prow < nr ? (uint32_t)(((size_t)s_src[u * 16 + prow] * K + ppc * 8) * 2) : kNoFetch;
  uint16_t* xdst = xs + prow * kXStride + ppc * 8;

  u32x4 wb[kGuRing][2][2];    // FP8: [slot][gate, up][16-byte piece]
  u32x4 wq[kGuRing][2];       // MXFP4: [slot][gate, up] codes of the chunk
  uint32_t wsc[2][2];         // MXFP4: [chunk parity][gate, up] scale dwords, read a step ahead
  u32x4 xr[2][kPieces];
  f32x4 acc[2][kRT];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[st][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nrt = (nr + 15) >> 4;

  // chunks past the depth (the last round's padding) fetch nothing: zeros
#define WIDE_LOAD_W(c, SLOT)                                                                          \
  {                                                                                                   \
    if constexpr (FP4) {                                                                              \
      const uint32_t off = (c) < nch ? lo + (c) * (TILED ? 1024 : kKC / 2) : kNoFetch;               \
      const uint32_t hoff = TILED ? 512 : 32;                                                         \
      const u32x2 g0 = bload8(wrs0, off), g1 = bload8(wrs0, off + hoff);                             \
      const u32x2 u0 = bload8(wrs1, off), u1 = bload8(wrs1, off + hoff);                             \
      wq[SLOT][0] = u32x4{g0.x, g0.y, g1.x, g1.y};                                                   \
      wq[SLOT][1] = u32x4{u0.x, u0.y, u1.x, u1.y};                                                   \
    } else {                                                                                          \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                \
        const uint32_t off =                                                                          \
            (c) < nch ? lo + (TILED ? (c) * (kKC * kWaveCols) + j * 1024 : (c) * kKC + j * 64) : kNoFetch; \
        wb[SLOT][0][j] = bload(wrs0, off);                                                            \
        wb[SLOT][1][j] = bload(wrs1, off);                                                            \
      }                                                                                               \
    }                                                                                                 \
  }
#define WIDE_LOAD_X(c, R)                                                                                         \
  {                                                                                                               \
    const uint32_t co = (c) < nch ? (uint32_t)(c) * (kKC * 2) : kNoFetch;                                        \
    _Pragma("unroll") for (int u = 0; u < kPieces; ++u)(R)[u] = bload(xrs, xo[u] + co);                          \
  }
#define WIDE_STORE_X(slot, R)                                                                                     \
  {                                                                                                               \
    _Pragma("unroll") for (int u = 0; u < kPieces; ++u) *reinterpret_cast<u32x4*>(                              \
        xdst + (slot) * (kRows * kXStride) + u * 16 * kXStride) = (R)[u];                                        \
  }

  // prologue: x and weights of chunks 0 and 1 requested, x(0) staged
  WIDE_LOAD_X(0, xr[0]);
  WIDE_LOAD_W(0, 0);
  WIDE_LOAD_X(1, xr[1]);
  WIDE_LOAD_W(1, 1);
  WIDE_STORE_X(0, xr[0]);
  __syncthreads();
  if constexpr (FP4) {
    wsc[0][0] = sc_row0[0];
    wsc[0][1] = sc_row1[0];
  }
  // step c: request x and weights of chunk c + 2, multiply chunk c (ring slot
  // c % 3, LDS slot c % 2), stage x(c + 1), barrier.  Six steps written out,
  // so every ring index is a constant and no step is conditional (a load under
  // a branch costs a full wait for every load in flight); the depth is padded
  // to whole rounds of 6 with chunks that fetch nothing (zero codes, x and
  // scales), which leave every sum as it is (a sum that starts at +0 and adds
  // rounded products is never -0, so adding zeros keeps its bits).
  const int nsteps = (nch + 5) / 6 * 6;
#define WIDE_GU_STEP(JJ)                                                                                   \
  {                                                                                                        \
    const int c = c0 + (JJ);                                                                               \
    WIDE_LOAD_X(c + 2, xr[(JJ) % 2]);                                                                      \
    WIDE_LOAD_W(c + 2, ((JJ) + 2) % 3);                                                                    \
    if constexpr (FP4) {                                                                                   \
      const int cn = min(c + 1, nch - 1);                                                                  \
      wsc[((JJ) + 1) % 2][0] = c + 1 < nch ? sc_row0[cn] : 0u;                                             \
      wsc[((JJ) + 1) % 2][1] = c + 1 < nch ? sc_row1[cn] : 0u;                                             \
    }                                                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    if constexpr (FP4)                                                                                     \
      gu_chunk_fp4(wq[(JJ) % 3], wsc[(JJ) % 2], xs + ((JJ) % 2) * (kRows * kXStride), nrt, q, r16, acc);     \
    else                                                                                                   \
      gu_chunk<ROWS>(wb[(JJ) % 3], xs + ((JJ) % 2) * (kRows * kXStride), nrt, q, r16, block_scale(sreg[0], c), \
                     block_scale(sreg[1], c), rs, acc);                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    WIDE_STORE_X(((JJ) + 1) % 2, xr[((JJ) + 1) % 2]);                                                      \
    __syncthreads();                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
  }
  for (int c0 = 0; c0 < nsteps; c0 += 6) {
    WIDE_GU_STEP(0)
    WIDE_GU_STEP(1)
    WIDE_GU_STEP(2)
    WIDE_GU_STEP(3)
    WIDE_GU_STEP(4)
    WIDE_GU_STEP(5)
  }
#undef WIDE_GU_STEP
#undef WIDE_LOAD_W
#undef WIDE_LOAD_X
#undef WIDE_STORE_X

  float* OUT = routed ? p.out : p.sout;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = rt * 16 + r16;
    if (rt < nrt && r < nr) {
      float4 v;
      v.x = silu_mul(acc[0][rt][0], acc[1][rt][0]);
      v.y = silu_mul(acc[0][rt][1], acc[1][rt][1]);
      v.z = silu_mul(acc[0][rt][2], acc[1][rt][2]);
      v.w = silu_mul(acc[0][rt][3], acc[1][rt][3]);
      *reinterpret_cast<float4*>(OUT + (size_t)(row_base + r0 + r) * N + wcol + 4 * q) = v;
    }
  }
}

// --------------------------------------------------------------------- down --

constexpr int kAStride = 64 + kPad;                          // staged act row, bf16 elements (one half)
constexpr size_t kDnLds = (size_t)2 * 2 * kDnRows * kAStride * 2;  // two slots of (hi, lo)
constexpr int kDnRing = 4;                                   // weight halves in the register ring (3 ahead)
constexpr int kDnSets = 2;                                   // act register sets (requested 2 halves ahead)

// one 64-deep half: the wave's output tiles from the ring, act rows (hi, lo)
// from LDS slot ab; ROWS: the row scales of the wave's tiles from LDS (rsl,
// 16 per tile: held in registers they would not fit)
template <bool ROWS>
__device__ __forceinline__ void dn_half(const u32x4 (&w)[kDnTiles], const uint16_t* __restrict__ ab, int nrt, int q,
                                        int r16, int ntl, float sc, const float* __restrict__ rsl,
                                        f32x4 (&acc)[kDnTiles][kDnRows / 16]) {
  bf16x8 a[kDnTiles][2];
#pragma unroll
  for (int tt = 0; tt < kDnTiles; ++tt) {
    a[tt][0] = fp8x8_to_bf16(w[tt].x, w[tt].y);
    a[tt][1] = fp8x8_to_bf16(w[tt].z, w[tt].w);
  }
  constexpr int plane = kDnRows * kAStride;
#pragma unroll
  for (int rt = 0; rt < kDnRows / 16; ++rt) {
    if (rt < nrt) {
      bf16x8 b[2][2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          b[x][s] = as_bf16x8(
              *reinterpret_cast<const uint4*>(ab + x * plane + (rt * 16 + r16) * kAStride + q * 16 + s * 8));
#pragma unroll
      for (int tt = 0; tt < kDnTiles; ++tt) {
        if (tt < ntl) {
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int x = 0; x < 2; ++x) t = mfma(a[tt][s], b[x][s], t);
          f32x4 rsc = {sc, sc, sc, sc};
          if constexpr (ROWS) rsc = *reinterpret_cast<const f32x4*>(rsl + tt * 16 + 4 * q);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tt][rt][i] = add_rn(acc[tt][rt][i], mul_rn(rsc[i], t[i]));
        }
      }
    }
  }
}

// MXFP4: one 64-deep half (hodd: the chunk's second), the wave's tiles' codes
// (8 bytes each) and the scale dwords of their rows for the chunk
__device__ __forceinline__ void dn_half_fp4(const u32x2 (&w)[kDnTiles], const uint32_t (&sc)[kDnTiles],
                                            const uint16_t* __restrict__ ab, int nrt, int q, int r16, int ntl, int hodd,
                                            f32x4 (&acc)[kDnTiles][kDnRows / 16]) {
  bf16x8 a[kDnTiles][2];
#pragma unroll
  for (int tt = 0; tt < kDnTiles; ++tt) {
    // this lane's 16 k of the half lie in 32-deep block 2 hodd + q / 2
    const float bs = e8m0_at(sc[tt], 16 * hodd + 8 * (q >> 1));
    a[tt][0] = fp4x8_to_bf16(w[tt].x, bs);
    a[tt][1] = fp4x8_to_bf16(w[tt].y, bs);
  }
  constexpr int plane = kDnRows * kAStride;
#pragma unroll
  for (int rt = 0; rt < kDnRows / 16; ++rt) {
    if (rt < nrt) {
      bf16x8 b[2][2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          b[x][s] = as_bf16x8(
              *reinterpret_cast<const uint4*>(ab + x * plane + (rt * 16 + r16) * kAStride + q * 16 + s * 8));
#pragma unroll
      for (int tt = 0; tt < kDnTiles; ++tt) {
        if (tt < ntl) {
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int x = 0; x < 2; ++x) t = mfma(a[tt][s], b[x][s], t);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tt][rt][i] = add_rn(acc[tt][rt][i], t[i]);
        }
      }
    }
  }
}

// Grid (1-D): the shared expert's (32-token pass, 64-row group of H) units,
// then the routed (pass item, 256-row group) units, the group fastest.  A
// routed wave owns output tiles 4 (4g + w) .. +3, a shared wave tile 4g + w
// (tiles past N: none of its work).  The halves run in rounds of 4 (the ring
// length); a half past the depth multiplies zeros (its loads lie past their
// buffers and fetch nothing; scale 0), which leaves every sum as it is.
template <int FMT, bool ROWS, bool TILED>
__global__ __launch_bounds__(kThreads, kDnOcc) void wide_down_kernel(GroupedArgs p) {
  constexpr bool FP4 = FMT == kFmtFP4;
  static_assert(!(FP4 && ROWS), "MXFP4 has block scales only");
  constexpr int kRows = kDnRows, kShRows = kDnShRows, kRT = kRows / 16, kPieces = pieces_of<kRows>();
  extern __shared__ __attribute__((aligned(16))) uint16_t as[];  // [2 slots][hi, lo][kRows][kAStride]
  __shared__ int s_item[4 + 2 * kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;

  const int sng = p.sw0 != nullptr ? (p.sN + kDnShCols - 1) / kDnShCols : 0;
  const int nshared = p.sgroups * sng;
  const bool routed = (int)blockIdx.x >= nshared;
  int g, e = 0, r0 = 0, nr, row_base;
  if (routed) {
    const int r = (int)blockIdx.x - nshared;
    const int ng = (p.N + kDnCols - 1) / kDnCols;
    const Pass ps = locate_pass<kRows>(p, r / ng, s_item);
    if (ps.e < 0) return;
    g = r % ng;
    e = ps.e;
    r0 = ps.r0;
    nr = min(kRows, ps.count - r0);
    row_base = ps.offset;
  } else {
    g = (int)blockIdx.x % sng;
    row_base = (int)blockIdx.x / sng * kShRows;
    nr = min(kShRows, p.M - row_base);
  }
  const int N = routed ? p.N : p.sN, K = routed ? p.K : p.sK;
  const int nh = K / 64;
  // routed: 4 output tiles per wave; shared: 1 (its units are deeper, so narrower)
  const int tpw = routed ? kDnTiles : 1;
  const int tile0 = (g * kWaves + wave) * tpw;                     // first output tile of this wave
  const int ntl = min(tpw, max(0, N / kWaveCols - tile0));         // its tiles inside N

  const size_t wstride = FP4 ? (size_t)N * K / 2 : (size_t)N * K;  // bytes of one matrix
  const char* W = routed ? static_cast<const char*>(p.w0) + (size_t)e * wstride : static_cast<const char*>(p.sw0);
  const size_t sstride = FP4 ? (size_t)N * (K / kMxBlock) : ROWS ? (size_t)N : (size_t)(N / kFp8Block) * (K / kFp8Block);
  const size_t sbytes = FP4 ? sstride : sstride * 4;
  const char* SB = routed ? static_cast<const char*>(p.s0) + (size_t)e * sbytes : static_cast<const char*>(p.ss0);
  const float* S = reinterpret_cast<const float*>(SB);
  // the expert's [N, K] matrix as a buffer; per tile: tiled, one run of chunk
  // fragments (FP8: 2 KB, 1 KB per half, this lane's 16 bytes at 16 * lane;
  // MXFP4: 1 KB, 512 bytes per half, 8 bytes at 8 * lane); row-major, the
  // lane's row.  A tile past the wave's count fetches nothing.
  const __amdgpu_buffer_rsrc_t wrs = rsrc(W, (uint32_t)wstride);
  uint32_t wo[kDnTiles];
#pragma unroll
  for (int tt = 0; tt < kDnTiles; ++tt) {
    const int t = tile0 + tt;
    if constexpr (FP4)
      wo[tt] = tt < ntl ? (uint32_t)(TILED ? (size_t)t * (K / 2) * kWaveCols + lane * 8
                                           : (size_t)(t * kWaveCols + r16) * (K / 2) + q * 8)
                        : kNoFetch;
    else
      wo[tt] = tt < ntl ? (uint32_t)(TILED ? (size_t)t * K * kWaveCols + lane * 16
                                           : (size_t)(t * kWaveCols + r16) * K + q * 16)
                        : kNoFetch;
  }
  float sreg[kSL];
  // ROWS: lane l of each wave puts the scale of row l % 16 of its tile l / 16 in LDS
  __shared__ float s_rs[ROWS ? kWaves * kDnTiles * kWaveCols : 1];
  float* const rsl = s_rs + (ROWS ? wave * kDnTiles * kWaveCols : 0);
  if constexpr (FP4) {
#pragma unroll
    for (int i = 0; i < kSL; ++i) sreg[i] = 0.f;
  } else if constexpr (ROWS) {
    const int tt = lane >> 4;
    if (tt < kDnTiles) rsl[lane] = tt < ntl ? S[(tile0 + tt) * kWaveCols + (lane & 15)] : 0.f;
#pragma unroll
    for (int i = 0; i < kSL; ++i) sreg[i] = 0.f;
  } else {
    // the wave's rows lie in one 128-row block; past the depth the scale is 0
    const int kb = K / kFp8Block;
    const float* sw = S + (size_t)(min(tile0, N / kWaveCols - 1) * kWaveCols / kFp8Block) * kb;
#pragma unroll
    for (int i = 0; i < kSL; ++i) sreg[i] = lane + 64 * i < kb ? sw[lane + 64 * i] : 0.f;
  }

  // MXFP4: the scale dwords ([N, K / 32] bytes, one dword per row and chunk)
  // of the workgroup's rows (its waves' tiles: consecutive rows of N), staged
  // in LDS once behind the act slots; the lane reads its row's dword of each
  // tile from there (a tile past N reads the wave's first row: not stored)
  const int kd = K / kKC;
  uint32_t* const s_sc = reinterpret_cast<uint32_t*>(as + 2 * 2 * kRows * kAStride);
  if constexpr (FP4) {
    const int row0 = g * kWaves * tpw * kWaveCols;
    stage_scales(s_sc, SB + (size_t)row0 * kd * 4, min(kWaves * tpw * kWaveCols, N - row0) * kd);
  }
  const uint32_t* const sc_lane = s_sc + (wave * tpw * kWaveCols + r16) * kd;

  // the pass's act rows (consecutive: sorted positions, or tokens) as a buffer
  // of exactly nr rows; rows u*16 + prow, 4 floats at 4 * ppc of each half
  // (rows past nr lie past the buffer: no fetch, zeros)
  const char* A = routed ? static_cast<const char*>(p.x) : static_cast<const char*>(p.sx);
  const __amdgpu_buffer_rsrc_t ars = rsrc(A + (size_t)(row_base + r0) * K * 4, (uint32_t)((size_t)nr * K * 4));
  const int prow = tid >> 4, ppc = tid & 15;
  uint32_t ao[kPieces];
#pragma unroll
  for (int u = 0; u < kPieces; ++u)
    ao[u] = u * 16 + prow < nr ? (uint32_t)(((u * 16 + prow) * K + ppc * 4) * 4) : kNoFetch;
  uint16_t* adst = as + prow * kAStride + ppc * 4;
  constexpr int plane = kRows * kAStride;

  u32x4 wb[kDnRing][kDnTiles];        // FP8: [slot][tile] 16 bytes of the half
  u32x2 wq[kDnRing][kDnTiles];        // MXFP4: [slot][tile] 8 bytes of the half
  uint32_t wsc[2][kDnTiles];          // MXFP4: [half parity][tile] scale dwords, read a step ahead
  u32x4 xr[kDnSets][kPieces];
  f32x4 acc[kDnTiles][kRT];
#pragma unroll
  for (int tt = 0; tt < kDnTiles; ++tt)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nrt = (nr + 15) >> 4;
  const int nsteps = (nh + 3) / 4 * 4;  // whole rounds of 4

  // halves past the depth: offsets past the buffers (zeros, nothing fetched)
#define WIDE_LOAD_W(h, SLOT)                                                                                \
  {                                                                                                         \
    if constexpr (FP4) {                                                                                    \
      const uint32_t off =                                                                                  \
          (h) < nh ? (TILED ? ((h) >> 1) * 1024 + ((h) & 1) * 512 : ((h) >> 1) * (kKC / 2) + ((h) & 1) * 32) \
                   : kNoFetch;                                                                              \
      _Pragma("unroll") for (int tt = 0; tt < kDnTiles; ++tt) wq[SLOT][tt] = bload8(wrs, wo[tt] + off);    \
    } else {                                                                                                \
      const uint32_t off = (h) < nh ? (TILED ? ((h) >> 1) * (kKC * kWaveCols) + ((h) & 1) * 1024 : (h) * 64) \
                                    : kNoFetch;                                                             \
      _Pragma("unroll") for (int tt = 0; tt < kDnTiles; ++tt) wb[SLOT][tt] = bload(wrs, wo[tt] + off);     \
    }                                                                                                       \
  }
#define WIDE_LOAD_A(h, R)                                                                                   \
  {                                                                                                         \
    const uint32_t ho = (h) < nh ? (uint32_t)(h) * 256 : kNoFetch;                                          \
    _Pragma("unroll") for (int u = 0; u < kPieces; ++u)(R)[u] = bload(ars, ao[u] + ho);                    \
  }
  // act as bf16 hi + lo (the hi rounded to nearest even, the lo of the rest)
#define WIDE_STORE_A(slot, R)                                                                               \
  {                                                                                                         \
    _Pragma("unroll") for (int u = 0; u < kPieces; ++u) {                                                  \
      const u32x4 v = (R)[u];                                                                               \
      uint16_t hi[4], lw[4];                                                                                \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                      \
        const float f = __uint_as_float(v[i]);                                                              \
        hi[i] = bf16_rne_bits(f);                                                                           \
        lw[i] = bf16_rne_bits(f - bf16_bits_to_f32(hi[i]));                                                \
      }                                                                                                     \
      uint16_t* d = adst + (slot) * (2 * plane) + u * 16 * kAStride;                                       \
      *reinterpret_cast<uint2*>(d) = uint2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)}; \
      *reinterpret_cast<uint2*>(d + plane) =                                                                \
          uint2{lw[0] | ((uint32_t)lw[1] << 16), lw[2] | ((uint32_t)lw[3] << 16)};                          \
    }                                                                                                       \
  }

  // prologue: act of halves 0, 1 and weights of 0, 1, 2 requested, act(0) staged
  WIDE_LOAD_A(0, xr[0]);
  WIDE_LOAD_W(0, 0);
  WIDE_LOAD_A(1, xr[1]);
  WIDE_LOAD_W(1, 1);
  WIDE_LOAD_W(2, 2);
  WIDE_STORE_A(0, xr[0]);
  __syncthreads();
  if constexpr (FP4) {
#pragma unroll
    for (int tt = 0; tt < kDnTiles; ++tt) wsc[0][tt] = sc_lane[tt < ntl ? tt * kWaveCols * kd : 0];
  }
  // step h: request the weights of h + 3 and the act of h + 2 (set h % 2 held
  // act(h), staged a step ago), multiply half h (ring slot h % 4, LDS slot
  // h % 2), stage act(h + 1) (requested a step ago), barrier.  Four steps
  // written out, so every ring index is a constant and no step is conditional.
  // MXFP4: the scale dwords of half h + 1 (its chunk's, per tile) are read from
  // LDS a step ahead.
#define WIDE_DN_STEP(JJ)                                                                                    \
  {                                                                                                         \
    const int h = h0 + (JJ);                                                                                \
    WIDE_LOAD_W(h + 3, ((JJ) + 3) % 4);                                                                     \
    WIDE_LOAD_A(h + 2, xr[(JJ) % 2]);                                                                       \
    if constexpr (FP4) {                                                                                    \
      const int cn = min((h + 1) >> 1, kd - 1);                                                             \
      _Pragma("unroll") for (int tt = 0; tt < kDnTiles; ++tt) wsc[((JJ) + 1) % 2][tt] =                    \
          h + 1 < nh ? sc_lane[(tt < ntl ? tt * kWaveCols * kd : 0) + cn] : 0u;                             \
    }                                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    if constexpr (FP4)                                                                                      \
      dn_half_fp4(wq[(JJ) % 4], wsc[(JJ) % 2], as + ((JJ) % 2) * (2 * plane), nrt, q, r16, ntl, (JJ) & 1, acc); \
    else                                                                                                    \
      dn_half<ROWS>(wb[(JJ) % 4], as + ((JJ) % 2) * (2 * plane), nrt, q, r16, ntl, block_scale(sreg, h >> 1), \
                    rsl, acc);                                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    WIDE_STORE_A(((JJ) + 1) % 2, xr[((JJ) + 1) % 2]);                                                       \
    __syncthreads();                                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
  }
  for (int h0 = 0; h0 < nsteps; h0 += 4) {
    WIDE_DN_STEP(0)
    WIDE_DN_STEP(1)
    WIDE_DN_STEP(2)
    WIDE_DN_STEP(3)
  }
#undef WIDE_DN_STEP
#undef WIDE_LOAD_W
#undef WIDE_LOAD_A
#undef WIDE_STORE_A

  float* OUT = routed ? p.out : p.sout;
#pragma unroll
  for (int tt = 0; tt < kDnTiles; ++tt) {
    if (tt < ntl) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const int r = rt * 16 + r16;
        if (rt < nrt && r < nr) {
          const f32x4 v = acc[tt][rt];
          *reinterpret_cast<float4*>(OUT + (size_t)(row_base + r0 + r) * N + (tile0 + tt) * kWaveCols + 4 * q) =
              float4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
}

// dynamic LDS of a launch: the staged activation slots, and (MXFP4) the scale
// dwords of a workgroup's weight rows behind them
inline size_t gu_lds(int fmt, const GroupedArgs& a) {
  const int kd = max(a.K, a.sw0 != nullptr ? a.sK : 0) / kKC;
  return kGuLds + (fmt == kFmtFP4 ? (size_t)2 * kGuCols * kd * 4 : 0);
}
inline size_t dn_lds(int fmt, const GroupedArgs& a) {
  const size_t routed = (size_t)kDnCols * (a.K / kKC), shared = a.sw0 != nullptr ? (size_t)kDnShCols * (a.sK / kKC) : 0;
  return kDnLds + (fmt == kFmtFP4 ? max(routed, shared) * 4 : 0);
}

// the most RP-row passes n slots can need: sum over experts of
// ceil(count / RP) <= (n + active * (RP - 1)) / RP
inline int64_t max_items(const GroupedArgs& a, int RP) {
  const int64_t n = (int64_t)a.M * a.top_k;
  return (n + (int64_t)a.cap * (RP - 1)) / RP;
}

template <int FMT, bool ROWS, bool TILED>
hipError_t launch_gu(const GroupedArgs& a, hipStream_t s) {
  GroupedArgs b = a;
  const int64_t items = max_items(a, kGuRows);
  b.sgroups = a.sw0 != nullptr ? (a.M + kGuShRows - 1) / kGuShRows : 0;
  const long long blocks =
      (long long)b.sgroups * (a.sw0 != nullptr ? a.sN / kGuCols : 0) + (long long)items * ((a.N / kGuCols + 7) / 8 * 8);
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT_MAX || items > INT_MAX) return hipErrorInvalidValue;
  b.items = (int)items;
  hipLaunchKernelGGL((wide_gate_up_kernel<FMT, ROWS, TILED>), dim3((unsigned)blocks), dim3(kThreads), gu_lds(FMT, a), s,
                     b);
  return hipGetLastError();
}

template <int FMT, bool ROWS, bool TILED>
hipError_t launch_dn(const GroupedArgs& a, hipStream_t s) {
  GroupedArgs b = a;
  const int64_t items = max_items(a, kDnRows);
  b.sgroups = a.sw0 != nullptr ? (a.M + kDnShRows - 1) / kDnShRows : 0;
  const long long blocks = (long long)b.sgroups * (a.sw0 != nullptr ? (a.sN + kDnShCols - 1) / kDnShCols : 0) +
                           (long long)items * ((a.N + kDnCols - 1) / kDnCols);
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT_MAX || items > INT_MAX) return hipErrorInvalidValue;
  b.items = (int)items;
  hipLaunchKernelGGL((wide_down_kernel<FMT, ROWS, TILED>), dim3((unsigned)blocks), dim3(kThreads), dn_lds(FMT, a), s,
                     b);
  return hipGetLastError();
}

}  // namespace wide_detail

bool grouped_wide(int fmt, const GroupedArgs& a, bool gate_up) {
  // FP8 or MXFP4, tables from the align launch (not the fused align), experts
  // that can hold more rows than one 16-row pass (M > 16) and hold 4 or more
  // on average (n >= 4E: a sparser routing leaves most passes a few rows,
  // which the 16-row kernels stream as fast), FP8 depth within the scale
  // registers, gate+up widths in whole 64-column groups (MXFP4 allows any
  // multiple of 16), MXFP4 scales of a workgroup's rows within 64 KB of LDS
  // with the staged rows, and every buffer the kernels address under 2^31
  // bytes.  Both kernels pad the depth to whole rounds themselves.
  constexpr int64_t kLim = (int64_t)1 << 31;
  const bool fp4 = fmt == kFmtFP4;
  auto ok = [&](int N, int K) {
    return K % mma::kKC == 0 && (fp4 || K / kFp8Block <= wide_detail::kMaxScaleBlocks) &&
           (!gate_up || N % wide_detail::kGuCols == 0) && (int64_t)N * K < kLim &&
           (!gate_up || (int64_t)a.M * K * 2 < kLim);
  };
  const size_t lds = gate_up ? wide_detail::gu_lds(fmt, a) : wide_detail::dn_lds(fmt, a);
  return (fmt == kFmtFP8 || fp4) && a.ids == nullptr && a.M > 16 && (int64_t)a.M * a.top_k >= 4 * (int64_t)a.E &&
         ok(a.N, a.K) && (a.sw0 == nullptr || ok(a.sN, a.sK)) && lds + 1024 <= 65536;
}

hipError_t launch_wide_gate_up(int fmt, const GroupedArgs& a, bool tiled, hipStream_t s) {
  using namespace wide_detail;
  if (fmt == kFmtFP4) return tiled ? launch_gu<kFmtFP4, false, true>(a, s) : launch_gu<kFmtFP4, false, false>(a, s);
  if (a.scale_rows)
    return tiled ? launch_gu<kFmtFP8, true, true>(a, s) : launch_gu<kFmtFP8, true, false>(a, s);
  return tiled ? launch_gu<kFmtFP8, false, true>(a, s) : launch_gu<kFmtFP8, false, false>(a, s);
}

hipError_t launch_wide_down(int fmt, const GroupedArgs& a, bool tiled, hipStream_t s) {
  using namespace wide_detail;
  if (fmt == kFmtFP4) return tiled ? launch_dn<kFmtFP4, false, true>(a, s) : launch_dn<kFmtFP4, false, false>(a, s);
  if (a.scale_rows)
    return tiled ? launch_dn<kFmtFP8, true, true>(a, s) : launch_dn<kFmtFP8, true, false>(a, s);
  return tiled ? launch_dn<kFmtFP8, false, true>(a, s) : launch_dn<kFmtFP8, false, false>(a, s);
}

}  // namespace moe
