// Grouped expert projections for gfx950: gate+up with SiLU, and down.
//
// What is computed (metrale fp8_moe_grouped.rs: module doc, and the gate+up and
// down launchers' docs; nbxtensor moe_decode_vec.py: the SwiGLU epilogue):
//   gate+up: act[p, c] = silu(g) * u, g = sum_k Wg[e][c][k] x[t][k],
//            u = sum_k Wu[e][c][k] x[t][k], for each sorted position p holding a
//            slot of active expert e (t = slot / top_k); the shared expert does
//            the same for every token t into sh_act[t, c].
//   down:    out[p, c] = sum_k Wd[e][c][k] act[p][k] (shared: rows are tokens).
// A workgroup owns one pass (up to 16 rows) of one active expert, or one group
// of shared-expert rows, and one or two 64-column tiles of the output, and
// applies each weight row it streams from HBM to every row of its pass.  Rows
// of the intermediates are sorted positions.
//
// gfx950 design (not the pages' CUDA geometry):
//  * Matrix cores: v_mfma_f32_16x16x32_bf16.  The weights are the A operand
//    (16 output columns per wave), the expert's rows the B operand (16-row
//    tiles; rows past the expert's count are fed as zeros).  FP8 e4m3 codes
//    convert exactly to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8, scale
//    1); bf16 activations are exact, so the only rounding is the float32
//    accumulation.  Each 128-deep FP8 scale block is accumulated alone and then
//    multiplied by its scale.  MXFP4 codes convert to bf16 with their 32-deep
//    block's E8M0 scale applied in the same instruction
//    (v_cvt_scalef32_pk_bf16_fp4): a power-of-two multiple of an E2M1 value is
//    exact in bf16, so these accumulate like bf16 weights.  The down projection's float32 input is split into
//    bf16 hi + lo and both halves go through the matrix core, so it keeps ~16
//    bits of the input's mantissa.
//  * Memory: each lane streams 16-byte (dwordx4) loads of its weight row,
//    several 128-deep chunks ahead in a register ring.  The expert's activation
//    rows are staged in LDS once per workgroup and read as B operands by all
//    four waves: for the whole depth at once when they fit ("resident": the
//    weight stream then runs with no barrier at all), else 128 deep at a time
//    in two LDS slots with one barrier per chunk.  LDS rows are padded by 16
//    bytes against bank conflicts.
//  * Row invariance: a row's value depends only on its own inputs: every output
//    element is the same sequence of MFMA k-steps, scale FMAs and chunk sums
//    whatever tile, slot, pass or staging mode the row goes through, and the
//    rows per pass come from the shape class, never from the routing.
//  * Work items: one workgroup runs one pass (rowcap rows) of one expert over a
//    group of 64-column tiles.  The grid is (shared row groups + the most passes
//    any routing of n slots can need, column groups), sized from shapes only; a
//    routed workgroup finds its expert and pass from the active list and counts
//    (a block scan of the experts' pass counts), and one past the routing's
//    passes exits after that.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "align_device.h"
#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace grouped_detail {

using namespace mma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;  // 4 wave64 per workgroup
constexpr int kTileCols = 64;   // output columns per workgroup
constexpr int kMaxRowCap = 128; // most rows one pass stages
constexpr size_t kResidentLdsBudget = 80 * 1024;
constexpr int kMaxScaleBlocks = 128;  // FP8 depth limit: 128 scale blocks = 16384
constexpr int kMaxTilesPerGroup = 2;  // most 64-column tiles one workgroup runs in a row
constexpr int kStaged = 0, kResident = 1, kRoutedResident = 2;  // activation staging modes

// LDS bytes of the fused alignment region for E experts and n slots.
__host__ __device__ constexpr size_t fused_align_lds(int E, int n) {
  return ((size_t)kWaves * E + E + (E + 1) + E + 2 * kWaves + 2 + n) * sizeof(int);
}
// LDS bytes of the MXFP4 scale area: per weight stream, the scale dwords (one
// per row and 128-deep chunk) of ctw 64-row tiles at depth K
__host__ __device__ constexpr size_t mx_scale_area(int streams, int ctw, int K) {
  return (size_t)streams * ctw * kTileCols * (K / kKC) * sizeof(uint32_t);
}

// FMT: the weight format (kFmtBF16, kFmtFP8, kFmtFP4).
// ROWS (FP8 only): one float32 scale per weight row, [E, N], instead of one per
// 128x128 block; it multiplies the same places the block scale does (each
// 128-deep gate/up chunk's sum, each 64-deep down half), per output column.
// RES: how a workgroup stages its rows' activations: kStaged (128 deep at a
// time, one barrier per chunk), kResident (the whole depth at once, no barrier
// in the weight stream), or kRoutedResident (routed items resident, the shared
// expert's deeper rows staged; chosen when only the routed depth fits in LDS).
template <int FMT, bool ROWS, bool GATE_UP, int RT, int RES, bool TILED, bool FUSED, typename IdT>
__global__ __launch_bounds__(kThreads) void grouped_kernel(GroupedArgs p, int rowcap, int ctw, size_t xs_bytes) {
  constexpr bool FP8 = FMT == kFmtFP8;
  constexpr bool FP4 = FMT == kFmtFP4;
  constexpr bool BMAP = FMT != kFmtBF16;  // byte-coded weights: whole 128-deep chunks, the FP8 k map
  constexpr int NS = GATE_UP ? 2 : 1;   // weight streams (gate, up) or (down)
  constexpr int NX = GATE_UP ? 1 : 2;   // B planes: bf16 x, or bf16 hi + lo of act
  constexpr int WL = FP4 ? 1 : (FP8 ? 2 : 4);  // 16 bytes of weights per lane per chunk, in WL registers
  constexpr int ESZ = FP8 ? 1 : 2;      // weight element bytes (MXFP4: half a byte, see wbytes)
  constexpr int NBUF = RES == kStaged ? 2 : 3;  // weight chunks in the register ring
  constexpr int EPP = GATE_UP ? 8 : 4;  // source elements per 16-byte staging piece
  constexpr int SL = kMaxScaleBlocks / 64;  // scale registers per stream (one scale per lane)

  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [slot][plane][row][stride], then the align region
  __shared__ int s_src[kMaxRowCap];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  // ---- work item and column group of this workgroup.  The one-dimensional
  // grid holds first the shared expert's (row group, column group) pairs, so
  // its longer rows start first, then the routed (item, column group) pairs
  // with the item fastest: consecutive workgroups, which the dispatcher deals
  // round-robin to the XCDs, carry different items of one column group.
  // Routed item j is the j-th rowcap-row pass over the active experts taken in
  // ascending order, each expert contributing ceil(count / rowcap) passes; the
  // grid covers the most passes any routing of n slots can need, so it depends
  // on shapes only.
  const int ngs = (((p.sN + kTileCols - 1) / kTileCols) + ctw - 1) / ctw;  // shared column groups
  const int nshared = p.sgroups * ngs;
  const bool routed = (int)blockIdx.x >= nshared;
  int item, tgrp;
  if (routed) {
    const int r = (int)blockIdx.x - nshared;
    item = p.sgroups + r % p.items;
    tgrp = r / p.items;
  } else {
    item = (int)blockIdx.x / ngs;
    tgrp = (int)blockIdx.x % ngs;
  }
  const int N = routed ? p.N : p.sN, K = routed ? p.K : p.sK;
  const int t_begin = tgrp * ctw;
  const int t_end = min(t_begin + ctw, (N + kTileCols - 1) / kTileCols);
  if (t_begin >= t_end) return;

  int e = 0, rows = 0, row_base = 0, first_r0 = 0;
  const int* fsrc = nullptr;  // fused: sources of all of the expert's rows
  if (routed) {
    // which expert and pass item j is: every thread takes a run of active
    // indices, a block scan of their pass counts places the runs, and the
    // thread whose run holds pass j publishes (expert, pass, count, offset)
    __shared__ int s_item[4 + 2 * kWaves];
    const int j = item - p.sgroups;
    constexpr int kPer = (MOE_MAX_EXPERTS + kThreads - 1) / kThreads;
    const int per = (p.cap + kThreads - 1) / kThreads;
    const int a0 = min(p.cap, tid * per);
    auto find_item = [&](auto expert_of, auto count_of, auto offset_of) {
      int ex[kPer], cn[kPer], np = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) ex[i] = (i < per && a0 + i < p.cap) ? expert_of(a0 + i) : -1;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        cn[i] = ex[i] >= 0 ? count_of(ex[i]) : 0;
        np += (cn[i] + rowcap - 1) / rowcap;
      }
      if (tid == 0) s_item[0] = -1;
      int base, unused_ex, unused_tot, total;
      align_dev::block_scan2<kWaves>(np, 0, s_item + 4, s_item + 4 + kWaves, base, unused_ex, total, unused_tot);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int npi = (cn[i] + rowcap - 1) / rowcap;
        if (j >= base && j < base + npi) {
          s_item[0] = ex[i];
          s_item[1] = j - base;
          s_item[2] = cn[i];
          s_item[3] = offset_of(ex[i]);
        }
        base += npi;
      }
      __syncthreads();
      e = s_item[0];
      first_r0 = s_item[1] * rowcap;
      rows = s_item[2];
      row_base = s_item[3];
    };
    if constexpr (FUSED) {
      int* a = reinterpret_cast<int*>(reinterpret_cast<char*>(xs) + xs_bytes);
      const int E = p.E;
      const align_dev::ExpertLds s{a, a + kWaves * E, a + kWaves * E + E, a + kWaves * E + 2 * E + 1,
                                   a + kWaves * E + 3 * E + 1, a + kWaves * E + 3 * E + 1 + kWaves,
                                   a + kWaves * E + 3 * E + 1 + 2 * kWaves};
      int* src_all = s.scal + 2;
      const IdT* ids = static_cast<const IdT*>(p.ids);
      const int nbits = align_dev::id_bits(E);
      align_dev::count_pass<kWaves>(ids, p.n, E, nbits, s.cnt);
      align_dev::expert_scan<kWaves>(s, E, p.BS);
      const int nact = s.scal[0];
      find_item([&](int ai) { return ai < nact ? s.active[ai] : -1; }, [&](int ex) { return s.count[ex]; },
                [&](int ex) { return s.off[ex]; });
      if (e >= 0) align_dev::expert_rows<kWaves>(ids, p.n, E, nbits, s.cnt, e, p.top_k, src_all);
      if (item == p.sgroups && tgrp == 0) {  // the tables the later steps read
        __syncthreads();  // expert_rows is done with the bases scatter_pass advances
        align_dev::scatter_pass<kWaves>(ids, p.n, E, nbits, s.cnt, s.off, p.tables.sorted_token_ids,
                                        p.tables.token_to_perm);
        align_dev::write_rest<kWaves>(s, p.n, E, p.BS, p.max_total, p.cap, p.tables);
      }
      fsrc = src_all;
    } else {
      // active_experts holds -1 past the active count
      find_item([&](int ai) { return p.active_experts[ai]; }, [&](int ex) { return p.expert_counts[ex]; },
                [&](int ex) { return p.expert_offsets[ex]; });
    }
    if (e < 0) return;  // no such pass for this routing
  } else {
    row_base = item * rowcap;
    rows = min(rowcap, p.M - row_base);
  }

  // bytes of n weight elements
  auto wbytes = [](size_t n) -> size_t { return FP4 ? n / 2 : n * ESZ; };
  const char *W0, *W1 = nullptr;
  const float *S0 = nullptr, *S1 = nullptr;      // FP8 scales
  const uint8_t *B0 = nullptr, *B1 = nullptr;    // MXFP4 E8M0 scale bytes [N, K/32]
  const char* X;
  float* OUT;
  if (routed) {
    const size_t wstride = wbytes((size_t)N * (TILED ? round_up(K, kKC) : K));
    W0 = static_cast<const char*>(p.w0) + (size_t)e * wstride;
    if (GATE_UP) W1 = static_cast<const char*>(p.w1) + (size_t)e * wstride;
    if (FP8) {
      const size_t sstride = ROWS ? (size_t)N : (size_t)(N / kFp8Block) * (K / kFp8Block);
      S0 = static_cast<const float*>(p.s0) + (size_t)e * sstride;
      if (GATE_UP) S1 = static_cast<const float*>(p.s1) + (size_t)e * sstride;
    }
    if (FP4) {
      const size_t sstride = (size_t)N * (K / kMxBlock);
      B0 = static_cast<const uint8_t*>(p.s0) + (size_t)e * sstride;
      if (GATE_UP) B1 = static_cast<const uint8_t*>(p.s1) + (size_t)e * sstride;
    }
    X = static_cast<const char*>(p.x);
    OUT = p.out;
  } else {
    W0 = static_cast<const char*>(p.sw0);
    W1 = static_cast<const char*>(p.sw1);
    S0 = static_cast<const float*>(p.ss0);
    S1 = static_cast<const float*>(p.ss1);
    B0 = static_cast<const uint8_t*>(p.ss0);
    B1 = static_cast<const uint8_t*>(p.ss1);
    X = static_cast<const char*>(p.sx);
    OUT = p.sout;
  }
  const int nch = (K + kKC - 1) / kKC;
  const int nv = (t_end - t_begin) * nch;  // (tile, chunk) steps of one pass
  const int kpad = TILED ? round_up(K, kKC) : K;
  const int kblocks = K / kFp8Block;
  // MXFP4: the scale dwords of this workgroup's weight rows (its tiles' rows,
  // consecutive rows of N) per stream, in LDS behind the alignment region;
  // staged with the first activation rows, read where a chunk is multiplied
  const int kd = K / kKC;
  uint32_t* const s_sc = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(xs) + xs_bytes +
                                                     (FUSED ? fused_align_lds(p.E, p.n) : 0));
  auto stage_mx_scales = [&]() {
    if constexpr (FP4) {
      const int row0 = t_begin * kTileCols;
      const int n = (min(N, t_end * kTileCols) - row0) * kd;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(st == 0 ? B0 : B1) + (size_t)row0 * kd;
        uint32_t* dst = s_sc + st * ctw * kTileCols * kd;
        for (int b0 = 0; b0 < n; b0 += 8 * kThreads) {
          uint32_t v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = b0 + u * kThreads + tid;
            v[u] = i < n ? src[i] : 0u;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = b0 + u * kThreads + tid;
            if (i < n) dst[i] = v[u];
          }
        }
      }
    }
  };

  // a wave whose 16 columns lie past N reads the tile's first columns (valid
  // memory), multiplies nothing and stores nothing
  auto wave_col = [&](int t, bool& on) {
    const int c0 = t * kTileCols + wave * kWaveCols;
    on = c0 < N;
    return on ? c0 : t * kTileCols;
  };
  // row-major: this lane's weight row (A operand row r16 of the wave's tile);
  // tiled: the wave's 16-row tile, one contiguous run of 128-deep fragments
  // (MXFP4: each fragment two 512-byte halves, this lane's 8 bytes at 8 * lane)
  auto lane_offset = [&](int wcol) -> size_t {
    return TILED ? wbytes((size_t)(wcol / kWaveCols) * kpad * kWaveCols) + lane * (FP4 ? 8 : 16)
                 : wbytes((size_t)(wcol + r16) * K);
  };

  // load cursor: tile `lt`, chunk `lc` of the next weight load, and this lane's
  // pointers into that tile (recomputed only when the tile changes)
  int lt = t_begin, lc = 0;
  const char* lp0 = nullptr;
  const char* lp1 = nullptr;
  auto set_load_tile = [&](int t) {
    bool on;
    const int wcol = wave_col(t, on);
    const size_t lo = lane_offset(wcol);
    lp0 = W0 + lo;
    if (GATE_UP) lp1 = W1 + lo;
  };
  // unconditional loads of the cursor's chunk, then advance the cursor (past the
  // last step it stays on the last chunk, which is then loaded again): the
  // steady state has no branch around loads and no integer division.  MXFP4:
  // the lane's 16 bytes are half 0 then half 1 of the chunk (k = 64h + 16q ..
  // +15 each), and `sr` gets the row's four scale bytes of the chunk.
  auto load_next = [&](uint4 (&wr)[NS][WL], uint32_t (&sr)[NS]) {
    if constexpr (FP4) {
      const size_t off = TILED ? (size_t)lc * 1024 : (size_t)lc * (kKC / 2) + 8 * q;
      const size_t hoff = TILED ? 512 : 32;
      const uint2 a0 = *reinterpret_cast<const uint2*>(lp0 + off);
      const uint2 a1 = *reinterpret_cast<const uint2*>(lp0 + off + hoff);
      wr[0][0] = uint4{a0.x, a0.y, a1.x, a1.y};
      sr[0] = 0u;  // the scales come from LDS where the chunk is multiplied
      if (GATE_UP) {
        const uint2 b0 = *reinterpret_cast<const uint2*>(lp1 + off);
        const uint2 b1 = *reinterpret_cast<const uint2*>(lp1 + off + hoff);
        wr[NS - 1][0] = uint4{b0.x, b0.y, b1.x, b1.y};
        sr[NS - 1] = 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < (FP4 ? 0 : WL); ++j) {
      if (TILED) {
        const size_t off = (size_t)lc * kKC * kWaveCols * ESZ + j * 1024;
        wr[0][j] = *reinterpret_cast<const uint4*>(lp0 + off);
        if (GATE_UP) wr[NS - 1][j] = *reinterpret_cast<const uint4*>(lp1 + off);
      } else {
        // bf16 depth past K (a partial last chunk) loads a valid address and is zeroed
        const int kk = lc * kKC + k_of_step<FP8>(FP8 ? 2 * j : j, q);
        const int kc = FP8 ? kk : min(kk, K - 8);
        uint4 v0 = *reinterpret_cast<const uint4*>(lp0 + (size_t)kc * ESZ);
        uint4 v1 = GATE_UP ? *reinterpret_cast<const uint4*>(lp1 + (size_t)kc * ESZ) : v0;
        if (!FP8 && kk >= K) v0 = v1 = uint4{0u, 0u, 0u, 0u};
        wr[0][j] = v0;
        if (GATE_UP) wr[NS - 1][j] = v1;
      }
    }
    if (lc + 1 < nch) {
      ++lc;
    } else if (lt + 1 < t_end) {
      ++lt;
      lc = 0;
      set_load_tile(lt);
    }
  };

  // the first weight chunks of the first pass go out before anything else
  uint4 wb[NBUF][NS][WL];
  uint32_t sb[NBUF][NS];  // MXFP4 scale bytes of each ring chunk (unused otherwise)
  set_load_tile(lt);
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) load_next(wb[j], sb[j]);

  // the FP8 scales of a tile's 16 columns of this wave: one 128-deep block per
  // lane, or (ROWS) the scales of this lane's 4 output columns
  float sreg[NS][SL];
  f32x4 rs[NS];
  auto load_scales = [&](int t) {
    if (!FP8) return;
    bool on;
    const int wcol = wave_col(t, on);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if constexpr (ROWS) {
        rs[st] = *reinterpret_cast<const f32x4*>((st == 0 ? S0 : S1) + wcol + 4 * q);
      } else {
        const float* sw = (st == 0 ? S0 : S1) + (size_t)(wcol / kFp8Block) * kblocks;
#pragma unroll
        for (int i = 0; i < SL; ++i) sreg[st][i] = lane + 64 * i < kblocks ? sw[lane + 64 * i] : 0.f;
      }
    }
  };
  auto scale_of = [&](int st, int c) -> float {
    if (SL == 1 || c < 64) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sreg[st][0]), c & 63));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sreg[st][SL - 1]), c & 63));
  };

  const bool resident = RES == kResident || (RES == kRoutedResident && routed);
  const int stride = (resident ? K : kKC) + kPad;     // staged row length (bf16 elements)
  const int plane = rowcap * stride;                  // elements per B plane
  const int pieces = (resident ? K : kKC) / EPP;      // 16-byte pieces per staged row

  // one 16-byte piece of a source row, as loaded (bf16 x) or as fp32 act
  auto load_piece = [&](int src, int kk) -> uint4 {
    if (kk >= K) return uint4{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const uint4*>(X + ((size_t)src * K + kk) * (GATE_UP ? 2 : 4));
  };
  // write a piece at element offset `col` of staged row `r` in LDS slot `slot`
  auto store_piece = [&](uint4 v, int slot, int r, int col) {
    uint16_t* base = xs + (size_t)slot * NX * plane + r * stride + col;
    if (GATE_UP) {
      *reinterpret_cast<uint4*>(base) = v;
    } else {
      const float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
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
      *reinterpret_cast<uint2*>(base) = h2;
      *reinterpret_cast<uint2*>(base + plane) = l2;
    }
  };

  {  // this workgroup's one pass: rows [first_r0, first_r0 + rowcap) of the expert
    const int r0 = first_r0;
    const int nr = min(rowcap, rows - r0);
    const int nrt = (nr + 15) >> 4;
    load_scales(t_begin);

    // the source rows of this pass: fused from the LDS row list, else from the
    // tables (token of a slot for gate+up, the sorted position for down)
    const int* srcv = s_src;
    if (FUSED && routed) {
      srcv = fsrc + r0;
      __syncthreads();
    } else {
      int my_src = 0;
      if (tid < nr) {
        if (!routed)
          my_src = row_base + r0 + tid;                                   // token
        else if (GATE_UP)
          my_src = p.sorted_token_ids[row_base + r0 + tid] / p.top_k;     // token of the slot
        else
          my_src = row_base + r0 + tid;                                   // sorted position
      }
      __syncthreads();  // the previous pass is done with LDS
      if (tid < nr) s_src[tid] = my_src;
      __syncthreads();
    }

    f32x4 acc[NS][RT];
    auto zero_acc = [&]() {
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[st][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    zero_acc();

    // multiply chunk c: A from registers, B from LDS slot `slot` at element `kb`
    auto compute = [&](const uint4 (&wc)[NS][WL], const uint32_t (&scb)[NS], int slot, int kb, int c) {
      const int k0 = c * kKC;
      bf16x8 a[NS][4];
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (FP4) {
            // step s lies in half s / 2, whose 16 k of this lane are 32-deep
            // block 2 (s / 2) + q / 2 of the chunk
            const uint4 v = wc[st][0];
            const uint32_t d = s == 0 ? v.x : (s == 1 ? v.y : (s == 2 ? v.z : v.w));
            a[st][s] = fp4x8_to_bf16(d, e8m0_at(scb[st], 16 * (s >> 1) + 8 * (q >> 1)));
          } else if constexpr (FP8) {
            const uint4 v = wc[st][s >> 1];
            a[st][s] = (s & 1) ? fp8x8_to_bf16(v.z, v.w) : fp8x8_to_bf16(v.x, v.y);
          } else {
            a[st][s] = as_bf16x8(wc[st][s]);
          }
        }
      float sc[NS];
      if (FP8 && !ROWS) {
#pragma unroll
        for (int st = 0; st < NS; ++st) sc[st] = scale_of(st, c);
      }
      // the scale of output column i of this lane (a column's block or row scale)
      auto col_scale = [&](int st, int i) -> float {
        if constexpr (ROWS) return rs[st][i];
        return sc[st];
      };
      const uint16_t* xb = xs + (size_t)slot * NX * plane + kb;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt < nrt) {
          // B column n = row r16 of the tile.  Rows past the expert's count
          // (stale LDS, or the last staged row again when the tile is wider
          // than the staged rows) only reach output columns that are never
          // stored: each MFMA output column depends on its own B column alone.
          const int rowc = min(rt * 16 + r16, rowcap - 1);
          bf16x8 b[NX][4];
#pragma unroll
          for (int x = 0; x < NX; ++x)
#pragma unroll
            for (int s = 0; s < 4; ++s)
              b[x][s] = as_bf16x8(
                  *reinterpret_cast<const uint4*>(xb + x * plane + rowc * stride + k_of_step<BMAP>(s, q)));
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            if (GATE_UP && FP8) {
              f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < 4; ++s) t = mfma(a[st][s], b[0][s], t);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[st][rt][i] = fmaf(col_scale(st, i), t[i], acc[st][rt][i]);
            } else if (GATE_UP) {
              // bf16 depth comes in whole 32-deep steps; steps past K are skipped
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (BMAP || k0 + s * 32 < K) acc[st][rt] = mfma(a[st][s], b[0][s], acc[st][rt]);
            } else {
              // down: each 64-deep half of the chunk is multiplied from zero,
              // scaled (FP8), rounded and then added to the sum (no fused
              // multiply-add), so partial sums over 64-deep slices formed
              // elsewhere and added in the same order give the same bits;
              // bf16 steps past K are skipped, a half wholly past K adds nothing
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                if (BMAP || k0 + 64 * h < K) {
                  f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int s = 2 * h; s < 2 * h + 2; ++s)
                    if (BMAP || k0 + s * 32 < K)
#pragma unroll
                      for (int x = 0; x < NX; ++x) t = mfma(a[st][s], b[x][s], t);
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    acc[st][rt][i] = add_rn(acc[st][rt][i], FP8 ? mul_rn(col_scale(st, i), t[i]) : t[i]);
                }
              }
            }
          }
        }
      }
    };

    // lane holds columns wcol + 4q .. +3 of tile row r16
    auto epilogue = [&](int wcol) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = rt * 16 + r16;
        if (rt < nrt && r < nr) {
          float4 v;
          if (GATE_UP) {
            const f32x4 g = acc[0][rt], u = acc[NS - 1][rt];
            v.x = silu_mul(g[0], u[0]);
            v.y = silu_mul(g[1], u[1]);
            v.z = silu_mul(g[2], u[2]);
            v.w = silu_mul(g[3], u[3]);
          } else {
            v.x = acc[0][rt][0];
            v.y = acc[0][rt][1];
            v.z = acc[0][rt][2];
            v.w = acc[0][rt][3];
          }
          *reinterpret_cast<float4*>(OUT + (size_t)(row_base + r0 + r) * N + wcol + 4 * q) = v;
        }
      }
    };

    // compute cursor: tile `ct`, chunk `cc`; one step multiplies the chunk and,
    // at a tile's last chunk, stores the tile and moves to the next
    int ct = t_begin, cc = 0;
    bool con;
    int cwcol = wave_col(ct, con);
    auto step = [&](const uint4 (&wc)[NS][WL], const uint32_t (&scb)[NS], int slot, int kb) {
      if (con) {
        if constexpr (FP4) {
          // the lane's row of the tile: its scale dword of chunk cc, per stream
          const int row = (ct - t_begin) * kTileCols + wave * kWaveCols + r16;
          uint32_t scl[NS];
#pragma unroll
          for (int st = 0; st < NS; ++st) scl[st] = s_sc[(st * ctw * kTileCols + row) * kd + cc];
          compute(wc, scl, slot, kb, cc);
        } else {
          compute(wc, scb, slot, kb, cc);
        }
      }
      if (cc + 1 < nch) {
        ++cc;
      } else {
        if (con) epilogue(cwcol);
        zero_acc();
        cc = 0;
        if (++ct < t_end) {
          cwcol = wave_col(ct, con);
          load_scales(ct);
        }
      }
    };

    stage_mx_scales();  // visible after the barrier that ends the row staging
    if (resident) {
      // every row of this pass, the whole depth
      const int total = nr * pieces;
      for (int base = 0; base < total; base += 8 * kThreads) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = base + u * kThreads + tid;
          v[u] = idx < total ? load_piece(srcv[idx / pieces], (idx % pieces) * EPP) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = base + u * kThreads + tid;
          if (idx < total) store_piece(v[u], 0, idx / pieces, (idx % pieces) * EPP);
        }
      }
      __syncthreads();
      // steady state: the load of step v + NBUF - 1 goes out before step v is
      // multiplied; no barrier and no branch around loads
      for (int v0 = 0; v0 < nv; v0 += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          load_next(wb[(j + NBUF - 1) % NBUF], sb[(j + NBUF - 1) % NBUF]);
          if (v0 + j < nv) step(wb[j], sb[j], 0, cc * kKC);
        }
      }
    } else {
      // 128 deep at a time through two LDS slots, one barrier per step
      constexpr int XP = (RT * 16 * (kKC / EPP) + kThreads - 1) / kThreads;
      const int total = nr * pieces;
      uint4 xr[XP];
      auto load_x = [&](int c) {
#pragma unroll
        for (int u = 0; u < XP; ++u) {
          const int idx = u * kThreads + tid;
          xr[u] = idx < total ? load_piece(srcv[idx / pieces], c * kKC + (idx % pieces) * EPP)
                              : uint4{0u, 0u, 0u, 0u};
        }
      };
      auto store_x = [&](int slot) {
#pragma unroll
        for (int u = 0; u < XP; ++u) {
          const int idx = u * kThreads + tid;
          if (idx < total) store_piece(xr[u], slot, idx / pieces, (idx % pieces) * EPP);
        }
      };
      load_x(0);
      store_x(0);
      __syncthreads();
      for (int v0 = 0; v0 < nv; v0 += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int v = v0 + j;
          if (v < nv) {
            load_x(cc + 1 < nch ? cc + 1 : 0);  // issued before the weights: waiting on it leaves them in flight
            load_next(wb[(j + NBUF - 1) % NBUF], sb[(j + NBUF - 1) % NBUF]);
            step(wb[j], sb[j], v & 1, 0);
            if (v + 1 < nv) store_x((v + 1) & 1);
            __syncthreads();
          }
        }
      }
    }
  }
}

// compute units of the current device (cached per device)
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <int FMT, bool ROWS, bool GATE_UP, int RT, int RES, bool TILED, bool FUSED, typename IdT>
hipError_t launch_one(const GroupedArgs& a, int rowcap, size_t xs_bytes, int tiles, hipStream_t s) {
  auto kern = grouped_kernel<FMT, ROWS, GATE_UP, RT, RES, TILED, FUSED, IdT>;
  // MXFP4: the scale area for ctw tiles at the deeper of the routed and shared depths
  const int kmax = (a.sw0 != nullptr && a.sK > a.K) ? a.sK : a.K;
  auto lds_for = [&](int ctw_) {
    return xs_bytes + (FUSED ? fused_align_lds(a.E, a.n) : 0) +
           (FMT == kFmtFP4 ? mx_scale_area(GATE_UP ? 2 : 1, ctw_, kmax) : 0);
  };
  constexpr size_t kLdsMax = 160 * 1024;
  const int max_ctw = lds_for(kMaxTilesPerGroup) <= kLdsMax ? kMaxTilesPerGroup : 1;
  size_t lds = lds_for(1);
  if (lds > kLdsMax) return hipErrorInvalidValue;  // MXFP4 scales of a 64-row tile past the LDS (depth > 16k)
  static std::atomic<size_t> allowed[kMaxCachedDevices];
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds_for(max_ctw), allowed);
  if (e != hipSuccess) return e;
  // column tiles per workgroup: the fewest that let every workgroup of the
  // worst case (every item busy) be resident at once, but at most
  // kMaxTilesPerGroup, so a wide grid (many experts, large M) keeps its
  // parallelism instead of serialising the columns inside few workgroups
  static std::atomic<uint64_t> occupancy[kMaxCachedDevices];
  int occ_per_cu = 0;
  e = occupancy_per_cu(reinterpret_cast<const void*>(kern), kThreads, lds, occupancy, occ_per_cu);
  if (e != hipSuccess) return e;
  const int slots = std::max(1, occ_per_cu) * device_cus();
  // (the shared and routed items may have different column counts: `tiles` is the larger)
  const int items = a.sgroups + a.items;
  int ctw = 1;
  while (ctw < tiles && ctw < max_ctw && (long long)items * ((tiles + ctw - 1) / ctw) > slots) ++ctw;
  lds = lds_for(ctw);
  const long long groups_r = ((a.N + kTileCols - 1) / kTileCols + ctw - 1) / ctw;
  const long long groups_s = a.sgroups ? ((a.sN + kTileCols - 1) / kTileCols + ctw - 1) / ctw : 0;
  const long long blocks = a.sgroups * groups_s + a.items * groups_r;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;  // more workgroups than one launch takes
  const dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a, rowcap, ctw, xs_bytes);
  return hipGetLastError();
}

template <int FMT, bool ROWS, bool GATE_UP, int RT, int RES, bool TILED>
hipError_t launch_fused_or_not(const GroupedArgs& a, int rowcap, size_t xs_bytes, int tiles, hipStream_t s) {
  if (GATE_UP && a.ids != nullptr) {
    if (a.ids64)
      return launch_one<FMT, ROWS, GATE_UP, RT, RES, TILED, GATE_UP, int64_t>(a, rowcap, xs_bytes, tiles, s);
    return launch_one<FMT, ROWS, GATE_UP, RT, RES, TILED, GATE_UP, int32_t>(a, rowcap, xs_bytes, tiles, s);
  }
  return launch_one<FMT, ROWS, GATE_UP, RT, RES, TILED, false, int32_t>(a, rowcap, xs_bytes, tiles, s);
}

template <int FMT, bool ROWS, bool GATE_UP, int RT, bool TILED>
hipError_t launch_rt(const GroupedArgs& a, int rowcap, hipStream_t s) {
  constexpr int NX = GATE_UP ? 1 : 2;
  const int kmax = (a.sw0 != nullptr && a.sK > a.K) ? a.sK : a.K;
  // (MXFP4: the workgroup's scale area counts against the resident budget)
  const size_t mx = FMT == kFmtFP4 ? mx_scale_area(GATE_UP ? 2 : 1, kMaxTilesPerGroup, kmax) : 0;
  const size_t resident = (size_t)NX * rowcap * (kmax + kPad) * 2;
  const size_t routed_resident = (size_t)NX * rowcap * (a.K + kPad) * 2;
  const size_t chunked = (size_t)2 * NX * rowcap * (kKC + kPad) * 2;
  const int nmax = (a.sw0 != nullptr && a.sN > a.N) ? a.sN : a.N;
  const int tiles = (nmax + kTileCols - 1) / kTileCols;
  GroupedArgs b = a;
  b.sgroups = a.sw0 != nullptr ? (a.M + rowcap - 1) / rowcap : 0;
  // the most rowcap-row passes n slots can need: sum over experts of
  // ceil(count / rowcap) <= (n + active * (rowcap - 1)) / rowcap
  const int64_t n = (int64_t)a.M * a.top_k;
  b.items = (int)((n + (int64_t)a.cap * (rowcap - 1)) / rowcap);
  if (resident + mx <= kResidentLdsBudget)
    return launch_fused_or_not<FMT, ROWS, GATE_UP, RT, kResident, TILED>(b, rowcap, resident, tiles, s);
  // only the shared expert's depth is too deep: its items stage 128 deep at a
  // time while the routed items keep their rows resident
  if (routed_resident + mx <= kResidentLdsBudget)
    return launch_fused_or_not<FMT, ROWS, GATE_UP, RT, kRoutedResident, TILED>(
        b, rowcap, std::max(routed_resident, chunked), tiles, s);
  return launch_fused_or_not<FMT, ROWS, GATE_UP, RT, kStaged, TILED>(b, rowcap, chunked, tiles, s);
}

// one 16-row tile per pass: each pass of an expert is a workgroup of its own
template <int FMT, bool ROWS, bool GATE_UP>
hipError_t launch(const GroupedArgs& a, int rowcap, bool tiled, hipStream_t s) {
  return tiled ? launch_rt<FMT, ROWS, GATE_UP, 1, true>(a, rowcap, s)
               : launch_rt<FMT, ROWS, GATE_UP, 1, false>(a, rowcap, s);
}

}  // namespace grouped_detail
}  // namespace moe
