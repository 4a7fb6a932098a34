// Single-pass decode-width MoE layer for gfx950.
//
// What is computed is the layer of metrale forward_nvfp4_grouped_decode.rs
// (step order: sort, gate+up+SiLU, down, blend) over the sort of nbxtensor
// moe_align.py and the FP8 grouped kernels of metrale fp8_moe_grouped.rs:
//   act[r, c]  = silu(Wg[e][c] . x[t]) * (Wu[e][c] . x[t])       (row r = slot of expert e)
//   y[r, h]    = sum_c Wd[e][h][c] act[r, c]
//   out[t, h]  = bf16( sum_k w[t,k] y[slot t*top_k+k, h]  (+ shared expert) )
//
// Decomposition (not the pages' geometry).  At decode width every expert holds
// a row or two, so the layer is a stream of expert weights.  One workgroup of 4
// waves owns one active expert and one 64-wide slice j of the intermediate:
//   1. it aligns topk_ids in LDS (ballot counts, no atomics) to find its
//      expert and that expert's slots; workgroup (0, 0) also writes the tables;
//   2. gate+up: each wave streams 16 rows of Wg and Wu (all of H) and leaves
//      act[:, 16 columns] in LDS, split into bf16 hi + lo;
//   3. down: after one barrier, the 4 waves stream the 64-deep slice j of Wd
//      (all H rows, four 16-row tiles per step) against act from LDS, and store
//      part[j][slot][h] = scale * (the slice's product), float32.
// The weight stream runs through one register ring across both phases, so the
// first down tiles are in flight while gate+up finishes, and the x rows are
// requested before the first weights so the two round trips overlap.  Nothing
// waits on another workgroup.  A second kernel forms y = sum_j part[j] (j
// ascending, from 0, no fused multiply-add) and blends it as the blend kernel
// does; the separate down kernel sums 64-deep halves of its chunks the same
// way, so this path and the separate calls give the same bits.
//
// Row invariance: every output element is the same sequence of MFMA k-steps,
// scale multiplies and ordered sums whatever the number of tokens; the rows per
// pass come from the shape class (M), never from the routing.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "align_device.h"
#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace layer_detail {

using namespace mma;

constexpr int kColTiles = 4;                // 16-column tiles of the intermediate per workgroup
constexpr int kSlice = kColTiles * kWaveCols;  // 64: intermediate columns per workgroup = down depth per workgroup
constexpr int kNarrowSlots = 8;             // slot counts up to this take the 8-wave (split gate / up) kernel
constexpr int kNarrowMinH = 1024;           // ... when H is at least this (small layers are faster on 4 waves)
static_assert(2 * kSlice == kKC, "a slice is half of one 128-deep chunk (one FP8 scale block)");
constexpr int kDownTiles = 4;               // 16-row tiles of H per down step
constexpr int kMaxScaleBlocks = 128;        // FP8 depth limit of H: 128 scale blocks
constexpr size_t kLdsBudget = 96 * 1024;
constexpr int kMaxRowCap = 64;              // rows per pass (4 row tiles) this kernel keeps in registers
constexpr int kXFirst = 4;                  // x pieces per thread requested before the first weights

__host__ __device__ constexpr size_t align_lds_bytes(int E, int n, int waves) {
  return ((size_t)waves * E + E + (E + 1) + E + 2 * waves + 2 + n) * sizeof(int);
}
__host__ __device__ constexpr size_t x_lds_bytes(int rowcap, int H) { return (size_t)rowcap * (H + kPad) * 2; }
// MXFP4 scale bytes: gate and up rows of the slice ([kSlice][H/32 + 4] each, the
// 4 pad bytes against bank conflicts), then one 16-bit pair per down row [H]
__host__ __device__ constexpr int mx_row_bytes(int H) { return H / kMxBlock + 4; }
__host__ __device__ constexpr size_t mx_scale_lds_bytes(int H) { return (size_t)2 * kSlice * mx_row_bytes(H) + (size_t)H * 2; }
// act as bf16 hi + lo, plus (8-wave kernel) the up sums handed to the gate waves
__host__ __device__ constexpr size_t act_lds_bytes(int rowcap, bool split) {
  return (size_t)2 * rowcap * (kSlice + kPad) * 2 + (split ? (size_t)rowcap * kSlice * 4 : 0);
}

// W = 4: wave w streams gate and up tile w of the slice.  W = 8 (narrow
// widths, few workgroups): waves 0-3 stream the gate tiles and 4-7 the up
// tiles, two 128-deep chunks per step, and the up sums reach the gate waves
// through LDS; each wave then streams half the bytes, which helps when the
// whole layer is only a few hundred workgroups.  Same arithmetic either way.
// FMT: the weight format (kFmtBF16, kFmtFP8, kFmtFP4).  MXFP4 codes become
// bf16 with their E8M0 block scale in the conversion (exact), so they
// accumulate as bf16 weights do.  A workgroup stages the scale bytes it uses
// in LDS once, before its first pass: the 64 gate and 64 up rows of its slice
// (every 32-deep block of H) and, for each of the H down rows, the two bytes
// of its 64-deep half-chunk; each step then reads them from LDS, not HBM.
// ROWS (FP8 only): one float32 scale per weight row ([E, N]) instead of one
// per 128x128 block; it multiplies where the block scale does, per output
// column (gate/up: the lane's 4 intermediate columns; down: its 4 rows of H,
// read from a copy of the expert's down row scales in LDS).
template <int FMT, bool ROWS, int RT, typename IdT, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(RT == 1 ? 3 : 2))) void layer_kernel(
    FusedLayerArgs p, int rowcap, size_t xs_bytes, size_t act_bytes) {
  constexpr int kWaves = W;
  constexpr int kThreads = W * 64;
  constexpr bool SPLIT = W == 2 * kColTiles;
  static_assert(W == kColTiles || SPLIT, "4 waves (gate + up per wave) or 8 (gate and up on separate waves)");
  constexpr bool FP8 = FMT == kFmtFP8;
  constexpr bool FP4 = FMT == kFmtFP4;
  constexpr bool BMAP = FMT != kFmtBF16;      // byte-coded weights: whole chunks, the byte k map
  constexpr int WL = FP4 ? 1 : (FP8 ? 2 : 4); // 16-byte registers per lane per 16x128 fragment
  constexpr int HL = FP8 ? 1 : 2;             // per 64-deep half fragment (MXFP4: 8 bytes, half a register)
  constexpr int NL = 2 * WL;                  // registers per lane per step (both phases)
  constexpr int FB = kWaveCols * kKC * (FP4 ? 1 : (FP8 ? 2 : 4)) / 2;  // bytes of one fragment
  constexpr int LB = FP4 ? 8 : 16;            // bytes of one lane in a (half) fragment
  constexpr int NBUF = FP8 || FP4 ? 3 : 2;      // steps in the register ring
  constexpr int SL = kMaxScaleBlocks / 64;

  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* xs = lds;                                                                   // [rowcap][H + pad]
  uint16_t* as = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(lds) + xs_bytes);  // [2][rowcap][64 + pad]
  int* al = reinterpret_cast<int*>(reinterpret_cast<char*>(lds) + xs_bytes + act_bytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int by = blockIdx.y, slice = blockIdx.x;
  const bool routed = by < p.cap;
  const int NI = routed ? p.I : p.S;  // intermediate width: gate/up rows, down depth
  if (slice * kSlice >= NI) return;
  const int H = p.H;

  // ---- which expert and rows
  int e = 0, rows = 0, row_base = 0;
  const int* slots = nullptr;
  if (routed) {
    const int E = p.E;
    const align_dev::ExpertLds s{al, al + kWaves * E, al + kWaves * E + E, al + kWaves * E + 2 * E + 1,
                                 al + kWaves * E + 3 * E + 1, al + kWaves * E + 3 * E + 1 + kWaves,
                                 al + kWaves * E + 3 * E + 1 + 2 * kWaves};
    int* slot_all = s.scal + 2;
    const IdT* ids = static_cast<const IdT*>(p.ids);
    const int nbits = align_dev::id_bits(E);
    align_dev::count_pass<kWaves>(ids, p.n, E, nbits, s.cnt);
    align_dev::expert_scan<kWaves>(s, E, p.BS);
    const int nact = s.scal[0];
    if (by < nact) {
      e = s.active[by];
      rows = s.count[e];
      align_dev::expert_rows<kWaves>(ids, p.n, E, nbits, s.cnt, e, 1, slot_all);
    }
    if (slice == 0 && by == 0) {  // the tables
      __syncthreads();  // expert_rows is done with the bases scatter_pass advances
      align_dev::scatter_pass<kWaves>(ids, p.n, E, nbits, s.cnt, s.off, p.tables.sorted_token_ids,
                                      p.tables.token_to_perm);
      align_dev::write_rest<kWaves>(s, p.n, E, p.BS, p.max_total, p.cap, p.tables);
    }
    if (by >= nact) return;
    slots = slot_all;
    __syncthreads();  // every wave's part of the slot list is in LDS before any wave reads it
  } else {
    row_base = (by - p.cap) * rowcap;
    rows = min(rowcap, p.M - row_base);
  }

  // ---- weight streams
  const int kpH = round_up(H, kKC), kpI = round_up(NI, kKC);
  const int nchH = kpH / kKC;                           // 128-deep chunks of H
  const size_t tile_g = (size_t)kpH / kKC * FB;  // bytes of one 16-row tile of Wg / Wu
  const size_t tile_d = (size_t)kpI / kKC * FB;  // of Wd
  const char *G, *U, *D;
  const float *SG = nullptr, *SU = nullptr, *SD = nullptr;        // FP8 scales
  const uint8_t *BG = nullptr, *BU = nullptr, *BD = nullptr;      // MXFP4 E8M0 bytes [N, K/32]
  float* OUT;
  if (routed) {
    G = static_cast<const char*>(p.w[0]) + (size_t)e * NI * tile_g / kWaveCols;
    U = static_cast<const char*>(p.w[1]) + (size_t)e * NI * tile_g / kWaveCols;
    D = static_cast<const char*>(p.w[2]) + (size_t)e * H * tile_d / kWaveCols;
    if (FP8) {
      const size_t ss = (size_t)(NI / kFp8Block) * (H / kFp8Block);
      SG = static_cast<const float*>(p.s[0]) + e * (ROWS ? (size_t)NI : ss);
      SU = static_cast<const float*>(p.s[1]) + e * (ROWS ? (size_t)NI : ss);
      SD = static_cast<const float*>(p.s[2]) + e * (ROWS ? (size_t)H : ss);
    }
    if (FP4) {
      const size_t ss = (size_t)NI * (H / kMxBlock);  // the same count for [I, H/32] and [H, I/32]
      BG = static_cast<const uint8_t*>(p.s[0]) + e * ss;
      BU = static_cast<const uint8_t*>(p.s[1]) + e * ss;
      BD = static_cast<const uint8_t*>(p.s[2]) + e * ss;
    }
    OUT = p.part + (size_t)slice * p.n * H;
  } else {
    G = static_cast<const char*>(p.sw[0]);
    U = static_cast<const char*>(p.sw[1]);
    D = static_cast<const char*>(p.sw[2]);
    SG = static_cast<const float*>(p.ss[0]);
    SU = static_cast<const float*>(p.ss[1]);
    SD = static_cast<const float*>(p.ss[2]);
    BG = static_cast<const uint8_t*>(p.ss[0]);
    BU = static_cast<const uint8_t*>(p.ss[1]);
    BD = static_cast<const uint8_t*>(p.ss[2]);
    OUT = p.sh_part + (size_t)slice * p.M * H;
  }
  // gate+up: this wave's 16 intermediate columns (a wave past NI loads the
  // slice's first tile, multiplies nothing and leaves its act columns unused)
  const int st = SPLIT ? wave / kColTiles : 0;  // split: stream of this wave (0 gate, 1 up)
  const int ct = SPLIT ? wave % kColTiles : wave;
  const int tg = slice * kColTiles + ct;
  const bool gon = tg * kWaveCols < NI;
  const int tgl = gon ? tg : slice * kColTiles;  // the tile this wave loads
  const char* gbase = (SPLIT && st ? U : G) + (size_t)tgl * tile_g + lane * LB;
  const char* ubase = U + (size_t)tgl * tile_g + lane * LB;
  const int ngs = SPLIT ? (nchH + 1) / 2 : nchH;  // gate/up steps (split: two chunks of one stream each)
  // down: this wave's run of 16-row tiles of H, kDownTiles per step (tiles past
  // H load the last tile again and store nothing); the slice is half `hf` of
  // chunk slice / 2 of each tile
  const int ntd = H / kWaveCols;
  const int per = round_up((ntd + kWaves - 1) / kWaves, kDownTiles);
  const int dfirst = wave * per;
  const int nd = per / kDownTiles;
  const int nv = ngs + nd;
  const int hf = slice & 1;
  const char* dbase = D + (size_t)(slice >> 1) * FB + hf * (FB / 2) + lane * LB;

  // one step's weights into the ring
  auto load_step = [&](int v, uint4 (&wr)[NL]) {
    v = min(v, nv - 1);
    if constexpr (FP4) {
      // both branches fill every register of the slot (a slot written in part
      // on one branch is kept in scratch memory by the compiler)
      uint4 r0, r1;
      if (v < ngs) {
        const int c0 = SPLIT ? 2 * v : v, c1 = SPLIT ? min(2 * v + 1, nchH - 1) : v;
        const char* a0 = gbase + (size_t)c0 * FB;
        const char* a1 = (SPLIT ? gbase : ubase) + (size_t)c1 * FB;
        const uint2 g0 = *reinterpret_cast<const uint2*>(a0), g1 = *reinterpret_cast<const uint2*>(a0 + FB / 2);
        const uint2 u0 = *reinterpret_cast<const uint2*>(a1), u1 = *reinterpret_cast<const uint2*>(a1 + FB / 2);
        r0 = uint4{g0.x, g0.y, g1.x, g1.y};
        r1 = uint4{u0.x, u0.y, u1.x, u1.y};
      } else {
        const int T0 = dfirst + kDownTiles * (v - ngs);
        uint2 d[kDownTiles];
#pragma unroll
        for (int u = 0; u < kDownTiles; ++u)
          d[u] = *reinterpret_cast<const uint2*>(dbase + (size_t)min(T0 + u, ntd - 1) * tile_d);
        r0 = uint4{d[0].x, d[0].y, d[1].x, d[1].y};
        r1 = uint4{d[2].x, d[2].y, d[3].x, d[3].y};
      }
      wr[0] = r0;
      wr[1] = r1;
    } else if (v < ngs) {
      const char* a0 = gbase + (size_t)(SPLIT ? 2 * v : v) * FB;
      const char* a1 = SPLIT ? gbase + (size_t)min(2 * v + 1, nchH - 1) * FB : ubase + (size_t)v * FB;
#pragma unroll
      for (int j = 0; j < WL; ++j) {
        wr[j] = *reinterpret_cast<const uint4*>(a0 + j * 1024);
        wr[WL + j] = *reinterpret_cast<const uint4*>(a1 + j * 1024);
      }
    } else {
      const int T0 = dfirst + kDownTiles * (v - ngs);
#pragma unroll
      for (int u = 0; u < kDownTiles; ++u) {
        const char* a = dbase + (size_t)min(T0 + u, ntd - 1) * tile_d;
#pragma unroll
        for (int j = 0; j < HL; ++j) wr[u * HL + j] = *reinterpret_cast<const uint4*>(a + j * 1024);
      }
    }
  };

  // FP8 scales, one per lane: gate/up over the K blocks of H (row block =
  // slice / 2), down per step (row block of the step's tiles, depth block =
  // slice / 2)
  float sg[SL], su[SL], sd = 0.f;
  f32x4 rsg = {0.f, 0.f, 0.f, 0.f}, rsu = rsg;  // ROWS: scales of this lane's 4 gate / up columns
  if (FP8 && ROWS) {
    const int c0 = (gon ? tg : slice * kColTiles) * kWaveCols + 4 * q;
    rsg = *reinterpret_cast<const f32x4*>((SPLIT && st ? SU : SG) + c0);
    if (!SPLIT) rsu = *reinterpret_cast<const f32x4*>(SU + c0);
  } else if (FP8) {
    const int kbH = H / kFp8Block, kbI = NI / kFp8Block;
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int c = lane + 64 * i;
      sg[i] = c < kbH ? (SPLIT && st ? SU : SG)[(size_t)(slice >> 1) * kbH + c] : 0.f;
      su[i] = c < kbH && !SPLIT ? SU[(size_t)(slice >> 1) * kbH + c] : 0.f;
    }
    if (lane < nd) sd = SD[(size_t)(min(dfirst + kDownTiles * lane, ntd - 1) / 8) * kbI + (slice >> 1)];
  }
  auto lane_scale = [&](const float (&r)[SL], int c) -> float {
    if (SL == 1 || c < 64) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[0]), c & 63));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[SL - 1]), c & 63));
  };

  const int xstride = H + kPad;
  const int astride = kSlice + kPad;
  const int aplane = rowcap * astride;
  const int pieces = H / 8;  // 16-byte pieces of one x row
  // ROWS: the expert's down row scales [H] in LDS, after act (and the up sums);
  // the first barrier of the pass below orders them before any read
  float* rsd = reinterpret_cast<float*>(as + 2 * aplane) + (SPLIT ? rowcap * kSlice : 0);
  if constexpr (FP8 && ROWS) {
    for (int i = tid; i < H / 4; i += kThreads)
      *reinterpret_cast<f32x4*>(rsd + 4 * i) = *reinterpret_cast<const f32x4*>(SD + 4 * i);
  }
  // MXFP4: the scale bytes of this workgroup (same place; ordered before any
  // read by the same barrier).  Gate / up: rows slice*64 .. +63 (rows past NI
  // repeat the last row; waves past NI multiply nothing), a contiguous run of
  // 64 * H/32 bytes copied a dword at a time; down: row h's bytes 2*hf and
  // 2*hf + 1 of its dword for chunk slice / 2.
  const int mxrow = mx_row_bytes(H);
  uint8_t* msg = reinterpret_cast<uint8_t*>(rsd);  // [kSlice][mxrow] gate, then up
  uint8_t* msu = msg + kSlice * mxrow;
  uint16_t* msd = reinterpret_cast<uint16_t*>(msu + kSlice * mxrow);  // [H]
  if constexpr (FP4) {
    const int rdw = H / 128;  // dwords per row
    for (int i = tid; i < kSlice * rdw; i += kThreads) {
      const int r = i / rdw, c = i % rdw;
      const size_t row = (size_t)min(slice * kSlice + r, NI - 1);
      const size_t off = row * (H / kMxBlock) + 4 * c;
      *reinterpret_cast<uint32_t*>(msg + r * mxrow + 4 * c) = *reinterpret_cast<const uint32_t*>(BG + off);
      *reinterpret_cast<uint32_t*>(msu + r * mxrow + 4 * c) = *reinterpret_cast<const uint32_t*>(BU + off);
    }
    for (int h = tid; h < H; h += kThreads)
      msd[h] = *reinterpret_cast<const uint16_t*>(BD + (size_t)h * (NI / kMxBlock) + 4 * (slice >> 1) + 2 * hf);
  }

  uint4 wb[NBUF][NL];
  for (int r0 = 0; r0 < rows; r0 += rowcap) {
    const int nr = min(rowcap, rows - r0);
    const int nrt = (nr + 15) >> 4;
    const int total = nr * pieces;

    // x rows of this pass: the first kXFirst pieces per thread are requested
    // before the weights (always-valid addresses, so the wait for them can
    // leave the weight loads in flight)
    auto x_piece = [&](int idx) -> uint4 {
      const int r = idx / pieces;
      const int tok = routed ? slots[r0 + r] / p.top_k : row_base + r0 + r;
      return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + (size_t)tok * H +
                                             (idx % pieces) * 8);
    };
    uint4 xv[kXFirst];
#pragma unroll
    for (int u = 0; u < kXFirst; ++u) xv[u] = x_piece(min(u * kThreads + tid, total - 1));
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j) load_step(j, wb[j]);
#pragma unroll
    for (int u = 0; u < kXFirst; ++u) {
      const int idx = u * kThreads + tid;
      if (idx < total) *reinterpret_cast<uint4*>(xs + (idx / pieces) * xstride + (idx % pieces) * 8) = xv[u];
    }
    for (int idx = kXFirst * kThreads + tid; idx < total; idx += kThreads)
      *reinterpret_cast<uint4*>(xs + (idx / pieces) * xstride + (idx % pieces) * 8) = x_piece(idx);

    // destination row of each of this lane's row tiles (slot, or token for the shared expert)
    int dst[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + r16;
      dst[rt] = r < nr ? (routed ? slots[r0 + r] : row_base + r0 + r) : 0;
    }
    __syncthreads();

    f32x4 ag[RT], au[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ag[rt] = au[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MXFP4 scales of the lane's gate/up rows for chunk c (st: 0 gate, 1 up):
    // halves h = 0, 1 of the chunk hold this lane's k in 32-deep block
    // 2h + q/2, whose byte is at bit 8 (2h + q/2) of the row's chunk dword
    auto gu_scales = [&](int st, int c, float (&f)[2]) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>((st ? msu : msg) + (ct * kWaveCols + r16) * mxrow + 4 * c);
      f[0] = e8m0_at(w, 8 * (q >> 1));
      f[1] = e8m0_at(w, 16 + 8 * (q >> 1));
    };
    // gate+up: operand s (8 consecutive k per lane) of stream st of a ring slot
    // (MXFP4: step s lies in half s / 2, scaled by f[s / 2])
    auto gu_op = [&](const uint4 (&wc)[NL], const float (&f)[2], int st, int s) -> bf16x8 {
      if constexpr (FP4) {
        const uint4 v = wc[st];
        const uint32_t d = s == 0 ? v.x : (s == 1 ? v.y : (s == 2 ? v.z : v.w));
        return fp4x8_to_bf16(d, f[s >> 1]);
      } else if constexpr (FP8) {
        const uint4 v = wc[st * WL + (s >> 1)];
        return (s & 1) ? fp8x8_to_bf16(v.z, v.w) : fp8x8_to_bf16(v.x, v.y);
      } else {
        return as_bf16x8(wc[st * WL + s]);
      }
    };
    // down: operand s (0 or 1, within the 64-deep half) of tile u of a ring slot
    auto dn_op = [&](const uint4 (&wc)[NL], float f, int u, int s) -> bf16x8 {
      if constexpr (FP4) {
        const uint4 v = wc[u >> 1];
        const uint32_t d = (u & 1) ? (s ? v.w : v.z) : (s ? v.y : v.x);
        return fp4x8_to_bf16(d, f);
      } else if constexpr (FP8) {
        const uint4 v = wc[u * HL];
        return (s & 1) ? fp8x8_to_bf16(v.z, v.w) : fp8x8_to_bf16(v.x, v.y);
      } else {
        return as_bf16x8(wc[u * HL + s]);
      }
    };

    // gate+up step v: chunk v of this wave's 16 gate and 16 up columns, or
    // (split) chunks 2v and 2v + 1 of its one stream; each accumulator sees the
    // MFMA sequence of the separate gate+up kernel
    auto gate_up = [&](const uint4 (&wc)[NL], int v) {
      if constexpr (SPLIT) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int c = 2 * v + c2;
          if (c < nchH) {
            float f[2] = {1.f, 1.f};
            if constexpr (FP4) gu_scales(st, c, f);
            const float scg = FP8 && !ROWS ? lane_scale(sg, c) : 1.f;
            const uint16_t* xb = xs + c * kKC;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              if (rt < nrt) {
                const int rowc = min(rt * 16 + r16, rowcap - 1);
                if (FP8) {
                  f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int s = 0; s < 4; ++s) {
                    const bf16x8 b =
                        as_bf16x8(*reinterpret_cast<const uint4*>(xb + rowc * xstride + k_of_step<BMAP>(s, q)));
                    t4 = mfma(gu_op(wc, f, c2, s), b, t4);
                  }
#pragma unroll
                  for (int i = 0; i < 4; ++i) ag[rt][i] = fmaf(ROWS ? rsg[i] : scg, t4[i], ag[rt][i]);
                } else {
#pragma unroll
                  for (int s = 0; s < 4; ++s) {
                    if (BMAP || c * kKC + s * 32 < H) {
                      const bf16x8 b =
                          as_bf16x8(*reinterpret_cast<const uint4*>(xb + rowc * xstride + k_of_step<BMAP>(s, q)));
                      ag[rt] = mfma(gu_op(wc, f, c2, s), b, ag[rt]);
                    }
                  }
                }
              }
            }
          }
        }
      } else {
        const int c = v;
        const float scg = FP8 && !ROWS ? lane_scale(sg, c) : 1.f;
        const float scu = FP8 && !ROWS ? lane_scale(su, c) : 1.f;
        float fg[2] = {1.f, 1.f}, fu[2] = {1.f, 1.f};
        if constexpr (FP4) {
          gu_scales(0, c, fg);
          gu_scales(1, c, fu);
        }
        const uint16_t* xb = xs + c * kKC;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (rt < nrt) {
            const int rowc = min(rt * 16 + r16, rowcap - 1);
            if (FP8) {
              f32x4 tg4 = {0.f, 0.f, 0.f, 0.f}, tu4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(xb + rowc * xstride + k_of_step<BMAP>(s, q)));
                tg4 = mfma(gu_op(wc, fg, 0, s), b, tg4);
                tu4 = mfma(gu_op(wc, fu, 1, s), b, tu4);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                ag[rt][i] = fmaf(ROWS ? rsg[i] : scg, tg4[i], ag[rt][i]);
                au[rt][i] = fmaf(ROWS ? rsu[i] : scu, tu4[i], au[rt][i]);
              }
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                if (BMAP || c * kKC + s * 32 < H) {
                  const bf16x8 b =
                      as_bf16x8(*reinterpret_cast<const uint4*>(xb + rowc * xstride + k_of_step<BMAP>(s, q)));
                  ag[rt] = mfma(gu_op(wc, fg, 0, s), b, ag[rt]);
                  au[rt] = mfma(gu_op(wc, fu, 1, s), b, au[rt]);
                }
              }
            }
          }
        }
      }
    };

    // act = silu(g) * u of this wave's columns into LDS as bf16 hi + lo (split:
    // the up waves hand their sums over through LDS and the gate waves write
    // act; every wave calls it then, for its barrier)
    float* ub = reinterpret_cast<float*>(as + 2 * aplane);  // split: [rowcap][kSlice] up sums
    auto act_to_lds = [&]() {
      if constexpr (SPLIT) {
        if (st == 1 && gon) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int r = rt * 16 + r16;
            if (rt < nrt && r < rowcap)
              *reinterpret_cast<f32x4*>(ub + r * kSlice + ct * kWaveCols + 4 * q) = ag[rt];
          }
        }
        __syncthreads();  // the up sums are in LDS
        if (st == 1 || !gon) return;
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = rt * 16 + r16;
        if (rt < nrt && r < rowcap) {
          f32x4 u = au[rt];
          if constexpr (SPLIT) u = *reinterpret_cast<const f32x4*>(ub + r * kSlice + ct * kWaveCols + 4 * q);
          uint16_t hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float f = silu_mul(ag[rt][i], u[i]);
            hi[i] = bf16_rne_bits(f);
            lo[i] = bf16_rne_bits(f - bf16_bits_to_f32(hi[i]));
          }
          uint2 h2, l2;
          h2.x = hi[0] | ((uint32_t)hi[1] << 16);
          h2.y = hi[2] | ((uint32_t)hi[3] << 16);
          l2.x = lo[0] | ((uint32_t)lo[1] << 16);
          l2.y = lo[2] | ((uint32_t)lo[3] << 16);
          uint16_t* d = as + r * astride + ct * kWaveCols + 4 * q;
          *reinterpret_cast<uint2*>(d) = h2;
          *reinterpret_cast<uint2*>(d + aplane) = l2;
        }
      }
    };

    // down step i: tiles T0 .. T0 + 3 of this wave, depth = the slice; per tile
    // the MFMA sequence of one 64-deep half in the separate down kernel
    auto down = [&](const uint4 (&wc)[NL], int i) {
      const int T0 = dfirst + kDownTiles * i;
      // MXFP4: the scale of this lane's row of each tile for the slice's half
      // (its 16 k in 32-deep block 2 hf + q/2: byte q/2 of the row's pair)
      float fd[kDownTiles];
#pragma unroll
      for (int u = 0; u < kDownTiles; ++u)
        fd[u] = FP4 ? e8m0_at(msd[min(T0 + u, ntd - 1) * kWaveCols + r16], 8 * (q >> 1)) : 1.f;
      const float sc = FP8 && !ROWS ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sd), i)) : 1.f;
      const int k0 = slice * kSlice;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt < nrt) {
          const int rowc = min(rt * 16 + r16, rowcap - 1);
          f32x4 t[kDownTiles];
#pragma unroll
          for (int u = 0; u < kDownTiles; ++u) t[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            if (BMAP || k0 + s * 32 < NI) {
              const uint16_t* ab = as + rowc * astride + k_of_step<BMAP>(s, q);
              const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(ab));
              const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(ab + aplane));
#pragma unroll
              for (int u = 0; u < kDownTiles; ++u) {
                const bf16x8 a = dn_op(wc, fd[u], u, s);
                t[u] = mfma(a, bh, t[u]);
                t[u] = mfma(a, bl, t[u]);
              }
            }
          }
          if (rt * 16 + r16 < nr) {
#pragma unroll
            for (int u = 0; u < kDownTiles; ++u) {
              if (T0 + u < ntd) {
                f32x4 s4 = {sc, sc, sc, sc};
                if constexpr (ROWS) s4 = *reinterpret_cast<const f32x4*>(rsd + (T0 + u) * kWaveCols + 4 * q);
                float4 o;
                o.x = FP8 ? mul_rn(s4[0], t[u][0]) : t[u][0];
                o.y = FP8 ? mul_rn(s4[1], t[u][1]) : t[u][1];
                o.z = FP8 ? mul_rn(s4[2], t[u][2]) : t[u][2];
                o.w = FP8 ? mul_rn(s4[3], t[u][3]) : t[u][3];
                *reinterpret_cast<float4*>(OUT + (size_t)dst[rt] * H + (T0 + u) * kWaveCols + 4 * q) = o;
              }
            }
          }
        }
      }
    };

    auto step = [&](const uint4 (&wc)[NL], int v) {
      if (v < ngs) {
        if (gon) gate_up(wc, v);
        if (v == ngs - 1) {
          if (SPLIT || gon) act_to_lds();
          __syncthreads();  // every wave's act columns are in LDS
        }
      } else {
        down(wc, v - ngs);
      }
    };

    // steady state: the load of step v + NBUF - 1 goes out before step v is multiplied
    for (int v0 = 0; v0 < nv; v0 += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        load_step(v0 + j + NBUF - 1, wb[(j + NBUF - 1) % NBUF]);
        if (v0 + j < nv) step(wb[j], v0 + j);
      }
    }
    __syncthreads();  // the next pass restages LDS
  }
}

// out[t] = bf16( sum_k fma(w[t,k], y_k, .) (k ascending, valid slots only) + shared ),
// shared = the sum of the shared expert's slices, added (ungated) or through a
// fused multiply-add with its gate sigmoid(x[t] . g) (the steps-path blend's
// order and gate helper),
// y_k = sum_j part[j][t*top_k+k] (j ascending from 0).  A workgroup covers 32
// four-column groups of one token with 8 k-lanes each: k-lane kk sums the slices
// of k = kk, kk + 8, ... (up to 16 slices' loads issued together, together with
// the slot's id and weight), and k-lane 0 combines them in k order through LDS.
constexpr int kBlendGroups = 32;
constexpr int kBlendKLanes = 8;
constexpr int kBlendKMax = 16;     // slots of one token one round holds in LDS
constexpr int kBlendSlices = 16;   // slices loaded per batch

template <typename IdT>
__global__ __launch_bounds__(256) void blend_parts_kernel(uint16_t* __restrict__ out, const float* __restrict__ part,
                                                          int nsl, const float* __restrict__ sh_part, int nssl,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ sh_gate,
                                                          const IdT* __restrict__ ids, const float* __restrict__ w,
                                                          int M, int H, int top_k, int E, int n) {
  __shared__ float4 ys[kBlendKMax][kBlendGroups];
  __shared__ float red[256];  // the gate's dot product
  const bool gated = nssl > 0 && sh_gate != nullptr;
  __shared__ float ws[kBlendKMax];  // the slots' weights
  __shared__ int wv[kBlendKMax];    // and whether their ids are in [0, E)
  const int g = threadIdx.x % kBlendGroups, kk = threadIdx.x / kBlendGroups;
  const int h = (blockIdx.x * kBlendGroups + g) * 4;
  const bool col = h < H;
  const size_t slice_stride = (size_t)n * H;
  for (int t = blockIdx.y; t < M; t += gridDim.y) {
    const float gate = gated ? mma::shared_gate256(x + (size_t)t * H, sh_gate, H, red) : 1.f;
    const size_t slot0 = (size_t)t * top_k;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int kb = 0; kb < top_k; kb += kBlendKMax) {
      const int kn = min(kBlendKMax, top_k - kb);
      for (int k = kk; k < kn; k += kBlendKLanes) {
        if (g == 0) {
          const IdT id = ids[slot0 + kb + k];
          wv[k] = id >= 0 && id < (IdT)E;
          ws[k] = w[slot0 + kb + k];
        }
        if (col) {
          const float* pp = part + (slot0 + kb + k) * H + h;
          float4 y = {0.f, 0.f, 0.f, 0.f};
          for (int jb = 0; jb < nsl; jb += kBlendSlices) {
            float4 v[kBlendSlices];
#pragma unroll
            for (int j = 0; j < kBlendSlices; ++j)
              v[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(jb + j, nsl - 1) * slice_stride);
#pragma unroll
            for (int j = 0; j < kBlendSlices; ++j) {
              if (jb + j < nsl) {
                y.x = add_rn(y.x, v[j].x);
                y.y = add_rn(y.y, v[j].y);
                y.z = add_rn(y.z, v[j].z);
                y.w = add_rn(y.w, v[j].w);
              }
            }
          }
          ys[k][g] = y;
        }
      }
      __syncthreads();
      if (col && kk == 0) {
        for (int k = 0; k < kn; ++k) {
          if (!wv[k]) continue;
          const float wk = ws[k];
          const float4 y = ys[k][g];
          a0 = fmaf(wk, y.x, a0);
          a1 = fmaf(wk, y.y, a1);
          a2 = fmaf(wk, y.z, a2);
          a3 = fmaf(wk, y.w, a3);
        }
      }
      __syncthreads();  // ys, ws, wv are rewritten by the next k block or token
    }
    if (col && kk == 0) {
      if (nssl > 0) {
        const float* pp = sh_part + (size_t)t * H + h;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        for (int j = 0; j < nssl; ++j) {
          const float4 v = *reinterpret_cast<const float4*>(pp + (size_t)j * M * H);
          s0 = add_rn(s0, v.x);
          s1 = add_rn(s1, v.y);
          s2 = add_rn(s2, v.z);
          s3 = add_rn(s3, v.w);
        }
        if (gated) {
          a0 = fmaf(gate, s0, a0);
          a1 = fmaf(gate, s1, a1);
          a2 = fmaf(gate, s2, a2);
          a3 = fmaf(gate, s3, a3);
        } else {
          a0 += s0;
          a1 += s1;
          a2 += s2;
          a3 += s3;
        }
      }
      uint2 packed;
      packed.x = bf16_rne_out(a0) | (bf16_rne_out(a1) << 16);
      packed.y = bf16_rne_out(a2) | (bf16_rne_out(a3) << 16);
      *reinterpret_cast<uint2*>(out + (size_t)t * H + h) = packed;
    }
  }
}

// waves per workgroup: 8 (gate and up on separate waves) for narrow widths of
// wide layers (measured: M = 1 at top-8 over 2048 x 768 experts 6% faster; M = 2
// even; the 256-wide layer of 8 experts 9% slower)
inline int layer_waves(int n, int H) { return n <= kNarrowSlots && H >= kNarrowMinH ? 2 * kColTiles : kColTiles; }

template <int FMT, bool ROWS, int RT, typename IdT, int W>
hipError_t launch_kernel(const FusedLayerArgs& a, int rowcap, hipStream_t s) {
  auto kern = layer_kernel<FMT, ROWS, RT, IdT, W>;
  const size_t xs = x_lds_bytes(rowcap, a.H);
  const size_t ab = act_lds_bytes(rowcap, W == 2 * kColTiles) + (ROWS ? (size_t)a.H * 4 : 0) +
                    (FMT == kFmtFP4 ? mx_scale_lds_bytes(a.H) : 0);
  const size_t lds = xs + ab + align_lds_bytes(a.E, a.n, W);
  static std::atomic<size_t> allowed[kMaxCachedDevices];
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds, allowed);
  if (e != hipSuccess) return e;
  const int nsl = (a.I + kSlice - 1) / kSlice;
  const int nssl = a.sw[0] != nullptr ? (a.S + kSlice - 1) / kSlice : 0;
  const int groups = a.sw[0] != nullptr ? (a.M + rowcap - 1) / rowcap : 0;
  const dim3 grid(std::max(nsl, nssl), a.cap + groups);
  hipLaunchKernelGGL(kern, grid, dim3(W * 64), lds, s, a, rowcap, xs, ab);
  return hipGetLastError();
}

template <int FMT, bool ROWS, typename IdT>
hipError_t launch_rt(const FusedLayerArgs& a, hipStream_t s) {
  const int rowcap = grouped_rows_per_pass(a.M);
  if (layer_waves(a.n, a.H) == 2 * kColTiles) return launch_kernel<FMT, ROWS, 1, IdT, 2 * kColTiles>(a, rowcap, s);
  switch (rowcap <= 16 ? 1 : rowcap / 16) {
    case 1: return launch_kernel<FMT, ROWS, 1, IdT, kColTiles>(a, rowcap, s);
    case 2: return launch_kernel<FMT, ROWS, 2, IdT, kColTiles>(a, rowcap, s);
    default: return launch_kernel<FMT, ROWS, 4, IdT, kColTiles>(a, rowcap, s);
  }
}

template <int FMT, typename IdT>
hipError_t launch_scales(const FusedLayerArgs& a, hipStream_t s) {
  if constexpr (FMT == kFmtFP8)
    if (a.scale_rows) return launch_rt<FMT, true, IdT>(a, s);
  return launch_rt<FMT, false, IdT>(a, s);
}

template <typename IdT>
hipError_t launch_blend(const FusedLayerArgs& a, hipStream_t s) {
  const int nsl = (a.I + kSlice - 1) / kSlice;
  const int nssl = a.sw[0] != nullptr ? (a.S + kSlice - 1) / kSlice : 0;
  const dim3 grid((a.H / 4 + kBlendGroups - 1) / kBlendGroups, a.M < 65535 ? a.M : 65535);
  hipLaunchKernelGGL(blend_parts_kernel<IdT>, grid, dim3(256), 0, s, a.out, a.part, nsl, a.sh_part, nssl,
                     static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.sh_gate),
                     static_cast<const IdT*>(a.ids), a.topk_weights, a.M, a.H, a.top_k, a.E, a.n);
  return hipGetLastError();
}

}  // namespace layer_detail

bool fused_layer_fits(int fmt, bool scale_rows, int64_t M, int H, int I, int S, int E, int top_k) {
  using namespace layer_detail;
  const bool fp8 = fmt == kFmtFP8;
  const int64_t n = M * top_k;
  if (n < 1 || n > kFusedLayerMaxSlots) return false;
  if (fp8 && H > kMaxScaleBlocks * kFp8Block) return false;
  (void)I;
  (void)S;
  const int rowcap = grouped_rows_per_pass(M);
  if (rowcap > kMaxRowCap) return false;
  const int waves = layer_waves((int)n, H);
  const size_t lds = x_lds_bytes(rowcap, H) + act_lds_bytes(rowcap, waves == 2 * kColTiles) +
                     (fp8 && scale_rows ? (size_t)H * 4 : 0) + (fmt == kFmtFP4 ? mx_scale_lds_bytes(H) : 0) +
                     align_lds_bytes(E, (int)n, waves);
  return lds <= kLdsBudget;
}

hipError_t launch_layer_partials(const FusedLayerArgs& a, int fmt, hipStream_t s) {
  using namespace layer_detail;
  if (fmt == kFmtFP8) return a.ids64 ? launch_scales<kFmtFP8, int64_t>(a, s) : launch_scales<kFmtFP8, int32_t>(a, s);
  if (fmt == kFmtFP4) return a.ids64 ? launch_scales<kFmtFP4, int64_t>(a, s) : launch_scales<kFmtFP4, int32_t>(a, s);
  return a.ids64 ? launch_scales<kFmtBF16, int64_t>(a, s) : launch_scales<kFmtBF16, int32_t>(a, s);
}

hipError_t launch_blend_partials(const FusedLayerArgs& a, hipStream_t s) {
  using namespace layer_detail;
  return a.ids64 ? launch_blend<int64_t>(a, s) : launch_blend<int32_t>(a, s);
}

}  // namespace moe
