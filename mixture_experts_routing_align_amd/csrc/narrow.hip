// Narrow-width MoE layer for gfx950: a few tokens (n = M * top_k slots, at
// most kNarrowLayerMaxSlots), FP8 tiled weights.  Two launches.
//
// What is computed is the layer of the single pass and the steps path
// (metrale forward_nvfp4_grouped_decode.rs: sort, gate+up+SiLU, down, blend;
// the FP8 block or row scales of fp8_moe_grouped.rs), with the same bits:
//   act[s, c] = silu(g) * u,  g = sum over 128-deep chunks, ascending, of
//               fma(scale_c, (4-step MFMA sum of chunk c), g)   (u likewise)
//   y[s, h]   = sum over 64-deep halves, ascending, of scale * (2-step MFMA
//               sum of the half over bf16 hi + lo of act), rounded adds
//   out[t, h] = bf16( sum_k fma(w[t,k], y[t*top_k+k, h], .) (+ shared) )
//
// Decomposition.  At one token the layer is 8 experts of weights; the single
// pass streams them with 96 workgroups, so most compute units sit idle, and a
// wave's stream rate is bounded by its own bytes in flight.  Here:
//  1. gate+up: one workgroup per (slot that first names its expert, or the
//     shared expert) x 16-column tile.  Its 8 waves split the depth H: wave w
//     streams chunks [w*cw, (w+1)*cw) of the tile's gate and up rows and
//     leaves each chunk's MFMA sums in LDS; after one barrier a thread per
//     (row, column) runs the chunk chain in ascending order and writes act
//     (float32, by slot).  One more workgroup writes the alignment tables.
//  2. down + blend: one workgroup of 16 waves per 8 rows of H (half a 16-row
//     tile: a compute unit streams at a bounded rate, so the launch spreads
//     its bytes over as many units as it can).  It stages every slot's act
//     row in LDS (bf16 hi + lo), its waves share out the (expert, 64-deep
//     half) items and leave each half's scaled sum per (slot, row) in LDS;
//     then the halves are summed in ascending order and the token's slots
//     blended in k order, plus the shared expert.
// Depth splits only where the other paths already form separate sums (a
// chunk's 4 MFMA steps, a half's 2), and every chain runs in one thread in
// their order, so every path gives the same bits.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "align_device.h"
#include "mma_common.h"
#include "moe_internal.h"

namespace moe {
namespace narrow_detail {

using namespace mma;

constexpr int kGuWaves = 8;
constexpr int kGuThreads = kGuWaves * 64;
constexpr int kDnWaves = 16;
constexpr int kDnThreads = kDnWaves * 64;
constexpr int kMaxRT = 2;                        // row tiles: an expert holds at most 32 slots
constexpr int kDnRows = 8;                       // rows of H per down workgroup: half a 16-row tile
constexpr int kMaxSlots = kNarrowLayerMaxSlots;  // one wave's lanes
constexpr int kChunkBytes = kWaveCols * kKC;     // one 16 x 128 FP8 fragment: 2 KB
constexpr int kNbuf = 2;                         // steps in the gate+up register ring
constexpr int kNbufDn = 8;                       // items in the down register ring (1 KB each)
constexpr size_t kLdsBudget = 96 * 1024;
constexpr int kMaxChunks = 128;                  // depth H in 128-deep chunks (H <= 16384)
constexpr int kXFirst = 2;                       // x pieces per thread requested first
constexpr int kActPer = 6;                       // act float4s per thread requested first
static_assert(kMaxSlots <= 32, "slots are grouped by one wave's ballots and take at most 2 row tiles");

// LDS bytes of the gate+up launch: x rows of every token, then the chunk sums
// [nch][2][n rows][16] (the tables' workgroup uses that region for the align).
__host__ __device__ inline size_t gu_x_bytes(int M, int H) { return (size_t)M * (H + kPad) * 2; }
__host__ __device__ inline size_t gu_sum_bytes(int H, int n, int E) {
  const size_t sums = (size_t)(H / kKC) * 2 * n * kWaveCols * 4;
  const size_t align = ((size_t)kGuWaves * E + E + (E + 1) + E + 2 * kGuWaves + 2 + n) * sizeof(int);
  return std::max(sums, align);
}
// LDS bytes of the down + blend launch: act (hi, lo) by slot, the shared
// expert's act by token, the halves' sums, then y and the shared sums.
__host__ __device__ inline size_t dn_bytes(int M, int n, int I, int S) {
  return (size_t)n * (I + kPad) * 4 + (size_t)M * (S + kPad) * 4 + (size_t)n * (I / 64) * kDnRows * 4 +
         (size_t)M * (S / 64) * kDnRows * 4 + (size_t)(n + M) * kDnRows * 4;
}

// The slots of this launch grouped by expert, by wave 0: leader[s] = the first
// slot naming s's expert (-1: id out of range), group of each leader in
// first-slot order, each group's slots ascending.
struct SlotGroups {
  int ids[kMaxSlots];                 // expert of each slot, -1 out of range
  int leader[kMaxSlots];
  int group[kMaxSlots];               // group index of the slot's expert
  int expert[kMaxSlots];              // expert of each group
  int count[kMaxSlots];               // slots of each group
  int rows[kMaxSlots * kMaxSlots];    // [group][rank] slot
  int ngroups;
};

// Loads in the prologues below are unconditional and issued in the order their
// data is needed: a wave's loads complete in order, and a load under a
// divergent condition makes the compiler wait for every outstanding load at
// the next use of any of them.  Indices past the end wrap around (clamping
// would send every surplus lane of every workgroup to one cache line).

// Call from every thread with the raw id of slot (lane & 63) (any value past
// n); ends with a barrier.
template <typename IdT>
__device__ void group_slots(IdT raw, int n, int E, SlotGroups& g) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    const bool valid = lane < n && raw >= 0 && raw < (IdT)E;
    const int e = valid ? (int)raw : -1;
    const uint64_t m = align_dev::same_expert_mask(e, valid, align_dev::id_bits(E));
    const uint64_t leaders = __ballot(valid && align_dev::is_leader(m, lane));
    const int lead = valid ? __ffsll((unsigned long long)m) - 1 : -1;
    const int grp = valid ? __popcll(leaders & align_dev::lanes_below(lead)) : -1;
    if (lane < n) {
      g.ids[lane] = e;
      g.leader[lane] = lead;
      g.group[lane] = grp;
    }
    if (valid) g.rows[grp * kMaxSlots + __popcll(m & align_dev::lanes_below(lane))] = lane;
    if (valid && lead == lane) {
      g.expert[grp] = e;
      g.count[grp] = __popcll(m);
    }
    if (lane == 0) g.ngroups = __popcll(leaders);
  }
  __syncthreads();
}

// A value every lane of the wave holds alike (read from LDS, so the compiler
// keeps it per lane) moved to a scalar register, so that the index and address
// arithmetic built on it runs once per wave.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A wave's 8 FP8 codes of step s (0..3) from its two 16-byte fragment loads.
__device__ __forceinline__ bf16x8 fp8_step(const uint4& lo, const uint4& hi, int s) {
  const uint4 v = s < 2 ? lo : hi;
  return (s & 1) ? fp8x8_to_bf16(v.z, v.w) : fp8x8_to_bf16(v.x, v.y);
}

// ---- launch 1: gate+up, depth split over the waves
// grid (ceil(max(I, S) / 16), n + (S > 0) + 1): rows y < n the slots, then the
// shared expert, then the tables (column 0 only); ROWS: FP8 row scales [E, N];
// RT: row tiles of an expert (1 when n <= 16, so that no expert holds more).
template <bool ROWS, typename IdT, int RT>
__global__ __launch_bounds__(kGuThreads) void narrow_gate_up_kernel(FusedLayerArgs p, size_t x_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ SlotGroups g;
  __shared__ float s_csc[2 * kMaxChunks];  // block scales of the chain: gate chunks, then up

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int tl = blockIdx.x, y = blockIdx.y;
  const int n = p.n, E = p.E, H = p.H;
  const bool routed = y < n;
  const IdT* ids = static_cast<const IdT*>(p.ids);
  uint16_t* xs = lds;                                                                  // [M][H + pad]
  float* sums = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + x_bytes);      // [nch][2][n][16]

  if (y == n + (p.S > 0 ? 1 : 0)) {
    // the alignment tables (LDS: the chunk-sum region)
    if (tl != 0) return;
    int* a = reinterpret_cast<int*>(sums);
    const align_dev::ExpertLds s{a, a + kGuWaves * E, a + kGuWaves * E + E, a + kGuWaves * E + 2 * E + 1,
                                 a + kGuWaves * E + 3 * E + 1, a + kGuWaves * E + 3 * E + 1 + kGuWaves,
                                 a + kGuWaves * E + 3 * E + 1 + 2 * kGuWaves};
    const int nbits = align_dev::id_bits(E);
    align_dev::count_pass<kGuWaves>(ids, n, E, nbits, s.cnt);
    align_dev::expert_scan<kGuWaves>(s, E, p.BS);
    align_dev::scatter_pass<kGuWaves>(ids, n, E, nbits, s.cnt, s.off, p.tables.sorted_token_ids,
                                      p.tables.token_to_perm);
    align_dev::write_rest<kGuWaves>(s, n, E, p.BS, p.max_total, p.cap, p.tables);
    return;
  }
  const int N = routed ? p.I : p.S;
  if (tl * kWaveCols >= N) return;

  // requests in need order: this slot's expert (the weight addresses wait for
  // it), every slot's id (the grouping), the first x pieces, then the weights
  // and the chain's scales
  const IdT vy = ids[routed ? y : 0];
  const IdT raw = ids[min(lane, n - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep the grouping's load ahead of the x loads
  const int xstride = H + kPad, pieces = H / 8, xtotal = p.M * pieces;
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  auto x_piece = [&](int idx) -> uint4 {
    return *reinterpret_cast<const uint4*>(X + (size_t)(idx / pieces) * H + (idx % pieces) * 8);
  };
  uint4 xv[kXFirst];
#pragma unroll
  for (int u = 0; u < kXFirst; ++u) xv[u] = x_piece((u * kGuThreads + tid) % xtotal);
  if (routed && (vy < 0 || vy >= (IdT)E)) return;
  const int e = routed ? (int)vy : -1;

  // this wave's chunks of the tile's gate and up rows (a wave with none
  // loads the tile's last chunk and multiplies nothing)
  const int nch = H / kKC;
  const int cw = (nch + kGuWaves - 1) / kGuWaves;
  const int c0 = min(nch, wave * cw), nv = min(nch, c0 + cw) - c0;
  const size_t tile_bytes = (size_t)H * kWaveCols;
  const char* G = static_cast<const char*>(routed ? p.w[0] : p.sw[0]) + (routed ? (size_t)e * N * H : 0);
  const char* U = static_cast<const char*>(routed ? p.w[1] : p.sw[1]) + (routed ? (size_t)e * N * H : 0);
  G += (size_t)tl * tile_bytes + lane * 16;
  U += (size_t)tl * tile_bytes + lane * 16;
  auto load = [&](int v, uint4 (&w)[4]) {
    const size_t c = (size_t)min(c0 + v, nch - 1) * kChunkBytes;
    w[0] = *reinterpret_cast<const uint4*>(G + c);
    w[1] = *reinterpret_cast<const uint4*>(G + c + 1024);
    w[2] = *reinterpret_cast<const uint4*>(U + c);
    w[3] = *reinterpret_cast<const uint4*>(U + c + 1024);
  };
  uint4 wb[kNbuf][4];
#pragma unroll
  for (int j = 0; j < kNbuf - 1; ++j) load(j, wb[j]);

  // the chain's scales: block scales, one per chunk for the whole tile
  // (thread c < nch: gate, nch <= c < 2 nch: up), kept in registers until the
  // stream is done; row scales, the column tid % 16 this thread chains
  const float* SG = static_cast<const float*>(routed ? p.s[0] : p.ss[0]);
  const float* SU = static_cast<const float*>(routed ? p.s[1] : p.ss[1]);
  const int scol = tl * kWaveCols + tid % kWaveCols;
  float csc = 0.f, rsg = 0.f, rsu = 0.f;
  if constexpr (ROWS) {
    rsg = SG[(routed ? (size_t)e * N : 0) + scol];
    rsu = SU[(routed ? (size_t)e * N : 0) + scol];
  } else {
    const size_t blocks = (size_t)(N / kFp8Block) * (H / kFp8Block);
    const size_t base = (routed ? (size_t)e * blocks : 0) + (size_t)(tl * kWaveCols / kFp8Block) * (H / kFp8Block);
    const int c = min(tid, 2 * nch - 1);
    csc = (c < nch ? SG : SU)[base + c % nch];
  }

  // the expert's rows: its slots in ascending order (the workgroup of a slot
  // that is not its expert's first has nothing to do), or every token
  group_slots(raw, n, E, g);
  int nr, grp = -1;
  if (routed) {
    if (uniform(g.leader[y]) != y) return;
    grp = uniform(g.group[y]);
    nr = uniform(g.count[grp]);
  } else {
    nr = p.M;
  }

  // every token's x row
#pragma unroll
  for (int u = 0; u < kXFirst; ++u) {
    const int idx = u * kGuThreads + tid;
    if (idx < xtotal) *reinterpret_cast<uint4*>(xs + (idx / pieces) * xstride + (idx % pieces) * 8) = xv[u];
  }
  // the rest, if any, behind a block-uniform test: a divergent loop's latch
  // would wait for every outstanding load even when it runs no iteration
  if (kXFirst * kGuThreads < xtotal) {
    for (int idx = kXFirst * kGuThreads + tid; idx < xtotal; idx += kGuThreads)
      *reinterpret_cast<uint4*>(xs + (idx / pieces) * xstride + (idx % pieces) * 8) = x_piece(idx);
  }
  __syncthreads();

  // row r of the tile is slot rows[r] (token slot / top_k), or token r (shared)
  const int nrt = (nr + 15) >> 4;
  int tok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = min(rt * 16 + r16, nr - 1);
    tok[rt] = routed ? g.rows[grp * kMaxSlots + r] / p.top_k : r;
  }
  auto compute = [&](const uint4 (&w)[4], int c) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt < nrt) {
        const uint16_t* xb = xs + tok[rt] * xstride + c * kKC;
        f32x4 tg = {0.f, 0.f, 0.f, 0.f}, tu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(xb + k_of_step<true>(s, q)));
          tg = mfma(fp8_step(w[0], w[1], s), b, tg);
          tu = mfma(fp8_step(w[2], w[3], s), b, tu);
        }
        const int r = rt * 16 + r16;
        if (r < nr) {
          *reinterpret_cast<f32x4*>(sums + (((size_t)c * 2 + 0) * n + r) * kWaveCols + 4 * q) = tg;
          *reinterpret_cast<f32x4*>(sums + (((size_t)c * 2 + 1) * n + r) * kWaveCols + 4 * q) = tu;
        }
      }
    }
  };
  // (the down launch's ring below says why the loads are not conditional)
  if (nv <= kNbuf - 1) {
#pragma unroll
    for (int j = 0; j < kNbuf - 1; ++j)
      if (j < nv) compute(wb[j], c0 + j);
  } else {
    for (int v0 = 0; v0 < nv; v0 += kNbuf) {
#pragma unroll
      for (int j = 0; j < kNbuf; ++j) {
        load(min(v0 + j + kNbuf - 1, nv - 1), wb[(j + kNbuf - 1) % kNbuf]);
        if (v0 + j < nv) compute(wb[j], c0 + v0 + j);
      }
    }
  }
  if (!ROWS && tid < 2 * nch) s_csc[tid] = csc;
  __syncthreads();

  // the chunk chains, one thread per (row, column): the scaled chunk sums in
  // ascending chunk order (fused multiply-add), then silu(g) * u
  for (int j = tid; j < nr * kWaveCols; j += kGuThreads) {
    const int r = j / kWaveCols, col = j % kWaveCols;  // col = tid % 16
    const int gcol = tl * kWaveCols + col;
    float gs = 0.f, us = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float scg = ROWS ? rsg : s_csc[c], scu = ROWS ? rsu : s_csc[nch + c];
      gs = fmaf(scg, sums[(((size_t)c * 2 + 0) * n + r) * kWaveCols + col], gs);
      us = fmaf(scu, sums[(((size_t)c * 2 + 1) * n + r) * kWaveCols + col], us);
    }
    const float a = silu_mul(gs, us);
    if (routed)
      p.act[(size_t)g.rows[grp * kMaxSlots + r] * p.I + gcol] = a;
    else
      p.sh_act[(size_t)r * p.S + gcol] = a;
  }
}

// ---- launch 2: down + blend per 8 rows of H
// grid (H / 8); ROWS: FP8 row scales [E, H].  The MFMA tile is 16 rows of H:
// lanes of the other half load their partner lane's address (the same cache
// lines), and the duplicate output rows are dropped.
// AP: act float4 pieces each thread requests first (the launcher's ceil(act
// pieces / threads), at most kActPer); RT as for the gate+up launch.
template <bool ROWS, typename IdT, int AP, int RT>
__global__ __launch_bounds__(kDnThreads) void narrow_down_blend_kernel(FusedLayerArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ SlotGroups g;
  __shared__ float s_w[kMaxSlots];
  __shared__ float s_gate[kMaxSlots];
  __shared__ float red[256];
  __shared__ float s_rsd[(kMaxSlots + 1) * kDnRows];  // row scales: this workgroup's rows of each group's expert

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int T = blockIdx.x >> 1, hb = blockIdx.x & 1;  // rows 16T + 8hb .. + 7 of H
  const int row0 = T * kWaveCols + hb * kDnRows;
  const int src_lane = (lane & ~15) | (hb * kDnRows + (lane & 7));  // the lane whose row this lane loads
  const int n = p.n, E = p.E, H = p.H, I = p.I, S = p.S, M = p.M;
  const int nhI = I / 64, nhS = S / 64;
  const int astride = I + kPad, sstride = S + kPad;
  uint16_t* ah = lds;                                   // [n][I + pad] act, bf16 hi
  uint16_t* al = ah + (size_t)n * astride;              //                   and lo
  uint16_t* sh = al + (size_t)n * astride;              // [M][S + pad] shared act hi
  uint16_t* sl = sh + (size_t)M * sstride;              //                         lo
  float* P = reinterpret_cast<float*>(sl + (size_t)M * sstride);  // [n][nhI][8] scaled half sums
  float* Psh = P + (size_t)n * nhI * kDnRows;                     // [M][nhS][8]
  float* Y = Psh + (size_t)M * nhS * kDnRows;                     // [n][8]
  float* SY = Y + (size_t)n * kDnRows;                            // [M][8]

  const IdT* ids = static_cast<const IdT*>(p.ids);
  // requests in need order: every slot's id (the grouping) and weight, the
  // act rows, then the down weights
  const IdT raw = ids[min(lane, n - 1)];
  const float wslot = p.topk_weights[min(tid, n - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep the grouping's loads ahead of the act loads
  const int na = n * (I / 4), atot = na + M * (S / 4);  // float4 pieces of act, then of the shared act
  const float* ACT = p.act;
  const float* SHACT = S > 0 ? p.sh_act : p.act;
  auto act_piece = [=](int idx) -> float4 {
    const float* src = idx < na ? ACT + (size_t)idx * 4 : SHACT + (size_t)(idx - na) * 4;
    return *reinterpret_cast<const float4*>(src);
  };
  float4 av[AP];
#pragma unroll
  for (int u = 0; u < AP; ++u) av[u] = act_piece((u * kDnThreads + tid) % atot);
  group_slots(raw, n, E, g);
  if (tid < n) s_w[tid] = wslot;
  const int ngr = uniform(g.ngroups);

  // the down weights this workgroup streams: items (group, half) of the
  // routed experts, then the halves of the shared expert; wave w takes a
  // contiguous run of items (so its loads walk each tile's halves in order),
  // each with its FP8 scale (block: the half's 128 x 128 block; rows: this
  // lane's 4 rows of H)
  const int nitems = ngr * nhI + (S > 0 ? nhS : 0);
  const int per = (nitems + kDnWaves - 1) / kDnWaves;
  const int i0 = min(nitems, wave * per), ni = min(nitems, i0 + per) - i0;
  const float* SD = static_cast<const float*>(p.s[2]);
  const float* SSD = static_cast<const float*>(p.ss[2]);
  // Item descriptors, one per lane and all at once: lane j describes this
  // wave's item i0 + j (clamped; a layer with no item describes item 0 of
  // the routed weights, which exist): its group (ngr: the shared expert), its
  // half, its weight offset and its FP8 scale.  Item j then only reads them
  // with readlane, so the per-item bookkeeping is not repeated on the scalar
  // unit the compute unit's waves share.
  const bool any = nitems > 0;
  const int il = max(0, min(i0 + min(lane, max(ni - 1, 0)), nitems - 1));
  const bool lrt = il < ngr * nhI || !any;
  const int lg = lrt ? (any ? il / nhI : 0) : ngr;
  const int lh = lrt ? (any ? il % nhI : 0) : il - ngr * nhI;
  const int lK = lrt ? I : S;
  const int le = lrt && any ? g.expert[lg] : 0;
  const uint64_t loff = (uint64_t)le * H * lK + (uint64_t)T * kWaveCols * lK + (uint64_t)lh * 1024;
  float lsc = 0.f;  // block scale of the item (unused with row scales)
  if constexpr (!ROWS) {
    const size_t blocks = (size_t)(H / kFp8Block) * (lK / kFp8Block);
    lsc = (lrt ? SD : SSD)[(size_t)le * blocks + (size_t)(T * kWaveCols / kFp8Block) * (lK / kFp8Block) + (lh >> 1)];
  }
  // row scales: thread j < (ngr + 1) * 8 loads row j % 8 of this workgroup's
  // rows for group j / 8 (ngr: the shared expert); kept in LDS for the items
  float rsd = 0.f;
  const int rg = min(tid / kDnRows, ngr);
  if constexpr (ROWS) {
    const bool rr = rg < ngr || S == 0;
    rsd = (rr ? SD + (size_t)(rg < ngr ? g.expert[rg] : 0) * H : SSD)[row0 + tid % kDnRows];
  }
  const char* W2 = static_cast<const char*>(p.w[2]);
  const char* SW2 = static_cast<const char*>(S > 0 ? p.sw[2] : p.w[2]);
  auto item_g = [=](int j) { return __builtin_amdgcn_readlane(lg, j); };
  auto load_item = [=](int j, uint4& w) {
    const uint64_t off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)loff, j)) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(loff >> 32), j) << 32);
    const bool routed_item = item_g(j) < ngr || !any;
    w = *reinterpret_cast<const uint4*>((routed_item ? W2 : SW2) + off + src_lane * 16);
  };
  uint4 wb[kNbufDn];
#pragma unroll
  for (int j = 0; j < kNbufDn - 1; ++j) load_item(min(j, max(ni - 1, 0)), wb[j]);

  // act rows as bf16 hi + lo (the split every path's down applies); a slot
  // whose id is out of range has no act row and is never read
  auto split4 = [](float4 v, uint2& hi2, uint2& lo2) {
    const float f[4] = {v.x, v.y, v.z, v.w};
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = bf16_rne_bits(f[i]);
      lo[i] = bf16_rne_bits(f[i] - bf16_bits_to_f32(hi[i]));
    }
    hi2.x = hi[0] | ((uint32_t)hi[1] << 16);
    hi2.y = hi[2] | ((uint32_t)hi[3] << 16);
    lo2.x = lo[0] | ((uint32_t)lo[1] << 16);
    lo2.y = lo[2] | ((uint32_t)lo[3] << 16);
  };
  auto store_act = [=](int idx, float4 v) {
    uint2 hi2, lo2;
    split4(v, hi2, lo2);
    uint16_t* hp;
    if (idx < na) {
      const int s2 = idx / (I / 4), c = (idx % (I / 4)) * 4;
      hp = ah + (size_t)s2 * astride + c;
    } else {
      const int t = (idx - na) / (S / 4), c = ((idx - na) % (S / 4)) * 4;
      hp = sh + (size_t)t * sstride + c;
    }
    const size_t lo_off = idx < na ? (size_t)n * astride : (size_t)M * sstride;
    *reinterpret_cast<uint2*>(hp) = hi2;
    *reinterpret_cast<uint2*>(hp + lo_off) = lo2;
  };
#pragma unroll
  for (int u = 0; u < AP; ++u) {
    const int idx = u * kDnThreads + tid;
    if (idx < atot) store_act(idx, av[u]);
  }
  if (ROWS && tid < (ngr + 1) * kDnRows) s_rsd[tid] = rsd;
  if (AP * kDnThreads < atot) {  // block-uniform (see the x rows of the gate+up launch)
    for (int idx = AP * kDnThreads + tid; idx < atot; idx += kDnThreads) store_act(idx, act_piece(idx));
  }
  __syncthreads();

  // item j: the half's 2 MFMA steps over hi then lo, times its FP8 scale, per
  // (row of the item's expert, row of H)
  auto compute = [=](const uint4& v, int j) {
    const int gi = item_g(j), h = __builtin_amdgcn_readlane(lh, j);
    const bool routed_item = gi < ngr;
    const int nr = routed_item ? uniform(g.count[gi]) : M;
    f32x4 sc;
    if constexpr (ROWS) {
      sc = *reinterpret_cast<const f32x4*>(s_rsd + gi * kDnRows + 4 * (q & 1));
    } else {
      const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsc), j));
      sc = f32x4{v1, v1, v1, v1};
    }
    const uint16_t* bh = routed_item ? ah : sh;
    const uint16_t* bl = routed_item ? al : sl;
    const int stride = routed_item ? astride : sstride;
    const bf16x8 a0 = fp8x8_to_bf16(v.x, v.y), a1 = fp8x8_to_bf16(v.z, v.w);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt * 16 < nr) {
        const int r = min(rt * 16 + r16, nr - 1);
        const int src = routed_item ? g.rows[gi * kMaxSlots + r] : r;
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const size_t o = (size_t)src * stride + 64 * h + k_of_step<true>(s2, q);
          const bf16x8 a = s2 ? a1 : a0;
          t = mfma(a, as_bf16x8(*reinterpret_cast<const uint4*>(bh + o)), t);
          t = mfma(a, as_bf16x8(*reinterpret_cast<const uint4*>(bl + o)), t);
        }
        if (rt * 16 + r16 < nr && q < 2) {  // output rows 4q + i < 8: this half's rows
          f32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) o[k] = mul_rn(sc[k], t[k]);
          float* d = routed_item ? P + ((size_t)src * nhI + h) * kDnRows : Psh + ((size_t)src * nhS + h) * kDnRows;
          *reinterpret_cast<f32x4*>(d + 4 * q) = o;
        }
      }
    }
  };
  // A load under a condition would make every later wait a wait for all
  // loads, so: when the first loads already hold every item, no more loads;
  // else a ring whose loads are unconditional (past the last item they load
  // it again).
  if (ni <= kNbufDn - 1) {
#pragma unroll
    for (int j = 0; j < kNbufDn - 1; ++j)
      if (j < ni) compute(wb[j], j);
  } else {
    for (int v0 = 0; v0 < ni; v0 += kNbufDn) {
#pragma unroll
      for (int j = 0; j < kNbufDn; ++j) {
        load_item(min(v0 + j + kNbufDn - 1, ni - 1), wb[(j + kNbufDn - 1) % kNbufDn]);
        if (v0 + j < ni) compute(wb[j], v0 + j);
      }
    }
  }
  __syncthreads();

  // y of every slot and the shared expert's sum per token: halves in
  // ascending order, rounded adds from 0
  for (int j = tid; j < n * kDnRows; j += kDnThreads) {
    const int s = j / kDnRows, r = j % kDnRows;
    if (g.ids[s] < 0) continue;
    float yv = 0.f;
    for (int h = 0; h < nhI; ++h) yv = add_rn(yv, P[((size_t)s * nhI + h) * kDnRows + r]);
    Y[s * kDnRows + r] = yv;
  }
  for (int j = tid; j < M * kDnRows && S > 0; j += kDnThreads) {
    const int t = j / kDnRows, r = j % kDnRows;
    float sv = 0.f;
    for (int h = 0; h < nhS; ++h) sv = add_rn(sv, Psh[((size_t)t * nhS + h) * kDnRows + r]);
    SY[t * kDnRows + r] = sv;
  }
  const bool gated = S > 0 && p.sh_gate != nullptr;
  if (gated) {
    for (int t = 0; t < M; ++t) {
      const float gv = shared_gate256(static_cast<const uint16_t*>(p.x) + (size_t)t * H,
                                      static_cast<const uint16_t*>(p.sh_gate), H, red);
      if (tid == 0) s_gate[t] = gv;
    }
  }
  __syncthreads();

  // the blend: the token's valid slots in k order (fused multiply-add), then
  // the shared expert (through its gate, or added)
  for (int j = tid; j < M * kDnRows; j += kDnThreads) {
    const int t = j / kDnRows, r = j % kDnRows;
    float a = 0.f;
    for (int k = 0; k < p.top_k; ++k) {
      const int s = t * p.top_k + k;
      if (g.ids[s] >= 0) a = fmaf(s_w[s], Y[s * kDnRows + r], a);
    }
    if (S > 0) {
      if (gated)
        a = fmaf(s_gate[t], SY[t * kDnRows + r], a);
      else
        a += SY[t * kDnRows + r];
    }
    p.out[(size_t)t * H + row0 + r] = (uint16_t)bf16_rne_out(a);
  }
}

template <bool ROWS, typename IdT, int AP, int RT>
hipError_t launch_both(const FusedLayerArgs& a, hipStream_t s) {
  auto gu = narrow_gate_up_kernel<ROWS, IdT, RT>;
  auto dn = narrow_down_blend_kernel<ROWS, IdT, AP, RT>;
  const size_t xb = gu_x_bytes(a.M, a.H);
  const size_t lds_gu = xb + gu_sum_bytes(a.H, a.n, a.E);
  const size_t lds_dn = dn_bytes(a.M, a.n, a.I, a.S);
  static std::atomic<size_t> allowed_gu[kMaxCachedDevices], allowed_dn[kMaxCachedDevices];
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(gu), lds_gu, allowed_gu);
  if (e != hipSuccess) return e;
  e = allow_dynamic_lds(reinterpret_cast<const void*>(dn), lds_dn, allowed_dn);
  if (e != hipSuccess) return e;
  const int tiles = (std::max(a.I, a.S) + kWaveCols - 1) / kWaveCols;
  hipLaunchKernelGGL(gu, dim3(tiles, a.n + (a.S > 0 ? 1 : 0) + 1), dim3(kGuThreads), lds_gu, s, a, xb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dn, dim3(a.H / kDnRows), dim3(kDnThreads), lds_dn, s, a);
  return hipGetLastError();
}

template <bool ROWS, int AP, int RT>
hipError_t launch_ids(const FusedLayerArgs& a, hipStream_t s) {
  return a.ids64 ? launch_both<ROWS, int64_t, AP, RT>(a, s) : launch_both<ROWS, int32_t, AP, RT>(a, s);
}

template <bool ROWS, int AP>
hipError_t launch_rt(const FusedLayerArgs& a, hipStream_t s) {
  return a.n <= 16 ? launch_ids<ROWS, AP, 1>(a, s) : launch_ids<ROWS, AP, kMaxRT>(a, s);
}

template <bool ROWS>
hipError_t launch_ap(const FusedLayerArgs& a, hipStream_t s) {
  const int pieces = a.n * (a.I / 4) + a.M * (a.S / 4);
  const int ap = (pieces + kDnThreads - 1) / kDnThreads;
  if (ap <= 2) return launch_rt<ROWS, 2>(a, s);
  if (ap <= 4) return launch_rt<ROWS, 4>(a, s);
  return launch_rt<ROWS, kActPer>(a, s);
}

}  // namespace narrow_detail

bool narrow_layer_fits(int fmt, int64_t M, int H, int I, int S, int E, int top_k) {
  using namespace narrow_detail;
  const int64_t n = M * top_k;
  if (fmt != kFmtFP8 || n < 1 || n > kMaxSlots || H / kKC > kMaxChunks) return false;
  if (gu_x_bytes((int)M, H) + gu_sum_bytes(H, (int)n, E) > kLdsBudget) return false;
  // a down wave describes its items one per lane
  if (((int)n * (I / 64) + S / 64 + kDnWaves - 1) / kDnWaves > 64) return false;
  return dn_bytes((int)M, (int)n, I, S) <= kLdsBudget;
}

hipError_t launch_narrow_layer(const FusedLayerArgs& a, hipStream_t s) {
  using namespace narrow_detail;
  return a.scale_rows ? launch_ap<true>(a, s) : launch_ap<false>(a, s);
}

}  // namespace moe
