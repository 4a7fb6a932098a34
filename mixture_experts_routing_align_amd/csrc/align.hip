// Deterministic MoE token alignment for gfx950: one workgroup of 16 wave64s, or
// for many slots three launches over blocks of 1024 slots (see below).
//
// What it computes (nbxtensor 0.0.1 wheel page, moe_align.py: module docstring
// and the stage-1/2/3 kernel docstrings; metrale fp8_moe_grouped.rs:
// moe_fp8_grouped_sort): see align_device.h.  One launch, no atomics:
//   pass 1   per-wave per-expert counts from wave ballots (leaders only write),
//            every id requested up front and kept in registers;
//   scan     per-wave bases, padded exclusive offsets, ascending active list;
//   pass 2   stable scatter of every slot and token_to_perm;
//   rest     counts, offsets, active list, total, padding sentinels, block owners.
// The layer forward fuses the same steps into the gate+up kernel when the
// slot count is small (see grouped.hip); this kernel serves every size.
#include <hip/hip_runtime.h>

#include "align_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kAlignWaves = 16;
constexpr int kAlignThreads = kAlignWaves * 64;
constexpr int kMaxExperts = 1024;
constexpr int kAlignBlocksMinSlots = 4096;  // from here on the alignment runs over several blocks

// Below kAlignBlocksMinSlots each wave walks at most kWaveChunks chunks of 64
// slots: all of them are requested at once (before the count rows are
// cleared), and their ids and same-expert masks stay in registers from the
// count pass to the scatter pass.
constexpr int kWaveChunks = kAlignBlocksMinSlots / kAlignThreads;
static_assert(kWaveChunks * kAlignThreads == kAlignBlocksMinSlots, "whole chunks per wave");

template <typename IdT>
__global__ __launch_bounds__(kAlignThreads) void align_kernel(const IdT* __restrict__ ids, int n, int E, int BS,
                                                              int max_total, int cap, int nbits, AlignOut o) {
  __shared__ int cnt[kAlignWaves * kMaxExperts];  // [wave][expert]: counts, then bases
  __shared__ int s_count[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_active[kMaxExperts];
  __shared__ int s_wa[kAlignWaves], s_wb[kAlignWaves], s_scal[2];
  const align_dev::ExpertLds s{cnt, s_count, s_off, s_active, s_wa, s_wb, s_scal};
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int beg, end;
  align_dev::wave_range<kAlignWaves>(n, w, beg, end);

  int id[kWaveChunks];
  bool valid[kWaveChunks];
  uint64_t m[kWaveChunks];
#pragma unroll
  for (int j = 0; j < kWaveChunks; ++j) id[j] = align_dev::load_id(ids, beg + 64 * j + lane, end, E, valid[j]);
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) cnt[i] = 0;
  __syncthreads();

  // pass 1: per-wave counts, chunks in order, leaders only
  int* my = cnt + w * E;
#pragma unroll
  for (int j = 0; j < kWaveChunks; ++j) {
    m[j] = 0;
    if (beg + 64 * j < end) {
      m[j] = align_dev::same_expert_mask(id[j], valid[j], nbits);
      if (valid[j] && align_dev::is_leader(m[j], lane)) my[id[j]] += __popcll(m[j]);
    }
  }
  __syncthreads();
  align_dev::expert_scan<kAlignWaves>(s, E, BS);

  // pass 2: the stable scatter from the kept ids and masks, in the same order
#pragma unroll
  for (int j = 0; j < kWaveChunks; ++j) {
    const int i = beg + 64 * j + lane;
    if (valid[j]) {
      const int pos = s_off[id[j]] + my[id[j]] + __popcll(m[j] & align_dev::lanes_below(lane));
      o.sorted_token_ids[pos] = i;
      o.token_to_perm[i] = pos;
    } else if (i < end) {
      o.token_to_perm[i] = -1;
    }
    // every lane has read its base above (a wave's LDS operations run in order)
    if (valid[j] && align_dev::is_leader(m[j], lane)) my[id[j]] += __popcll(m[j]);
  }
  align_dev::write_rest<kAlignWaves>(s, n, E, BS, max_total, cap, o);
}

// ---- large slot counts: three launches over blocks of kChunk slots ----------
//
// No atomics and no workspace: each block's per-expert counts, and later its
// per-expert bases, live in the first E entries of its own token_to_perm range
// (kChunk >= MOE_MAX_EXPERTS), which only that block's scatter overwrites, after
// it has read them.  Order is the stable host order: blocks ascending, waves
// ascending within a block, lanes ascending within a wave.
constexpr int kChunk = 1024;      // slots per block (the last block also takes the remainder)
constexpr int kBlockWaves = 8;
constexpr int kBlockThreads = kBlockWaves * 64;
static_assert(kChunk >= kMaxExperts, "a block's token_to_perm range must hold E counts");

__device__ __forceinline__ void block_range(int n, int G, int& lo, int& hi) {
  lo = blockIdx.x * kChunk;
  hi = (int)blockIdx.x == G - 1 ? n : lo + kChunk;
}

// per-wave per-expert counts of the block's slots into cnt[wave][expert]
template <typename IdT>
__device__ void block_counts(const IdT* __restrict__ ids, int lo, int hi, int E, int nbits, int* cnt) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kBlockWaves * E; i += kBlockThreads) cnt[i] = 0;
  __syncthreads();
  const int per = (((hi - lo + kBlockWaves - 1) / kBlockWaves) + 63) & ~63;
  const int beg = min(hi, lo + w * per), end = min(hi, beg + per);
  int* my = cnt + w * E;
  for (int c = beg; c < end; c += 64) {
    bool valid;
    const int id = align_dev::load_id(ids, c + lane, end, E, valid);
    const uint64_t m = align_dev::same_expert_mask(id, valid, nbits);
    if (valid && align_dev::is_leader(m, lane)) my[id] += __popcll(m);
  }
  __syncthreads();
}

// launch 1: the block's count of every expert -> dst[blockIdx.x * stride + e]
// (token_to_perm[lo + e] with stride kChunk; a caller's workspace [G][E] with
// stride E)
template <typename IdT>
__global__ __launch_bounds__(kBlockThreads) void align_count_blocks(const IdT* __restrict__ ids, int n, int G, int E,
                                                                   int nbits, int32_t* dst, int stride) {
  __shared__ int cnt[kBlockWaves * kMaxExperts];
  int lo, hi;
  block_range(n, G, lo, hi);
  block_counts(ids, lo, hi, E, nbits, cnt);
  for (int e = threadIdx.x; e < E; e += kBlockThreads) {
    int s = 0;
    for (int w = 0; w < kBlockWaves; ++w) s += cnt[w * E + e];
    dst[(size_t)blockIdx.x * stride + e] = s;
  }
}

// launch 2 (one workgroup): per-expert totals, padded offsets, the active list,
// every table that is not a slot, and each block's base per expert (the
// expert's offset plus the counts of the blocks before it) in place of its count
__global__ __launch_bounds__(kAlignThreads) void align_scan_blocks(int n, int G, int E, int BS, int max_total, int cap,
                                                                  AlignOut o) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_active[kMaxExperts];
  __shared__ int s_wa[kAlignWaves], s_wb[kAlignWaves];
  // J threads per expert, each over a contiguous run of `per` blocks; counts of
  // up to kBatch blocks are loaded together and kept for the bases
  constexpr int kBatch = 16;
  __shared__ int s_part[kAlignThreads];
  const int tid = threadIdx.x;
  const int J = max(1, kAlignThreads / E);
  const int per = (G + J - 1) / J;
  const int ex = tid % E, jx = tid / E;  // a wave reads consecutive experts of one block row
  const bool owner = jx < J;
  const int b_lo = min(G, jx * per), b_hi = min(G, b_lo + per);
  int32_t* col = o.token_to_perm + (owner ? ex : 0);
  int c[kBatch];
  int part = 0;
  if (owner) {
    for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) c[j] = b0 + j < b_hi ? col[(size_t)(b0 + j) * kChunk] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) part += c[j];
    }
    s_part[tid] = part;
  }
  __syncthreads();
  const int e = tid;  // E <= threads
  int count = 0;
  if (e < E) {
    for (int j = 0; j < J; ++j) count += s_part[j * E + e];
  }
  const int pad = (count + BS - 1) / BS * BS;
  int ex_pad, ex_act, total, nact;
  align_dev::block_scan2<kAlignWaves>(pad, count > 0 ? 1 : 0, s_wa, s_wb, ex_pad, ex_act, total, nact);
  if (e < E) {
    s_off[e] = ex_pad;
    if (count > 0) s_active[ex_act] = e;
  }
  __syncthreads();
  if (owner) {
    // block b's base: the expert's offset plus the counts of blocks 0..b-1
    int run = s_off[ex];
    for (int j = 0; j < jx; ++j) run += s_part[j * E + ex];
    for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
      if (b0 > b_lo || b_hi - b_lo > kBatch) {  // reload unless this run fit one batch
#pragma unroll
        for (int j = 0; j < kBatch; ++j) c[j] = b0 + j < b_hi ? col[(size_t)(b0 + j) * kChunk] : 0;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (b0 + j < b_hi) col[(size_t)(b0 + j) * kChunk] = run;
        run += c[j];
      }
    }
  }
  // every table that is not a slot and not an expert's padding or block map
  // (those the scatter blocks write, one wave per expert)
  if (e < E) {
    o.expert_counts[e] = count;
    o.expert_offsets[e] = ex_pad;
  }
  if (e == 0) {
    o.expert_offsets[E] = total;
    *o.total = total;
    *o.active_count = nact;
  }
  for (int j = tid; j < cap; j += kAlignThreads) o.active_experts[j] = j < nact ? s_active[j] : -1;
  for (int p = total + tid; p < max_total; p += kAlignThreads) o.sorted_token_ids[p] = n;
  for (int b = total / BS + tid; b < max_total / BS; b += kAlignThreads) o.block_expert_ids[b] = -1;
}

// launch 3: the stable scatter of the block's slots from its bases; besides,
// wave w of block b writes the padding sentinels and block owners of experts
// b + G * (w + kBlockWaves * i), lanes over consecutive entries.  Everything
// the block reads (its bases, its ids, the first padded expert's offsets and
// count) is requested before any of it is used, and the ids stay in registers
// from the count to the scatter.
constexpr int kScatterChunks = (2 * kChunk / kBlockWaves + 63) / 64;  // 64-slot chunks of a wave (the last block's too)
template <typename IdT>
__global__ __launch_bounds__(kBlockThreads) void align_scatter_blocks(const IdT* __restrict__ ids, int n, int G, int E,
                                                                     int BS, int nbits, AlignOut o) {
  __shared__ int cnt[kBlockWaves * kMaxExperts];
  __shared__ int base[kMaxExperts];
  constexpr int kBaseLoads = kMaxExperts / kBlockThreads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int lo, hi;
  block_range(n, G, lo, hi);
  const int per = (((hi - lo + kBlockWaves - 1) / kBlockWaves) + 63) & ~63;
  const int beg = min(hi, lo + w * per), end = min(hi, beg + per);

  int bv[kBaseLoads];
#pragma unroll
  for (int u = 0; u < kBaseLoads; ++u) {
    const int e = u * kBlockThreads + tid;
    bv[u] = e < E ? o.token_to_perm[lo + e] : 0;
  }
  IdT iv[kScatterChunks];
#pragma unroll
  for (int c = 0; c < kScatterChunks; ++c) iv[c] = beg + 64 * c < end ? ids[min(beg + 64 * c + lane, end - 1)] : (IdT)-1;
  const int e_first = blockIdx.x + G * w;  // the first expert whose padding this wave writes
  int f_lo = 0, f_hi = 0, f_cnt = 0;
  if (e_first < E) {
    f_lo = o.expert_offsets[e_first];
    f_hi = o.expert_offsets[e_first + 1];
    f_cnt = o.expert_counts[e_first];
  }

#pragma unroll
  for (int u = 0; u < kBaseLoads; ++u) {
    const int e = u * kBlockThreads + tid;
    if (e < E) base[e] = bv[u];
  }
  for (int i = tid; i < kBlockWaves * E; i += kBlockThreads) cnt[i] = 0;
  __syncthreads();  // every base is read (above) before any slot is written
  int* my = cnt + w * E;
  auto id_of = [&](int c, bool& valid) -> int {
    const IdT v = iv[c];
    valid = beg + 64 * c + lane < end && v >= 0 && v < (IdT)E;
    return valid ? (int)v : -1;
  };
#pragma unroll
  for (int c = 0; c < kScatterChunks; ++c) {
    if (beg + 64 * c < end) {  // wave-uniform
      bool valid;
      const int id = id_of(c, valid);
      const uint64_t m = align_dev::same_expert_mask(id, valid, nbits);
      if (valid && align_dev::is_leader(m, lane)) my[id] += __popcll(m);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kBlockThreads) {
    int run = base[e];
    for (int k = 0; k < kBlockWaves; ++k) {
      const int c = cnt[k * E + e];
      cnt[k * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kScatterChunks; ++c) {
    if (beg + 64 * c < end) {  // wave-uniform
      const int i = beg + 64 * c + lane;
      bool valid;
      const int id = id_of(c, valid);
      const uint64_t m = align_dev::same_expert_mask(id, valid, nbits);
      if (valid) {
        const int pos = my[id] + __popcll(m & align_dev::lanes_below(lane));
        o.sorted_token_ids[pos] = i;
        o.token_to_perm[i] = pos;
      } else if (i < end) {
        o.token_to_perm[i] = -1;
      }
      // every lane has read its base above (a wave's LDS operations run in order)
      if (valid && align_dev::is_leader(m, lane)) my[id] += __popcll(m);
    }
  }
  for (int e = e_first; e < E; e += G * kBlockWaves) {
    int e_lo = f_lo, e_hi = f_hi, e_cnt = f_cnt;
    if (e != e_first) {
      e_lo = o.expert_offsets[e];
      e_hi = o.expert_offsets[e + 1];
      e_cnt = o.expert_counts[e];
    }
    for (int p = e_lo + e_cnt + lane; p < e_hi; p += 64) o.sorted_token_ids[p] = n;
    for (int b = e_lo / BS + lane; b < e_hi / BS; b += 64) o.block_expert_ids[b] = e;
  }
}

// ---- with a workspace for the block counts: two launches -----------------
//
// Launch 1 is align_count_blocks writing block b's counts to counts[b][e].
// Launch 2: every block reads all G x E counts and forms the totals, padded
// offsets and active list itself (the same block scan in every block), and its
// own bases (each expert's offset plus the counts of the blocks before it);
// then it counts and scatters its slots exactly as align_scatter_blocks does.
// Besides, wave w of block b writes the padding of experts b + G * (w + 8 i),
// the blocks share the tail past the total, and block 0 writes the counts,
// offsets, active list and scalars.  The workspace only separates the counts
// from the tables the scatter overwrites; nothing is shared in any other way.
constexpr int kScanBatch = 16;                                           // block counts loaded together
constexpr int kExpertsPerThread = (kMaxExperts + kBlockThreads - 1) / kBlockThreads;  // a thread's run of experts
template <typename IdT>
__global__ __launch_bounds__(kBlockThreads) void align_scan_scatter_blocks(const IdT* __restrict__ ids, int n, int G,
                                                                          int E, int BS, int max_total, int cap,
                                                                          int nbits, const int32_t* __restrict__ counts,
                                                                          AlignOut o) {
  __shared__ int cnt[kBlockWaves * kMaxExperts];
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_active[kMaxExperts];
  __shared__ int s_wa[kBlockWaves], s_wb[kBlockWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  int lo, hi;
  block_range(n, G, lo, hi);
  const int per = (((hi - lo + kBlockWaves - 1) / kBlockWaves) + 63) & ~63;
  const int beg = min(hi, lo + w * per), end = min(hi, beg + per);

  // the block's ids first (they do not depend on the counts)
  IdT iv[kScatterChunks];
#pragma unroll
  for (int c = 0; c < kScatterChunks; ++c) iv[c] = beg + 64 * c < end ? ids[min(beg + 64 * c + lane, end - 1)] : (IdT)-1;

  // every block's count of each expert, summed in block order (and up to this
  // block, for the base).  Up to kBlockThreads experts: J = kBlockThreads / E
  // threads per expert each sum a run of blocks (one batch of loads at the
  // sizes measured), then thread t takes expert t's sums; above that, thread t
  // sums experts 2t and 2t + 1 alone.  Either way a thread owns a contiguous
  // run of kExpertsPerThread (or 1) experts for the scan.
  __shared__ int s_pt[kBlockThreads], s_pb[kBlockThreads];
  const int ept = E <= kBlockThreads ? 1 : kExpertsPerThread;  // experts per thread in the scan
  int tot[kExpertsPerThread], bef[kExpertsPerThread];
#pragma unroll
  for (int k = 0; k < kExpertsPerThread; ++k) tot[k] = bef[k] = 0;
  auto sum_blocks = [&](int e, int c_lo, int c_hi, int& t_sum, int& b_sum) {
    for (int c0 = c_lo; c0 < c_hi; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = c0 + j < c_hi ? counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (c0 + j < b) b_sum += v[j];
        t_sum += v[j];
      }
    }
  };
  // ept == 1: this thread's first batch of block counts is requested now and
  // stays in flight while the block counts its own slots (the ids are already
  // in registers); the sums then take it first, in block order as always
  const int J = ept == 1 ? kBlockThreads / E : 1;
  const int ex = tid % E, jx = tid / E;
  const int bper = (G + J - 1) / J;  // blocks per thread
  const int c_lo = ept == 1 && jx < J ? min(G, jx * bper) : 0;
  const int c_hi = ept == 1 && jx < J ? min(G, c_lo + bper) : 0;
  int pv[kScanBatch];
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j) pv[j] = c_lo + j < c_hi ? counts[(size_t)(c_lo + j) * E + ex] : 0;

  // the block's own slots, per wave
  for (int i = tid; i < kBlockWaves * E; i += kBlockThreads) cnt[i] = 0;
  __syncthreads();
  int* my = cnt + w * E;
  auto id_of = [&](int c, bool& valid) -> int {
    const IdT v = iv[c];
    valid = beg + 64 * c + lane < end && v >= 0 && v < (IdT)E;
    return valid ? (int)v : -1;
  };
#pragma unroll
  for (int c = 0; c < kScatterChunks; ++c) {
    if (beg + 64 * c < end) {  // wave-uniform
      bool valid;
      const int id = id_of(c, valid);
      const uint64_t m = align_dev::same_expert_mask(id, valid, nbits);
      if (valid && align_dev::is_leader(m, lane)) my[id] += __popcll(m);
    }
  }

  if (ept == 1) {
    int pt = 0, pb = 0;
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      if (c_lo + j < b) pb += pv[j];
      pt += pv[j];
    }
    if (c_lo + kScanBatch < c_hi) sum_blocks(ex, c_lo + kScanBatch, c_hi, pt, pb);
    s_pt[tid] = pt;
    s_pb[tid] = pb;
    __syncthreads();
    if (tid < E) {
      for (int j = 0; j < J; ++j) {  // the runs in block order
        tot[0] += s_pt[j * E + tid];
        bef[0] += s_pb[j * E + tid];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kExpertsPerThread; ++k) {
      const int e = tid * kExpertsPerThread + k;
      if (e < E) sum_blocks(e, 0, G, tot[k], bef[k]);
    }
  }
  int sum_pad = 0, sum_act = 0;
#pragma unroll
  for (int k = 0; k < kExpertsPerThread; ++k) {
    sum_pad += (tot[k] + BS - 1) / BS * BS;
    sum_act += tot[k] > 0 ? 1 : 0;
  }
  int ex_pad, ex_act, total, nact;
  align_dev::block_scan2<kBlockWaves>(sum_pad, sum_act, s_wa, s_wb, ex_pad, ex_act, total, nact);
#pragma unroll
  for (int k = 0; k < kExpertsPerThread; ++k) {
    const int e = tid * ept + k;
    if (k < ept && e < E) {
      s_off[e] = ex_pad;
      s_tot[e] = tot[k];
      s_base[e] = ex_pad + bef[k];
      if (tot[k] > 0) s_active[ex_act++] = e;
      ex_pad += (tot[k] + BS - 1) / BS * BS;
    }
  }
  if (tid == 0) s_off[E] = total;
  __syncthreads();  // the bases (and the block's own counts, counted above) are in LDS
  for (int e = tid; e < E; e += kBlockThreads) {
    int run = s_base[e];
    for (int k = 0; k < kBlockWaves; ++k) {
      const int c = cnt[k * E + e];
      cnt[k * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kScatterChunks; ++c) {
    if (beg + 64 * c < end) {  // wave-uniform
      const int i = beg + 64 * c + lane;
      bool valid;
      const int id = id_of(c, valid);
      const uint64_t m = align_dev::same_expert_mask(id, valid, nbits);
      if (valid) {
        const int pos = my[id] + __popcll(m & align_dev::lanes_below(lane));
        o.sorted_token_ids[pos] = i;
        o.token_to_perm[i] = pos;
      } else if (i < end) {
        o.token_to_perm[i] = -1;
      }
      // every lane has read its base above (a wave's LDS operations run in order)
      if (valid && align_dev::is_leader(m, lane)) my[id] += __popcll(m);
    }
  }
  for (int e = b + G * w; e < E; e += G * kBlockWaves) {
    const int e_lo = s_off[e], e_hi = s_off[e + 1];
    for (int p = e_lo + s_tot[e] + lane; p < e_hi; p += 64) o.sorted_token_ids[p] = n;
    for (int q = e_lo / BS + lane; q < e_hi / BS; q += 64) o.block_expert_ids[q] = e;
  }
  for (int p = total + b * kBlockThreads + tid; p < max_total; p += G * kBlockThreads) o.sorted_token_ids[p] = n;
  for (int q = total / BS + b * kBlockThreads + tid; q < max_total / BS; q += G * kBlockThreads)
    o.block_expert_ids[q] = -1;
  if (b == 0) {
    for (int e = tid; e < E; e += kBlockThreads) {
      o.expert_counts[e] = s_tot[e];
      o.expert_offsets[e] = s_off[e];
    }
    for (int j = tid; j < cap; j += kBlockThreads) o.active_experts[j] = j < nact ? s_active[j] : -1;
    if (tid == 0) {
      o.expert_offsets[E] = total;
      *o.total = total;
      *o.active_count = nact;
    }
  }
}

}  // namespace

int align_blocks(int n) { return n >= kAlignBlocksMinSlots ? n / kChunk : 0; }

hipError_t launch_align(const void* ids, bool ids64, int n, int E, int BS, int max_total, int cap,
                        const AlignOut& o, hipStream_t s) {
  const int nbits = align_dev::id_bits(E);
  const int G = align_blocks(n);
  if (G > 0) {  // many slots: count, scan, scatter over G blocks
    if (ids64)
      hipLaunchKernelGGL(align_count_blocks<int64_t>, dim3(G), dim3(kBlockThreads), 0, s,
                         static_cast<const int64_t*>(ids), n, G, E, nbits, o.token_to_perm, kChunk);
    else
      hipLaunchKernelGGL(align_count_blocks<int32_t>, dim3(G), dim3(kBlockThreads), 0, s,
                         static_cast<const int32_t*>(ids), n, G, E, nbits, o.token_to_perm, kChunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(align_scan_blocks, dim3(1), dim3(kAlignThreads), 0, s, n, G, E, BS, max_total, cap, o);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ids64)
      hipLaunchKernelGGL(align_scatter_blocks<int64_t>, dim3(G), dim3(kBlockThreads), 0, s,
                         static_cast<const int64_t*>(ids), n, G, E, BS, nbits, o);
    else
      hipLaunchKernelGGL(align_scatter_blocks<int32_t>, dim3(G), dim3(kBlockThreads), 0, s,
                         static_cast<const int32_t*>(ids), n, G, E, BS, nbits, o);
    return hipGetLastError();
  }
  if (ids64)
    hipLaunchKernelGGL(align_kernel<int64_t>, dim3(1), dim3(kAlignThreads), 0, s,
                       static_cast<const int64_t*>(ids), n, E, BS, max_total, cap, nbits, o);
  else
    hipLaunchKernelGGL(align_kernel<int32_t>, dim3(1), dim3(kAlignThreads), 0, s,
                       static_cast<const int32_t*>(ids), n, E, BS, max_total, cap, nbits, o);
  return hipGetLastError();
}

size_t align_workspace_bytes(int n, int E) { return (size_t)align_blocks(n) * E * sizeof(int32_t); }

// The workspace form's scan+scatter blocks each read every block's counts
// (E * G^2 loads in all), which outgrows the three launches' one scan: on
// MI355X at E = 256 the workspace form is faster up to 512 blocks (31.9 against
// 35.8 us) and slower from 576 (43.0 against 39.8 us).  Past that much work the
// three launches run instead (the same tables).
constexpr int64_t kAlignWsMaxWork = (int64_t)256 * 512 * 512;

hipError_t launch_align_ws(const void* ids, bool ids64, int n, int E, int BS, int max_total, int cap, int32_t* ws,
                           const AlignOut& o, hipStream_t s) {
  const int G = align_blocks(n);
  if (G == 0 || (int64_t)E * G * G > kAlignWsMaxWork) return launch_align(ids, ids64, n, E, BS, max_total, cap, o, s);
  const int nbits = align_dev::id_bits(E);
  if (ids64)
    hipLaunchKernelGGL(align_count_blocks<int64_t>, dim3(G), dim3(kBlockThreads), 0, s,
                       static_cast<const int64_t*>(ids), n, G, E, nbits, ws, E);
  else
    hipLaunchKernelGGL(align_count_blocks<int32_t>, dim3(G), dim3(kBlockThreads), 0, s,
                       static_cast<const int32_t*>(ids), n, G, E, nbits, ws, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ids64)
    hipLaunchKernelGGL(align_scan_scatter_blocks<int64_t>, dim3(G), dim3(kBlockThreads), 0, s,
                       static_cast<const int64_t*>(ids), n, G, E, BS, max_total, cap, nbits, ws, o);
  else
    hipLaunchKernelGGL(align_scan_scatter_blocks<int32_t>, dim3(G), dim3(kBlockThreads), 0, s,
                       static_cast<const int32_t*>(ids), n, G, E, BS, max_total, cap, nbits, ws, o);
  return hipGetLastError();
}

}  // namespace moe
