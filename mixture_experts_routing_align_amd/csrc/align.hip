// Deterministic MoE token alignment for gfx950: one workgroup of 16 wave64s.
//
// What it computes (nbxtensor 0.0.1 wheel page, moe_align.py: module docstring
// and the stage-1/2/3 kernel docstrings; metrale fp8_moe_grouped.rs:
// moe_fp8_grouped_sort): per-expert counts of the in-range slots, counts padded
// up to BS, the exclusive prefix of the padded counts and its total, the
// sentinel n at every position that holds no slot, the expert owning each BS
// block (-1 past the total), a stable within-expert rank (the number of earlier
// slots with the same expert) that places slot i at offset[id] + rank, its
// inverse token_to_perm, and the ascending list of active experts.
//
// How (gfx950 design, not the pages'): no atomics and no O(n^2) pairwise rank.
//  * Each wave owns a contiguous range of slots and walks it 64 slots at a time.
//    For a 64-slot chunk, a lane's "same expert" mask is built from wave ballots
//    over the id's bits (mask &= bit ? ballot(bit) : ~ballot(bit)); the lowest
//    lane of each group is its leader.
//  * Pass 1: the leader adds the group's popcount to the wave's private count
//    row in LDS (cnt[wave][expert]); no two lanes ever write one address.
//  * Scan: each expert's per-wave counts become per-wave bases, then a block
//    scan over experts gives the padded offsets and the active-list indices.
//  * Pass 2: the same masks give rank-in-chunk = popcount(mask & lanes below);
//    position = offset[id] + wave base + rank; the leader advances the base.
//  Order is lane order inside a chunk, chunk order inside a wave and wave
//  order across waves: exactly ascending flat slot index, i.e. the stable sort.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Lanes of this wave whose (valid) id equals this lane's id.
__device__ __forceinline__ uint64_t same_expert_mask(int id, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (id >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

template <typename IdT>
__device__ __forceinline__ int load_id(const IdT* ids, int i, int end, int E, bool& valid) {
  if (i >= end) {
    valid = false;
    return -1;
  }
  const IdT v = ids[i];
  valid = v >= 0 && v < (IdT)E;
  return valid ? (int)v : -1;
}

// Exclusive block-wide scan of two counters at once (1024 threads).
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* wave_a, int* wave_b,
                                                      int& ex_a, int& ex_b, int& tot_a, int& tot_b) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ta = __shfl_up(ia, d, 64);
    const int tb = __shfl_up(ib, d, 64);
    if (lane >= d) {
      ia += ta;
      ib += tb;
    }
  }
  if (lane == 63) {
    wave_a[w] = ia;
    wave_b[w] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0;
  tot_a = 0;
  tot_b = 0;
  for (int k = 0; k < kAlignWaves; ++k) {
    if (k < w) {
      pa += wave_a[k];
      pb += wave_b[k];
    }
    tot_a += wave_a[k];
    tot_b += wave_b[k];
  }
  ex_a = pa + ia - a;
  ex_b = pb + ib - b;
}

template <typename IdT>
__global__ __launch_bounds__(kAlignThreads) void align_kernel(const IdT* __restrict__ ids, int n, int E,
                                                              int BS, int max_total, int cap, int nbits,
                                                              AlignOut o) {
  __shared__ int cnt[kAlignWaves * kMaxExperts];  // [wave][expert]: counts, then bases
  __shared__ int s_off[kMaxExperts + 1];          // padded exclusive prefix
  __shared__ int s_cnt[kMaxExperts];              // per-expert counts
  __shared__ int s_wa[kAlignWaves], s_wb[kAlignWaves];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) cnt[i] = 0;
  __syncthreads();

  // each wave owns slots [beg, end), a whole number of 64-slot chunks
  const int per = (((n + kAlignWaves - 1) / kAlignWaves) + 63) & ~63;
  const int beg = min(n, w * per), end = min(n, beg + per);
  int* my_cnt = cnt + w * E;

  // pass 1: per-wave counts

  for (int c = beg; c < end; c += 64) {
    bool valid;
    const int id = load_id(ids, c + lane, end, E, valid);
    const uint64_t m = same_expert_mask(id, valid, nbits);
    if (valid && (__ffsll((unsigned long long)m) - 1) == lane) my_cnt[id] += __popcll(m);
  }
  __syncthreads();

  // per expert: counts of earlier waves become this wave's base
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = 0;
    for (int k = 0; k < kAlignWaves; ++k) {
      const int c = cnt[k * E + e];
      cnt[k * E + e] = run;
      run += c;
    }
    s_cnt[e] = run;
  }
  __syncthreads();

  // padded offsets and active-list slots (E <= 1024: one expert per thread)
  {
    const int e = tid;
    const int c = e < E ? s_cnt[e] : 0;
    const int padded = (c + BS - 1) / BS * BS;
    const int act = c > 0 ? 1 : 0;
    int ex_pad, ex_act, total, nact;
    block_exclusive_scan2(padded, act, s_wa, s_wb, ex_pad, ex_act, total, nact);
    if (e < E) {
      s_off[e] = ex_pad;
      o.expert_offsets[e] = ex_pad;
      o.expert_counts[e] = c;
      if (act) o.active_experts[ex_act] = e;
    }
    if (tid == 0) {
      s_off[E] = total;
      o.expert_offsets[E] = total;
      *o.total = total;
      *o.active_count = nact;
    }
    for (int j = nact + tid; j < cap; j += kAlignThreads) o.active_experts[j] = -1;
  }
  __syncthreads();

  // pass 2: stable scatter of the slots

  for (int c = beg; c < end; c += 64) {
    const int i = c + lane;
    bool valid;
    const int id = load_id(ids, i, end, E, valid);
    const uint64_t m = same_expert_mask(id, valid, nbits);
    if (valid) {
      const int pos = s_off[id] + my_cnt[id] + __popcll(m & lanes_below(lane));
      o.sorted_token_ids[pos] = i;
      o.token_to_perm[i] = pos;
    } else if (i < end) {
      o.token_to_perm[i] = -1;
    }
    // every lane has read its base above (DS operations of a wave run in order)
    if (valid && (__ffsll((unsigned long long)m) - 1) == lane) my_cnt[id] += __popcll(m);
  }

  // padding sentinels and block owners; disjoint from the slot positions
  for (int e = tid; e < E; e += kAlignThreads) {
    const int lo = s_off[e], hi = s_off[e + 1];
    for (int p = lo + s_cnt[e]; p < hi; ++p) o.sorted_token_ids[p] = n;
    for (int b = lo / BS; b < hi / BS; ++b) o.block_expert_ids[b] = e;
  }
  const int total = s_off[E];
  for (int p = total + tid; p < max_total; p += kAlignThreads) o.sorted_token_ids[p] = n;
  for (int b = total / BS + tid; b < max_total / BS; b += kAlignThreads) o.block_expert_ids[b] = -1;
}

}  // namespace

hipError_t launch_align(const void* ids, bool ids64, int n, int E, int BS, int max_total, int cap,
                        const AlignOut& o, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (ids64)
    hipLaunchKernelGGL(align_kernel<int64_t>, dim3(1), dim3(kAlignThreads), 0, s,
                       static_cast<const int64_t*>(ids), n, E, BS, max_total, cap, nbits, o);
  else
    hipLaunchKernelGGL(align_kernel<int32_t>, dim3(1), dim3(kAlignThreads), 0, s,
                       static_cast<const int32_t*>(ids), n, E, BS, max_total, cap, nbits, o);
  return hipGetLastError();
}

}  // namespace moe
