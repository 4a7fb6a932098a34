// Block-level pieces of the deterministic MoE alignment, shared by the
// standalone align kernel (16 waves) and the fused align + gate/up kernel
// (4 waves).  What they compute is restated from nbxtensor 0.0.1 wheel page,
// moe_align.py (module docstring; stage-1/2/3 kernel docstrings) and metrale
// fp8_moe_grouped.rs (moe_fp8_grouped_sort): per-expert counts of in-range
// slots, counts padded up to BS, their exclusive prefix and total, the
// sentinel n at every position holding no slot, the owner of every BS block
// (-1 past the total), a stable within-expert rank (the number of earlier slots
// with the same expert), token_to_perm, and the ascending active experts.
//
// No atomics.  Each wave owns a contiguous range of slots and walks it 64 at a
// time; a lane's "same expert" mask comes from wave ballots over the id's bits;
// the lowest lane of each group is its leader and alone updates the wave's
// private per-expert count row in LDS.  Order is lane order within a chunk,
// chunk order within a wave and wave order across waves: ascending flat slot
// index, the stable host sort.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace align_dev {

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

__device__ __forceinline__ bool is_leader(uint64_t m, int lane) { return (__ffsll((unsigned long long)m) - 1) == lane; }

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

// slots [beg, end) of wave w: whole 64-slot chunks, ascending by wave
template <int NW>
__device__ __forceinline__ void wave_range(int n, int w, int& beg, int& end) {
  const int per = (((n + NW - 1) / NW) + 63) & ~63;
  beg = min(n, w * per);
  end = min(n, beg + per);
}

// Pass 1: cnt[w*E + e] = slots of expert e in wave w's range.  Ends with a barrier.
template <int NW, typename IdT>
__device__ void count_pass(const IdT* __restrict__ ids, int n, int E, int nbits, int* cnt) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < NW * E; i += NW * 64) cnt[i] = 0;
  __syncthreads();
  int beg, end;
  wave_range<NW>(n, w, beg, end);
  int* my = cnt + w * E;
  for (int c = beg; c < end; c += 64) {
    bool valid;
    const int id = load_id(ids, c + lane, end, E, valid);
    const uint64_t m = same_expert_mask(id, valid, nbits);
    if (valid && is_leader(m, lane)) my[id] += __popcll(m);
  }
  __syncthreads();
}

// Inclusive scan over the wave's lanes on the DPP lane crossbar (no LDS round
// trip): shifts by 1, 2, 4 and 8 within each row of 16 lanes (a lane with no
// source adds 0), then the broadcasts of lane 15 into rows 1 and 3 and of lane
// 31 into rows 2 and 3 carry the row totals across.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Exclusive scan of (a, b) over the block's threads in thread order; also
// returns the totals.  Uses wa/wb [NW] of LDS; contains barriers.
template <int NW>
__device__ void block_scan2(int a, int b, int* wa, int* wb, int& ex_a, int& ex_b, int& tot_a, int& tot_b) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  __syncthreads();  // wa/wb free
  if (lane == 63) {
    wa[w] = ia;
    wb[w] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0;
  tot_a = 0;
  tot_b = 0;
  for (int k = 0; k < NW; ++k) {
    if (k < w) {
      pa += wa[k];
      pb += wb[k];
    }
    tot_a += wa[k];
    tot_b += wb[k];
  }
  ex_a = pa + ia - a;
  ex_b = pb + ib - b;
}

// LDS scratch of the expert scan.
struct ExpertLds {
  int* cnt;     // [NW*E] per-wave counts on entry; per-wave bases on exit
  int* count;   // [E]    slots per expert
  int* off;     // [E+1]  padded exclusive prefix, off[E] = total
  int* active;  // [min(n,E)] ascending active experts (the first nact entries)
  int* wa;      // [NW]
  int* wb;      // [NW]
  int* scal;    // [2]    nact, total
};

// From per-wave counts: per-wave bases, counts, padded offsets, the active list.
// Each thread owns a contiguous run of ceil(E / threads) experts.  Contains barriers.
template <int NW>
__device__ void expert_scan(const ExpertLds& s, int E, int BS) {
  constexpr int T = NW * 64;
  const int tid = threadIdx.x;
  const int per = (E + T - 1) / T;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int sum_pad = 0, sum_act = 0;
  for (int e = e0; e < e1; ++e) {
    // every wave's count requested before any base is stored
    int c[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) c[k] = s.cnt[k * E + e];
    int run = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      s.cnt[k * E + e] = run;
      run += c[k];
    }
    s.count[e] = run;
    sum_pad += (run + BS - 1) / BS * BS;
    sum_act += run > 0 ? 1 : 0;
  }
  int ex_pad, ex_act, total, nact;
  block_scan2<NW>(sum_pad, sum_act, s.wa, s.wb, ex_pad, ex_act, total, nact);
  for (int e = e0; e < e1; ++e) {
    const int c = s.count[e];
    s.off[e] = ex_pad;
    ex_pad += (c + BS - 1) / BS * BS;
    if (c > 0) s.active[ex_act++] = e;
  }
  if (tid == 0) {
    s.off[E] = total;
    s.scal[0] = nact;
    s.scal[1] = total;
  }
  __syncthreads();
}

// Pass 2: every in-range slot i goes to off[id] + (wave base) + (rank within
// the wave); writes sorted_token_ids[pos] = i and token_to_perm[i] (-1 for a
// dropped slot).  Advances the per-wave bases in cnt.  No barrier.
template <int NW, typename IdT>
__device__ void scatter_pass(const IdT* __restrict__ ids, int n, int E, int nbits, int* cnt, const int* off,
                             int32_t* sorted_token_ids, int32_t* token_to_perm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int beg, end;
  wave_range<NW>(n, w, beg, end);
  int* my = cnt + w * E;
  for (int c = beg; c < end; c += 64) {
    const int i = c + lane;
    bool valid;
    const int id = load_id(ids, i, end, E, valid);
    const uint64_t m = same_expert_mask(id, valid, nbits);
    if (valid) {
      const int pos = off[id] + my[id] + __popcll(m & lanes_below(lane));
      sorted_token_ids[pos] = i;
      token_to_perm[i] = pos;
    } else if (i < end) {
      token_to_perm[i] = -1;
    }
    // every lane has read its base above (a wave's LDS operations run in order)
    if (valid && is_leader(m, lane)) my[id] += __popcll(m);
  }
}

// The sources of expert e's rows, in sorted order: src[r] = slot / div of its
// r-th slot (div = top_k gives the token, div = 1 the slot itself).  Reads
// (does not advance) the per-wave bases.  No barrier.
template <int NW, typename IdT>
__device__ void expert_rows(const IdT* __restrict__ ids, int n, int E, int nbits, const int* cnt, int e, int div,
                            int* src) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int beg, end;
  wave_range<NW>(n, w, beg, end);
  int base = cnt[w * E + e];
  for (int c = beg; c < end; c += 64) {
    const int i = c + lane;
    bool valid;
    const int id = load_id(ids, i, end, E, valid);
    const bool mine = valid && id == e;
    const uint64_t m = __ballot(mine);
    if (mine) src[base + __popcll(m & lanes_below(lane))] = i / div;
    base += __popcll(m);
  }
}

// Everything of the tables that is not a slot: counts, offsets, the active
// list and its count, the total, padding sentinels and block owners.  No barrier.
template <int NW>
__device__ void write_rest(const ExpertLds& s, int n, int E, int BS, int max_total, int cap, const AlignOut& o) {
  constexpr int T = NW * 64;
  const int tid = threadIdx.x;
  const int nact = s.scal[0], total = s.scal[1];
  for (int e = tid; e < E; e += T) {
    o.expert_counts[e] = s.count[e];
    o.expert_offsets[e] = s.off[e];
    const int lo = s.off[e], hi = s.off[e + 1];
    for (int p = lo + s.count[e]; p < hi; ++p) o.sorted_token_ids[p] = n;
    for (int b = lo / BS; b < hi / BS; ++b) o.block_expert_ids[b] = e;
  }
  for (int j = tid; j < cap; j += T) o.active_experts[j] = j < nact ? s.active[j] : -1;
  if (tid == 0) {
    o.expert_offsets[E] = total;
    *o.total = total;
    *o.active_count = nact;
  }
  for (int p = total + tid; p < max_total; p += T) o.sorted_token_ids[p] = n;
  for (int b = total / BS + tid; b < max_total / BS; b += T) o.block_expert_ids[b] = -1;
}

__host__ __device__ inline int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

}  // namespace align_dev
}  // namespace moe
