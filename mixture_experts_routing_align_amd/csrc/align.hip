// Deterministic MoE token alignment for gfx950: one workgroup of 16 wave64s.
//
// What it computes (nbxtensor 0.0.1 wheel page, moe_align.py: module docstring
// and the stage-1/2/3 kernel docstrings; metrale fp8_moe_grouped.rs:
// moe_fp8_grouped_sort): see align_device.h.  One launch, no atomics:
//   pass 1   per-wave per-expert counts from wave ballots (leaders only write);
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

template <typename IdT>
__global__ __launch_bounds__(kAlignThreads) void align_kernel(const IdT* __restrict__ ids, int n, int E, int BS,
                                                              int max_total, int cap, int nbits, AlignOut o) {
  __shared__ int cnt[kAlignWaves * kMaxExperts];  // [wave][expert]: counts, then bases
  __shared__ int s_count[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_active[kMaxExperts];
  __shared__ int s_wa[kAlignWaves], s_wb[kAlignWaves], s_scal[2];
  const align_dev::ExpertLds s{cnt, s_count, s_off, s_active, s_wa, s_wb, s_scal};

  align_dev::count_pass<kAlignWaves>(ids, n, E, nbits, cnt);
  align_dev::expert_scan<kAlignWaves>(s, E, BS);
  align_dev::scatter_pass<kAlignWaves>(ids, n, E, nbits, cnt, s_off, o.sorted_token_ids, o.token_to_perm);
  align_dev::write_rest<kAlignWaves>(s, n, E, BS, max_total, cap, o);
}

}  // namespace

hipError_t launch_align(const void* ids, bool ids64, int n, int E, int BS, int max_total, int cap,
                        const AlignOut& o, hipStream_t s) {
  const int nbits = align_dev::id_bits(E);
  if (ids64)
    hipLaunchKernelGGL(align_kernel<int64_t>, dim3(1), dim3(kAlignThreads), 0, s,
                       static_cast<const int64_t*>(ids), n, E, BS, max_total, cap, nbits, o);
  else
    hipLaunchKernelGGL(align_kernel<int32_t>, dim3(1), dim3(kAlignThreads), 0, s,
                       static_cast<const int32_t*>(ids), n, E, BS, max_total, cap, nbits, o);
  return hipGetLastError();
}

}  // namespace moe
