// Internal interface between the C ABI layer (api.cpp) and the gfx950 kernels.
// Launchers validate nothing: api.cpp has checked every argument before calling.
#pragma once

#include <stdint.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime_api.h>

#include "moe_mi355x.h"

namespace moe {

// ---- host-side launch helpers (caches kept per device, safe across threads)
constexpr int kMaxCachedDevices = 64;

// The current device, or -1 when it cannot be cached (the helpers then ask HIP every time).
inline int cached_device() {
  int d = 0;
  return hipGetDevice(&d) == hipSuccess && d >= 0 && d < kMaxCachedDevices ? d : -1;
}

// Dynamic LDS above 64 KB per workgroup must be allowed per kernel and device.
// `allowed` (one array per kernel) holds the largest size allowed so far on each
// device; the attribute only ever grows, so concurrent launchers never shrink
// it under one another.
inline hipError_t allow_dynamic_lds(const void* kern, size_t lds, std::atomic<size_t> (&allowed)[kMaxCachedDevices]) {
  if (lds <= 64 * 1024) return hipSuccess;
  const int dev = cached_device();
  if (dev < 0) return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (lds <= allowed[dev].load(std::memory_order_acquire)) return hipSuccess;
  static std::mutex m;
  std::lock_guard<std::mutex> g(m);
  if (lds <= allowed[dev].load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) allowed[dev].store(lds, std::memory_order_release);
  return e;
}

// Workgroups of `kern` one compute unit holds at `lds` bytes of dynamic LDS on
// the current device; `cache` (one array per kernel) keeps the last size asked
// and its answer per device, packed in one word.
inline hipError_t occupancy_per_cu(const void* kern, int threads, size_t lds,
                                   std::atomic<uint64_t> (&cache)[kMaxCachedDevices], int& per_cu) {
  const int dev = cached_device();
  const uint64_t key = ((uint64_t)lds + 1) << 16;
  if (dev >= 0) {
    const uint64_t v = cache[dev].load(std::memory_order_relaxed);
    if ((v & ~(uint64_t)0xffff) == key) {
      per_cu = (int)(v & 0xffff);
      return hipSuccess;
    }
  }
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds);
  if (e != hipSuccess) return e;
  if (dev >= 0) cache[dev].store(key | (uint64_t)(n & 0xffff), std::memory_order_relaxed);
  per_cu = n;
  return hipSuccess;
}

constexpr int kFp8Block = 128;   // FP8 scale block edge (both N and K)

// Expert weight element formats of the kernels' templates.
//  kFmtBF16: bf16; kFmtFP8: OCP e4m3fn codes with float32 block or row scales;
//  kFmtFP4: OCP MXFP4, E2M1 codes two per byte (the lower nibble first) with one
//  E8M0 scale byte per 32 consecutive depth elements of a row.
constexpr int kFmtBF16 = 0, kFmtFP8 = 1, kFmtFP4 = 2;
constexpr int kMxBlock = 32;  // depth elements per E8M0 scale byte

// Record a failure for moe_last_error() and return `code` (api.cpp).
int fail_status(int code, const char* fmt, ...);

struct AlignOut {
  int32_t* sorted_token_ids;
  int32_t* block_expert_ids;
  int32_t* expert_offsets;
  int32_t* expert_counts;
  int32_t* token_to_perm;
  int32_t* active_experts;
  int32_t* active_count;
  int32_t* total;
};

// The whole alignment: one launch and one workgroup, or for n >= 4096 slots
// three launches over align_blocks(n) blocks (count, scan, scatter).
int align_blocks(int n);
hipError_t launch_align(const void* ids, bool ids64, int n, int E, int BS, int max_total, int cap,
                        const AlignOut& o, hipStream_t s);
// The same tables in two launches (count, then scan + scatter in every block)
// when the blocks' counts get a workspace of align_workspace_bytes(n, E)
// bytes (0 below the block threshold, where this is launch_align).
size_t align_workspace_bytes(int n, int E);
hipError_t launch_align_ws(const void* ids, bool ids64, int n, int E, int BS, int max_total, int cap, int32_t* ws,
                           const AlignOut& o, hipStream_t s);

// Operands of one grouped projection launch (routed experts + optional shared expert).
struct GroupedArgs {
  // routed experts
  const void* x;        // gate+up: bf16 [M, K] token rows; down: float32 [max_total, K] by position
  const void* w0;       // gate (gate+up) or down weights [E, N, K]
  const void* s0;       // its FP8 scales (float32 [E, N/128, K/128] or [E, N]) or MXFP4 E8M0 bytes [E, N, K/32]
  const void* w1;       // up weights (gate+up only)
  const void* s1;
  float* out;           // gate+up: act [max_total, N]; down: expert_out [max_total, N]
  int N, K;
  // shared expert (sw0 == nullptr: none)
  const void* sx;       // gate+up: bf16 [M, sK] (the same x); down: float32 sh_act [M, sK]
  const void* sw0;
  const void* ss0;
  const void* sw1;
  const void* ss1;
  float* sout;          // [M, sN]
  int sN, sK;
  // alignment tables
  const int32_t* sorted_token_ids;
  const int32_t* expert_offsets;
  const int32_t* expert_counts;
  const int32_t* active_experts;
  const int32_t* active_count;
  int M, top_k, cap;
  int scale_rows;  // FP8 scales are one per weight row, [E, N] (else per 128x128 block)
  int items;    // routed work items (rowcap-row passes of active experts) the grid covers; set at launch
  int sgroups;  // shared-expert row groups, ahead of the routed items; set at launch
  // fused alignment (gate+up only; ids != nullptr): every routed workgroup
  // aligns topk_ids in LDS itself, and workgroup (0, 0) writes `tables`
  const void* ids;
  int ids64, n, E, BS, max_total;
  AlignOut tables;
};

// Largest slot count the fused align + gate+up kernel takes (its per-workgroup
// alignment cost grows with n; above this the layer runs the align kernel).
constexpr int kFusedAlignMaxSlots = MOE_FUSED_ALIGN_MAX_SLOTS;

// Rows one pass over the weights stages: the most an expert holds when ids are
// distinct within a token (M), as a power of two of at least 4, at most 128.
// Chosen from the shape class, never from the routing.
int grouped_rows_per_pass(int64_t M);

// The separate grouped kernels: rows per pass (at most 16), and the passes an
// expert holding M rows needs (1: every expert fits one pass when ids are
// distinct within a token).
int grouped_step_rows(int64_t M);
int grouped_passes(int64_t M);

// Wide-pass kernels (wide.hip): every row an expert holds, 32 at a time, per
// (expert pass, column group), so each expert's weights are streamed once per
// column group per 32 rows; the same bits as the 16-row pass kernels.  Taken
// for FP8 and MXFP4 weights with the tables of the align launch when an
// expert can hold more than 16 rows (M > 16) and holds 4 on average.
bool grouped_wide(int fmt, const GroupedArgs& a, bool gate_up);
hipError_t launch_wide_gate_up(int fmt, const GroupedArgs& a, bool tiled, hipStream_t s);
hipError_t launch_wide_down(int fmt, const GroupedArgs& a, bool tiled, hipStream_t s);

// fmt: the weight element format, kFmtBF16 / kFmtFP8 / kFmtFP4
hipError_t launch_grouped_gate_up(const GroupedArgs& a, int fmt, bool tiled, hipStream_t s);
hipError_t launch_grouped_down(const GroupedArgs& a, int fmt, bool tiled, hipStream_t s);

// The tiled (MFMA-fragment-ordered) copy of row-major [E, N, K] weights.
size_t tiled_weight_bytes(int fmt, int64_t E, int N, int K);
hipError_t launch_tile_weights(const void* src, void* dst, int fmt, int64_t E, int N, int K, hipStream_t s);

// Single-pass decode layer: one launch aligns (in LDS), runs gate+up+SiLU for a
// 128-wide slice of the intermediate and the matching 128-deep slice of down
// per workgroup, and writes float32 partial outputs per slice; a second launch
// sums the slices and blends.  Tiled weights only.
struct FusedLayerArgs {
  const void* ids;
  int ids64;
  const void* x;          // bf16 [M, H]
  const void* w[3];       // routed gate, up [E, I, H] and down [E, H, I], tiled
  const void* s[3];       // their FP8 scales, or MXFP4 E8M0 bytes (unused for bf16)
  const void* sw[3];      // shared expert (sw[0] == nullptr: none), tiled
  const void* ss[3];
  const void* sh_gate;    // bf16 [H] gate vector of the shared expert, or nullptr (ungated)
  int scale_rows;         // FP8 scales are one per weight row, [E, N] (else per 128x128 block)
  const float* topk_weights;
  uint16_t* out;          // bf16 [M, H]
  float* part;            // [ceil(I/64)][n][H] routed partials by slot
  float* sh_part;         // [ceil(S/64)][M][H] shared partials by token
  float* act;             // narrow path: float32 [n][I] act by slot
  float* sh_act;          // narrow path: float32 [M][S] shared act by token
  int M, H, I, S, E, top_k, BS, n, cap, max_total;
  AlignOut tables;
};

// Most slots the single-pass layer takes (its partial outputs grow with n).
constexpr int kFusedLayerMaxSlots = 256;

// Whether the single-pass layer runs this shape (tiled weights assumed): slot
// count, depth limits and the LDS it needs.
bool fused_layer_fits(int fmt, bool scale_rows, int64_t M, int H, int I, int S, int E, int top_k);
// the first launch (align, gate+up+SiLU, down partials) and the second (sum + blend)
hipError_t launch_layer_partials(const FusedLayerArgs& a, int fmt, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_router(const void* x, const void* w, int M, int H, int E, int top_k, float* logits, void* ids,
                         bool ids64, float* wts, hipStream_t s);
hipError_t launch_blend_partials(const FusedLayerArgs& a, hipStream_t s);

// Narrow-width layer (narrow.hip): gate+up with the depth split over 8 waves
// per (expert, 16-column tile), then down + blend per 16 rows of H.  FP8 tiled
// weights, at most kNarrowLayerMaxSlots slots; the same bits as the other paths.
constexpr int kNarrowLayerMaxSlots = 32;
bool narrow_layer_fits(int fmt, int64_t M, int H, int I, int S, int E, int top_k);
hipError_t launch_narrow_layer(const FusedLayerArgs& a, hipStream_t s);

hipError_t launch_blend(uint16_t* out, const float* expert_out, const float* w, const int32_t* perm,
                        const float* sh_out, const void* x, const void* sh_gate, int M, int H, int top_k,
                        hipStream_t s);

}  // namespace moe
