// C ABI of libmoe_mi355x.so: argument checks, workspace layout, and the launch
// order of the layer.  See include/moe_mi355x.h for the contract of each call.
//
// Every entry point checks all host arguments before touching the HIP runtime,
// so a refused call launches nothing (the layer forward of metrale
// forward_nvfp4_grouped_decode.rs launches nothing when its admission predicate
// fails; the one-launch sort of fp8_moe_grouped.rs refuses more than 1024
// experts).  Nothing here allocates, synchronises or reads device memory.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>

#include "moe_internal.h"
#include "moe_mi355x.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace

int moe::fail_status(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

namespace {

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kInt32Limit = (int64_t)1 << 31;

struct AlignShape {
  int64_t n = 0, max_total = 0;
  int32_t cap = 0;
};

// Shape rules shared by every call that takes (M, top_k, E, BS).
int check_routing_shape(const char* fn, int64_t M, int32_t top_k, int32_t E, int32_t BS, AlignShape* s) {
  if (M < 0) return fail(MOE_ERR_SHAPE, "%s: M=%lld is negative", fn, (long long)M);
  if (top_k < 1) return fail(MOE_ERR_SHAPE, "%s: top_k=%d must be >= 1", fn, top_k);
  if (E < 1) return fail(MOE_ERR_SHAPE, "%s: E=%d must be >= 1", fn, E);
  if (BS < 1) return fail(MOE_ERR_SHAPE, "%s: BS=%d must be >= 1", fn, BS);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_LIMIT, "%s: E=%d exceeds the %d experts one align launch handles", fn, E,
                MOE_MAX_EXPERTS);
  if (M >= kInt32Limit / top_k)
    return fail(MOE_ERR_LIMIT, "%s: M*top_k = %lld*%d slots reach 2^31", fn, (long long)M, top_k);
  s->n = M * top_k;
  s->max_total = moe_align_max_total(s->n, E, BS);
  if (s->max_total >= kInt32Limit)
    return fail(MOE_ERR_LIMIT, "%s: worst-case table length %lld reaches 2^31", fn, (long long)s->max_total);
  s->cap = moe_active_cap(s->n, E);
  return MOE_OK;
}

int check_tables(const char* fn, const moe_align_tables* t, bool all) {
  if (t == nullptr) return fail(MOE_ERR_NULL, "%s: tables pointer is NULL", fn);
  if (!t->sorted_token_ids || !t->expert_offsets || !t->expert_counts || !t->active_experts ||
      !t->active_count)
    return fail(MOE_ERR_NULL, "%s: a required table pointer is NULL", fn);
  if (all && (!t->block_expert_ids || !t->token_to_perm || !t->total))
    return fail(MOE_ERR_NULL, "%s: a table pointer is NULL", fn);
  return MOE_OK;
}

bool is_rows(moe_weight_dtype wdt) { return wdt == MOE_W_FP8_E4M3_ROWS || wdt == MOE_W_FP8_E4M3_ROWS_TILED; }
bool is_fp8(moe_weight_dtype wdt) { return wdt == MOE_W_FP8_E4M3 || wdt == MOE_W_FP8_E4M3_TILED || is_rows(wdt); }
bool is_fp4(moe_weight_dtype wdt) { return wdt == MOE_W_MXFP4 || wdt == MOE_W_MXFP4_TILED; }
bool is_tiled(moe_weight_dtype wdt) {
  return wdt == MOE_W_BF16_TILED || wdt == MOE_W_FP8_E4M3_TILED || wdt == MOE_W_FP8_E4M3_ROWS_TILED ||
         wdt == MOE_W_MXFP4_TILED;
}
// the kernels' element format of a weight dtype
int fmt_of(moe_weight_dtype wdt) { return is_fp4(wdt) ? moe::kFmtFP4 : (is_fp8(wdt) ? moe::kFmtFP8 : moe::kFmtBF16); }

// The kernels move weights, x, act and the float32 intermediates 16 bytes per
// lane and the bf16 output 8 bytes per lane: a pointer off that alignment is
// refused (NULL is checked elsewhere).
int check_aligned(const char* fn, const char* what, const void* p, uintptr_t bytes) {
  if (p != nullptr && reinterpret_cast<uintptr_t>(p) % bytes)
    return fail(MOE_ERR_SHAPE, "%s: %s is not %d-byte aligned", fn, what, (int)bytes);
  return MOE_OK;
}

int check_weight(const char* fn, const char* name, const moe_weight* w, moe_weight_dtype wdt) {
  if (w == nullptr || w->w == nullptr) return fail(MOE_ERR_NULL, "%s: %s weights are NULL", fn, name);
  if (reinterpret_cast<uintptr_t>(w->w) % 16)
    return fail(MOE_ERR_SHAPE, "%s: %s weights are not 16-byte aligned", fn, name);
  if (is_fp8(wdt) && w->scale == nullptr) return fail(MOE_ERR_NULL, "%s: %s FP8 scales are NULL", fn, name);
  // per-row scales are read four rows at a time
  if (is_rows(wdt) && reinterpret_cast<uintptr_t>(w->scale) % 16)
    return fail(MOE_ERR_SHAPE, "%s: %s FP8 row scales are not 16-byte aligned", fn, name);
  if (is_fp4(wdt) && w->scale == nullptr) return fail(MOE_ERR_NULL, "%s: %s MXFP4 scales are NULL", fn, name);
  // a row's four scale bytes of one 128-deep chunk are read as one dword
  if (is_fp4(wdt) && reinterpret_cast<uintptr_t>(w->scale) % 4)
    return fail(MOE_ERR_SHAPE, "%s: %s MXFP4 scales are not 4-byte aligned", fn, name);
  return MOE_OK;
}

int check_wdt(const char* fn, moe_weight_dtype wdt) {
  if (wdt < MOE_W_BF16 || wdt > MOE_W_MXFP4_TILED)
    return fail(MOE_ERR_SHAPE, "%s: unknown weight dtype %d", fn, (int)wdt);
  return MOE_OK;
}

// A projection with N output rows and depth K: FP8 needs whole 128x128 scale
// blocks (with per-row scales too: the kernels walk K in the same 128-deep
// chunks); MXFP4 needs K in whole 128-deep chunks (four scale bytes each) and
// N in whole 16-row tiles; BF16 needs K in whole 32-deep MFMA steps and N in
// whole 16-row tiles.
int check_projection(const char* fn, const char* name, moe_weight_dtype wdt, int32_t N, int32_t K) {
  if (N < 1 || K < 1) return fail(MOE_ERR_SHAPE, "%s: %s is %dx%d", fn, name, N, K);
  if (is_fp4(wdt)) {
    if (N % 16 || K % 128)
      return fail(MOE_ERR_SHAPE, "%s: MXFP4 %s is %dx%d; needs N %% 16 == 0 and K %% 128 == 0", fn, name, N, K);
  } else if (is_fp8(wdt)) {
    if (N % moe::kFp8Block || K % moe::kFp8Block)
      return fail(MOE_ERR_SHAPE, "%s: FP8 %s is %dx%d, not whole 128x128 scale blocks", fn, name, N, K);
  } else if (N % 16 || K % 32) {
    return fail(MOE_ERR_SHAPE, "%s: BF16 %s is %dx%d; needs N %% 16 == 0 and K %% 32 == 0", fn, name, N, K);
  }
  return MOE_OK;
}

moe::AlignOut to_align_out(const moe_align_tables& t) {
  return moe::AlignOut{t.sorted_token_ids, t.block_expert_ids, t.expert_offsets, t.expert_counts,
                       t.token_to_perm,    t.active_experts,   t.active_count,   t.total};
}

void fill_tables(moe::GroupedArgs& a, const moe_align_tables* t) {
  a.sorted_token_ids = t->sorted_token_ids;
  a.expert_offsets = t->expert_offsets;
  a.expert_counts = t->expert_counts;
  a.active_experts = t->active_experts;
  a.active_count = t->active_count;
}

moe::GroupedArgs gate_up_args(const void* x_bf16, const moe_weight* gate, const moe_weight* up,
                              const moe_align_tables* t, float* act, const moe_weight* sh_gate,
                              const moe_weight* sh_up, float* sh_act, int64_t M, int32_t H, int32_t I, int32_t S,
                              int32_t top_k, int32_t cap) {
  moe::GroupedArgs a{};
  a.x = x_bf16;
  a.w0 = gate->w;
  a.s0 = gate->scale;
  a.w1 = up->w;
  a.s1 = up->scale;
  a.out = act;
  a.N = I;
  a.K = H;
  if (S > 0) {
    a.sx = x_bf16;
    a.sw0 = sh_gate->w;
    a.ss0 = sh_gate->scale;
    a.sw1 = sh_up->w;
    a.ss1 = sh_up->scale;
    a.sout = sh_act;
    a.sN = S;
    a.sK = H;
  }
  fill_tables(a, t);
  a.M = (int)M;
  a.top_k = top_k;
  a.cap = cap;
  return a;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// MOE_FORCE_PATH, read once per process: the path that replaces
// MOE_LAYER_PATH_AUTO ("steps", "single_pass" or "narrow"; anything else: none).
int forced_path() {
  static const int forced = [] {
    const char* v = getenv("MOE_FORCE_PATH");
    if (v == nullptr) return (int)MOE_LAYER_PATH_AUTO;
    if (!strcmp(v, "steps")) return (int)MOE_LAYER_PATH_STEPS;
    if (!strcmp(v, "single_pass")) return (int)MOE_LAYER_PATH_SINGLE_PASS;
    if (!strcmp(v, "narrow")) return (int)MOE_LAYER_PATH_NARROW;
    return (int)MOE_LAYER_PATH_AUTO;
  }();
  return forced;
}

// The path moe_layer_forward takes for a checked descriptor (shape only, never
// the routing): the one the descriptor (else MOE_FORCE_PATH) asks for, or by
// default the narrow path for a few tokens, else the single-pass layer where
// it fits (tiled weights at decode width), else the steps.  A forced path that
// does not fit is refused.
// Where the single pass fits, AUTO still takes the steps path where that
// measured faster on the decode layer (2048 x 768, 128 experts, top-8; both
// give the same bits, so only time decides): MXFP4 at every width (the single
// pass at best even, and 1.7-1.9x slower from 9 tokens), per-row FP8 scales
// (faster at 4-5 and 7-12 tokens, 1.2 us slower at 6), and block-scaled FP8
// when the slots exceed 6 times the rows of one pass in the 4- and 8-row pass
// classes (4, 7 and 8 tokens: 1.2, 1.8 and 3.1 us faster; at 5-6 tokens and
// in the 16-row class the single pass is as fast or faster).
bool auto_prefers_steps(moe_weight_dtype wdt, int64_t M, int64_t n) {
  if (is_fp4(wdt) || is_rows(wdt)) return true;
  if (!is_fp8(wdt)) return false;
  const int rowcap = moe::grouped_rows_per_pass(M);
  return rowcap <= 8 && n > 6 * (int64_t)rowcap;
}

int layer_path(const char* fn, const moe_layer_desc* d) {
  static_assert(MOE_NARROW_LAYER_MAX_SLOTS == moe::kNarrowLayerMaxSlots, "narrow slot limit");
  const int64_t n = d->M * d->top_k;
  const bool fits = is_tiled(d->wdt) &&
                    moe::fused_layer_fits(fmt_of(d->wdt), is_rows(d->wdt), d->M, d->H, d->I, d->S, d->E, d->top_k);
  const bool narrow_fits =
      is_tiled(d->wdt) && moe::narrow_layer_fits(fmt_of(d->wdt), d->M, d->H, d->I, d->S, d->E, d->top_k);
  const int want = d->path != MOE_LAYER_PATH_AUTO ? (int)d->path : forced_path();
  if (want == MOE_LAYER_PATH_STEPS) return MOE_LAYER_PATH_STEPS;
  if (want == MOE_LAYER_PATH_SINGLE_PASS && !fits)
    return fail(MOE_ERR_SHAPE,
                "%s: the single-pass path needs tiled weights, at most %d slots (M*top_k = %lld) and its LDS "
                "budget",
                fn, MOE_FUSED_LAYER_MAX_SLOTS, (long long)n);
  if (want == MOE_LAYER_PATH_NARROW && !narrow_fits)
    return fail(MOE_ERR_SHAPE,
                "%s: the narrow path needs tiled FP8 weights, at most %d slots (M*top_k = %lld) and its LDS budget",
                fn, MOE_NARROW_LAYER_MAX_SLOTS, (long long)n);
  if (want != MOE_LAYER_PATH_AUTO) return want;
  if (narrow_fits && n <= MOE_NARROW_AUTO_SLOTS) return MOE_LAYER_PATH_NARROW;
  return fits && !auto_prefers_steps(d->wdt, d->M, n) ? MOE_LAYER_PATH_SINGLE_PASS : MOE_LAYER_PATH_STEPS;
}

// MOE_LOG=1 (read once per process): one line on stderr the first time the
// layer runs each path.
void log_path_once(const moe_layer_desc* d, int path) {
  static const bool on = [] {
    const char* v = getenv("MOE_LOG");
    return v != nullptr && !strcmp(v, "1");
  }();
  if (!on) return;
  static std::atomic<unsigned> logged{0};
  const unsigned bit = 1u << path;
  if (logged.fetch_or(bit) & bit) return;
  static const char* names[] = {"auto", "steps", "single_pass", "narrow"};
  static const char* wnames[] = {"bf16",          "fp8_e4m3",            "bf16_tiled", "fp8_e4m3_tiled",
                                 "fp8_e4m3_rows", "fp8_e4m3_rows_tiled", "mxfp4",      "mxfp4_tiled"};
  fprintf(stderr,
          "moe_mi355x: moe_layer_forward path %s (M=%lld H=%d I=%d S=%d E=%d top_k=%d BS=%d weights %s%s)\n",
          names[path], (long long)d->M, d->H, d->I, d->S, d->E, d->top_k, d->BS, wnames[d->wdt],
          d->path != MOE_LAYER_PATH_AUTO ? ", forced by the descriptor"
                                         : (forced_path() != MOE_LAYER_PATH_AUTO ? ", forced by MOE_FORCE_PATH" : ""));
}

int layout(const moe_layer_desc* d, size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1], int* path = nullptr) {
  const char* fn = "moe_layer_workspace";
  if (d == nullptr) return fail(MOE_ERR_NULL, "%s: descriptor is NULL", fn);
  AlignShape s;
  int rc = check_routing_shape(fn, d->M, d->top_k, d->E, d->BS, &s);
  if (rc) return rc;
  if ((rc = check_wdt(fn, d->wdt))) return rc;
  if (d->idt != MOE_IDX_I32 && d->idt != MOE_IDX_I64)
    return fail(MOE_ERR_SHAPE, "%s: unknown index dtype %d", fn, (int)d->idt);
  if (d->S < 0) return fail(MOE_ERR_SHAPE, "%s: S=%d is negative", fn, d->S);
  if (d->path < MOE_LAYER_PATH_AUTO || d->path > MOE_LAYER_PATH_NARROW)
    return fail(MOE_ERR_SHAPE, "%s: unknown path %d", fn, (int)d->path);
  if ((rc = check_projection(fn, "gate/up", d->wdt, d->I, d->H))) return rc;
  if ((rc = check_projection(fn, "down", d->wdt, d->H, d->I))) return rc;
  if (d->S > 0) {
    if ((rc = check_projection(fn, "shared gate/up", d->wdt, d->S, d->H))) return rc;
    if ((rc = check_projection(fn, "shared down", d->wdt, d->H, d->S))) return rc;
  }
  const int lp = layer_path(fn, d);
  if (lp < 0) return lp;
  if (path) *path = lp;
  const bool single = lp == MOE_LAYER_PATH_SINGLE_PASS, narrow = lp == MOE_LAYER_PATH_NARROW;
  const size_t mt = (size_t)s.max_total, n = (size_t)s.n, M = (size_t)d->M, H = (size_t)d->H;
  const size_t S = (size_t)d->S, I = (size_t)d->I;
  size_t cur = 0;
  auto take = [&](int i, size_t bytes) {
    off[i] = cur;
    cur = align256(cur + bytes);
  };
  take(0, mt * 4);                                        // sorted_token_ids
  take(1, (mt / d->BS) * 4);                              // block_expert_ids
  take(2, ((size_t)d->E + 1) * 4);                        // expert_offsets
  take(3, (size_t)d->E * 4);                              // expert_counts
  take(4, n * 4);                                         // token_to_perm
  take(5, (size_t)s.cap * 4);                             // active_experts
  take(6, 4);                                             // active_count
  take(7, 4);                                             // total
  take(8, single ? 0 : (narrow ? n : mt) * I * 4);        // act (narrow: by slot)
  take(9, single || narrow ? 0 : mt * H * 4);             // expert_out
  take(10, single ? 0 : M * S * 4);                       // sh_act
  take(11, single || narrow ? 0 : M * H * 4);             // sh_out
  take(12, single ? ((I + 63) / 64) * n * H * 4 : 0);     // part: per 64-wide slice of I, per slot
  take(13, single ? ((S + 63) / 64) * M * H * 4 : 0);     // sh_part: per 64-wide slice of S, per token
  off[14] = cur;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 11; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

int64_t moe_align_max_total(int64_t n, int32_t E, int32_t BS) {
  if (n < 0 || E < 1 || BS < 1) return -1;
  const int64_t bound = std::min(n * (int64_t)BS, n + (int64_t)E * (BS - 1));
  return (bound + BS - 1) / BS * BS;
}

int32_t moe_active_cap(int64_t n, int32_t E) {
  if (n < 0 || E < 0) return -1;
  return (int32_t)std::min<int64_t>(n, E);
}

int moe_align(const void* topk_ids, moe_index_dtype idt, int64_t M, int32_t top_k, int32_t E, int32_t BS,
              const moe_align_tables* out, hipStream_t stream) {
  const char* fn = "moe_align";
  AlignShape s;
  int rc = check_routing_shape(fn, M, top_k, E, BS, &s);
  if (rc) return rc;
  if (idt != MOE_IDX_I32 && idt != MOE_IDX_I64)
    return fail(MOE_ERR_SHAPE, "%s: unknown index dtype %d", fn, (int)idt);
  if (M == 0) return MOE_OK;
  if (topk_ids == nullptr) return fail(MOE_ERR_NULL, "%s: topk_ids is NULL", fn);
  if ((rc = check_tables(fn, out, true))) return rc;
  return hip_status(moe::launch_align(topk_ids, idt == MOE_IDX_I64, (int)s.n, E, BS, (int)s.max_total,
                                      s.cap, to_align_out(*out), stream),
                    fn);
}

size_t moe_align_workspace_bytes(int64_t M, int32_t top_k, int32_t E) {
  AlignShape s;
  if (check_routing_shape("moe_align_workspace_bytes", M, top_k, E, 1, &s)) return 0;
  return moe::align_workspace_bytes((int)s.n, E);
}

int moe_align_ws(const void* topk_ids, moe_index_dtype idt, int64_t M, int32_t top_k, int32_t E, int32_t BS,
                 const moe_align_tables* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "moe_align_ws";
  AlignShape s;
  int rc = check_routing_shape(fn, M, top_k, E, BS, &s);
  if (rc) return rc;
  if (idt != MOE_IDX_I32 && idt != MOE_IDX_I64)
    return fail(MOE_ERR_SHAPE, "%s: unknown index dtype %d", fn, (int)idt);
  if (M == 0) return MOE_OK;
  if (topk_ids == nullptr) return fail(MOE_ERR_NULL, "%s: topk_ids is NULL", fn);
  if ((rc = check_tables(fn, out, true))) return rc;
  const size_t need = moe::align_workspace_bytes((int)s.n, E);
  if (need > 0) {
    if (workspace == nullptr) return fail(MOE_ERR_NULL, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if ((rc = check_aligned(fn, "workspace", workspace, 16))) return rc;
  }
  return hip_status(moe::launch_align_ws(topk_ids, idt == MOE_IDX_I64, (int)s.n, E, BS, (int)s.max_total, s.cap,
                                         static_cast<int32_t*>(workspace), to_align_out(*out), stream),
                    fn);
}

int moe_grouped_gate_up_silu(const void* x_bf16, moe_weight_dtype wdt, const moe_weight* gate,
                             const moe_weight* up, const moe_align_tables* t, float* act,
                             const moe_weight* sh_gate, const moe_weight* sh_up, float* sh_act, int64_t M,
                             int32_t H, int32_t I, int32_t S, int32_t E, int32_t top_k, int32_t BS,
                             hipStream_t stream) {
  const char* fn = "moe_grouped_gate_up_silu";
  AlignShape s;
  int rc = check_routing_shape(fn, M, top_k, E, BS, &s);
  if (rc) return rc;
  if ((rc = check_wdt(fn, wdt))) return rc;
  if (S < 0) return fail(MOE_ERR_SHAPE, "%s: S=%d is negative", fn, S);
  if ((rc = check_projection(fn, "gate/up", wdt, I, H))) return rc;
  if (S > 0 && (rc = check_projection(fn, "shared gate/up", wdt, S, H))) return rc;
  if (M == 0) return MOE_OK;
  if (x_bf16 == nullptr || act == nullptr) return fail(MOE_ERR_NULL, "%s: x or act is NULL", fn);
  if ((rc = check_aligned(fn, "x", x_bf16, 16)) || (rc = check_aligned(fn, "act", act, 16)) ||
      (rc = check_aligned(fn, "sh_act", sh_act, 16)))
    return rc;
  if ((rc = check_weight(fn, "gate", gate, wdt)) || (rc = check_weight(fn, "up", up, wdt))) return rc;
  if ((rc = check_tables(fn, t, false))) return rc;
  if (S > 0) {
    if ((rc = check_weight(fn, "shared gate", sh_gate, wdt)) || (rc = check_weight(fn, "shared up", sh_up, wdt)))
      return rc;
    if (sh_act == nullptr) return fail(MOE_ERR_NULL, "%s: sh_act is NULL with S > 0", fn);
  }
  moe::GroupedArgs a = gate_up_args(x_bf16, gate, up, t, act, sh_gate, sh_up, sh_act, M, H, I, S, top_k, s.cap);
  a.scale_rows = is_rows(wdt);
  a.E = E;
  return hip_status(
      moe::launch_grouped_gate_up(a, fmt_of(wdt), is_tiled(wdt), stream), fn);
}

int moe_align_gate_up_silu(const void* topk_ids, moe_index_dtype idt, const void* x_bf16, moe_weight_dtype wdt,
                           const moe_weight* gate, const moe_weight* up, const moe_align_tables* t, float* act,
                           const moe_weight* sh_gate, const moe_weight* sh_up, float* sh_act, int64_t M,
                           int32_t H, int32_t I, int32_t S, int32_t E, int32_t top_k, int32_t BS,
                           hipStream_t stream) {
  const char* fn = "moe_align_gate_up_silu";
  AlignShape s;
  int rc = check_routing_shape(fn, M, top_k, E, BS, &s);
  if (rc) return rc;
  if (idt != MOE_IDX_I32 && idt != MOE_IDX_I64)
    return fail(MOE_ERR_SHAPE, "%s: unknown index dtype %d", fn, (int)idt);
  if (s.n > moe::kFusedAlignMaxSlots)
    return fail(MOE_ERR_LIMIT, "%s: %lld slots exceed the fused limit %d", fn, (long long)s.n,
                moe::kFusedAlignMaxSlots);
  if ((rc = check_wdt(fn, wdt))) return rc;
  if (S < 0) return fail(MOE_ERR_SHAPE, "%s: S=%d is negative", fn, S);
  if ((rc = check_projection(fn, "gate/up", wdt, I, H))) return rc;
  if (S > 0 && (rc = check_projection(fn, "shared gate/up", wdt, S, H))) return rc;
  if (M == 0) return MOE_OK;
  if (topk_ids == nullptr || x_bf16 == nullptr || act == nullptr)
    return fail(MOE_ERR_NULL, "%s: topk_ids, x or act is NULL", fn);
  if ((rc = check_aligned(fn, "x", x_bf16, 16)) || (rc = check_aligned(fn, "act", act, 16)) ||
      (rc = check_aligned(fn, "sh_act", sh_act, 16)))
    return rc;
  if ((rc = check_weight(fn, "gate", gate, wdt)) || (rc = check_weight(fn, "up", up, wdt))) return rc;
  if ((rc = check_tables(fn, t, true))) return rc;
  if (S > 0) {
    if ((rc = check_weight(fn, "shared gate", sh_gate, wdt)) || (rc = check_weight(fn, "shared up", sh_up, wdt)))
      return rc;
    if (sh_act == nullptr) return fail(MOE_ERR_NULL, "%s: sh_act is NULL with S > 0", fn);
  }
  moe::GroupedArgs a = gate_up_args(x_bf16, gate, up, t, act, sh_gate, sh_up, sh_act, M, H, I, S, top_k, s.cap);
  a.ids = topk_ids;
  a.ids64 = idt == MOE_IDX_I64;
  a.n = (int)s.n;
  a.E = E;
  a.BS = BS;
  a.max_total = (int)s.max_total;
  a.tables = to_align_out(*t);
  a.scale_rows = is_rows(wdt);
  return hip_status(
      moe::launch_grouped_gate_up(a, fmt_of(wdt), is_tiled(wdt), stream), fn);
}

int moe_grouped_down(const float* act, moe_weight_dtype wdt, const moe_weight* down, const moe_align_tables* t,
                     float* expert_out, const moe_weight* sh_down, const float* sh_act, float* sh_out, int64_t M,
                     int32_t H, int32_t I, int32_t S, int32_t E, int32_t top_k, int32_t BS, hipStream_t stream) {
  const char* fn = "moe_grouped_down";
  AlignShape s;
  int rc = check_routing_shape(fn, M, top_k, E, BS, &s);
  if (rc) return rc;
  if ((rc = check_wdt(fn, wdt))) return rc;
  if (S < 0) return fail(MOE_ERR_SHAPE, "%s: S=%d is negative", fn, S);
  if ((rc = check_projection(fn, "down", wdt, H, I))) return rc;
  if (S > 0 && (rc = check_projection(fn, "shared down", wdt, H, S))) return rc;
  if (M == 0) return MOE_OK;
  if (act == nullptr || expert_out == nullptr) return fail(MOE_ERR_NULL, "%s: act or expert_out is NULL", fn);
  if ((rc = check_aligned(fn, "act", act, 16)) || (rc = check_aligned(fn, "expert_out", expert_out, 16)) ||
      (rc = check_aligned(fn, "sh_act", sh_act, 16)) || (rc = check_aligned(fn, "sh_out", sh_out, 16)))
    return rc;
  if ((rc = check_weight(fn, "down", down, wdt))) return rc;
  if ((rc = check_tables(fn, t, false))) return rc;
  if (S > 0) {
    if ((rc = check_weight(fn, "shared down", sh_down, wdt))) return rc;
    if (sh_act == nullptr || sh_out == nullptr)
      return fail(MOE_ERR_NULL, "%s: sh_act or sh_out is NULL with S > 0", fn);
  }
  moe::GroupedArgs a{};
  a.x = act;
  a.w0 = down->w;
  a.s0 = down->scale;
  a.out = expert_out;
  a.N = H;
  a.K = I;
  if (S > 0) {
    a.sx = sh_act;
    a.sw0 = sh_down->w;
    a.ss0 = sh_down->scale;
    a.sout = sh_out;
    a.sN = H;
    a.sK = S;
  }
  fill_tables(a, t);
  a.M = (int)M;
  a.top_k = top_k;
  a.cap = s.cap;
  a.E = E;
  a.scale_rows = is_rows(wdt);
  return hip_status(
      moe::launch_grouped_down(a, fmt_of(wdt), is_tiled(wdt), stream), fn);
}

int moe_blend(void* out_bf16, const float* expert_out, const float* topk_weights, const int32_t* token_to_perm,
              const float* sh_out, const void* x_bf16, const void* sh_expert_gate, int64_t M, int32_t H,
              int32_t top_k, hipStream_t stream) {
  const char* fn = "moe_blend";
  if (M < 0 || H < 1 || top_k < 1) return fail(MOE_ERR_SHAPE, "%s: M=%lld H=%d top_k=%d", fn, (long long)M, H, top_k);
  if (H % 4) return fail(MOE_ERR_SHAPE, "%s: H=%d must be a multiple of 4", fn, H);
  if (M >= kInt32Limit / top_k) return fail(MOE_ERR_LIMIT, "%s: M*top_k reaches 2^31", fn);
  if (M == 0) return MOE_OK;
  if (!out_bf16 || !expert_out || !topk_weights || !token_to_perm)
    return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (sh_out && sh_expert_gate && !x_bf16) return fail(MOE_ERR_NULL, "%s: x is NULL with a shared gate", fn);
  int rc;
  if ((rc = check_aligned(fn, "out", out_bf16, 8)) || (rc = check_aligned(fn, "expert_out", expert_out, 16)) ||
      (rc = check_aligned(fn, "sh_out", sh_out, 16)))
    return rc;
  return hip_status(moe::launch_blend(static_cast<uint16_t*>(out_bf16), expert_out, topk_weights, token_to_perm,
                                      sh_out, x_bf16, sh_out ? sh_expert_gate : nullptr, (int)M, H, top_k, stream),
                    fn);
}

size_t moe_tiled_weight_bytes(moe_weight_dtype wdt, int64_t E, int32_t N, int32_t K) {
  const char* fn = "moe_tiled_weight_bytes";
  if (wdt != MOE_W_BF16 && wdt != MOE_W_FP8_E4M3 && wdt != MOE_W_FP8_E4M3_ROWS && wdt != MOE_W_MXFP4) {
    fail(MOE_ERR_SHAPE, "%s: source dtype %d is not a row-major dtype", fn, (int)wdt);
    return 0;
  }
  if (E < 1 || check_projection(fn, "weights", wdt, N, K) != MOE_OK) {
    if (E < 1) fail(MOE_ERR_SHAPE, "%s: E=%lld", fn, (long long)E);
    return 0;
  }
  return moe::tiled_weight_bytes(fmt_of(wdt), E, N, K);
}

int moe_tile_weights(const void* src, void* dst, moe_weight_dtype wdt, int64_t E, int32_t N, int32_t K,
                     hipStream_t stream) {
  const char* fn = "moe_tile_weights";
  if (moe_tiled_weight_bytes(wdt, E, N, K) == 0) return MOE_ERR_SHAPE;
  if (src == nullptr || dst == nullptr) return fail(MOE_ERR_NULL, "%s: src or dst is NULL", fn);
  if (src == dst) return fail(MOE_ERR_SHAPE, "%s: src and dst must not alias", fn);
  int rc;
  if ((rc = check_aligned(fn, "src", src, 16)) || (rc = check_aligned(fn, "dst", dst, 16))) return rc;
  return hip_status(moe::launch_tile_weights(src, dst, fmt_of(wdt), E, N, K, stream), fn);
}

int moe_layer_workspace_layout(const moe_layer_desc* d, size_t offsets[MOE_LAYER_WORKSPACE_REGIONS + 1]) {
  if (offsets == nullptr) return fail(MOE_ERR_NULL, "moe_layer_workspace_layout: offsets is NULL");
  return layout(d, offsets);
}

size_t moe_layer_workspace_bytes(const moe_layer_desc* d) {
  size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1];
  if (layout(d, off) != MOE_OK) return 0;
  return off[MOE_LAYER_WORKSPACE_REGIONS];
}

int moe_layer_path(const moe_layer_desc* d) {
  size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1];
  int path = 0;
  const int rc = layout(d, off, &path);
  return rc ? rc : path;
}

}  // extern "C"

namespace {

// Checks shared by the layer calls: the descriptor, the workspace and the
// weights.  Fills the workspace offsets and the path.
int layer_setup(const char* fn, const moe_layer_desc* d, const void* workspace, size_t workspace_bytes,
                size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1], int* path) {
  int rc = layout(d, off, path);
  if (rc) return rc;
  if (d->M == 0) return MOE_OK;
  if (workspace == nullptr) return fail(MOE_ERR_NULL, "%s: workspace is NULL", fn);
  if (workspace_bytes < off[MOE_LAYER_WORKSPACE_REGIONS])
    return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes,
                off[MOE_LAYER_WORKSPACE_REGIONS]);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", fn);
  if ((rc = check_weight(fn, "gate", &d->gate, d->wdt)) || (rc = check_weight(fn, "up", &d->up, d->wdt)) ||
      (rc = check_weight(fn, "down", &d->down, d->wdt)))
    return rc;
  if (d->S > 0 && ((rc = check_weight(fn, "shared gate", &d->sh_gate, d->wdt)) ||
                   (rc = check_weight(fn, "shared up", &d->sh_up, d->wdt)) ||
                   (rc = check_weight(fn, "shared down", &d->sh_down, d->wdt))))
    return rc;
  if (d->sh_expert_gate != nullptr && d->S == 0)
    return fail(MOE_ERR_SHAPE, "%s: a shared gate vector is given without a shared expert (S = 0)", fn);
  return MOE_OK;
}

moe_align_tables workspace_tables(char* ws, const size_t* off) {
  moe_align_tables t;
  t.sorted_token_ids = reinterpret_cast<int32_t*>(ws + off[0]);
  t.block_expert_ids = reinterpret_cast<int32_t*>(ws + off[1]);
  t.expert_offsets = reinterpret_cast<int32_t*>(ws + off[2]);
  t.expert_counts = reinterpret_cast<int32_t*>(ws + off[3]);
  t.token_to_perm = reinterpret_cast<int32_t*>(ws + off[4]);
  t.active_experts = reinterpret_cast<int32_t*>(ws + off[5]);
  t.active_count = reinterpret_cast<int32_t*>(ws + off[6]);
  t.total = reinterpret_cast<int32_t*>(ws + off[7]);
  return t;
}

moe::FusedLayerArgs single_pass_args(const moe_layer_desc* d, char* ws, const size_t* off, const void* x_bf16,
                                     const void* topk_ids, const float* topk_weights, void* out_bf16) {
  const bool shared = d->S > 0;
  const int64_t n = d->M * d->top_k;
  moe::FusedLayerArgs a{};
  a.ids = topk_ids;
  a.ids64 = d->idt == MOE_IDX_I64;
  a.x = x_bf16;
  const moe_weight* w[3] = {&d->gate, &d->up, &d->down};
  const moe_weight* sw[3] = {&d->sh_gate, &d->sh_up, &d->sh_down};
  for (int i = 0; i < 3; ++i) {
    a.w[i] = w[i]->w;
    a.s[i] = w[i]->scale;
    a.sw[i] = shared ? sw[i]->w : nullptr;
    a.ss[i] = shared ? sw[i]->scale : nullptr;
  }
  a.sh_gate = shared ? d->sh_expert_gate : nullptr;
  a.scale_rows = is_rows(d->wdt);
  a.topk_weights = topk_weights;
  a.out = static_cast<uint16_t*>(out_bf16);
  a.part = reinterpret_cast<float*>(ws + off[12]);
  a.sh_part = shared ? reinterpret_cast<float*>(ws + off[13]) : nullptr;
  a.M = (int)d->M;
  a.H = d->H;
  a.I = d->I;
  a.S = d->S;
  a.E = d->E;
  a.top_k = d->top_k;
  a.BS = d->BS;
  a.n = (int)n;
  a.cap = moe_active_cap(n, d->E);
  a.max_total = (int)moe_align_max_total(n, d->E, d->BS);
  a.tables = to_align_out(workspace_tables(ws, off));
  return a;
}

}  // namespace

extern "C" {

int moe_layer_partials(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "moe_layer_partials";
  size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1];
  int path = 0;
  int rc = layer_setup(fn, d, workspace, workspace_bytes, off, &path);
  if (rc || d->M == 0) return rc;
  if (path != MOE_LAYER_PATH_SINGLE_PASS)
    return fail(MOE_ERR_SHAPE, "%s: this layer shape does not take the single-pass path", fn);
  if (!x_bf16 || !topk_ids) return fail(MOE_ERR_NULL, "%s: x or topk_ids is NULL", fn);
  if ((rc = check_aligned(fn, "x", x_bf16, 16))) return rc;
  const moe::FusedLayerArgs a =
      single_pass_args(d, static_cast<char*>(workspace), off, x_bf16, topk_ids, nullptr, nullptr);
  return hip_status(moe::launch_layer_partials(a, fmt_of(d->wdt), stream), fn);
}

int moe_layer_blend_partials(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids,
                             const float* topk_weights, void* out_bf16, const void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const char* fn = "moe_layer_blend_partials";
  size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1];
  int path = 0;
  int rc = layer_setup(fn, d, workspace, workspace_bytes, off, &path);
  if (rc || d->M == 0) return rc;
  if (path != MOE_LAYER_PATH_SINGLE_PASS)
    return fail(MOE_ERR_SHAPE, "%s: this layer shape does not take the single-pass path", fn);
  if (!topk_ids || !topk_weights || !out_bf16)
    return fail(MOE_ERR_NULL, "%s: topk_ids, topk_weights or out is NULL", fn);
  if (d->sh_expert_gate && !x_bf16) return fail(MOE_ERR_NULL, "%s: x is NULL with a shared gate", fn);
  if ((rc = check_aligned(fn, "out", out_bf16, 8))) return rc;
  const moe::FusedLayerArgs a = single_pass_args(d, static_cast<char*>(const_cast<void*>(workspace)), off, x_bf16,
                                                 topk_ids, topk_weights, out_bf16);
  return hip_status(moe::launch_blend_partials(a, stream), fn);
}

int moe_layer_forward(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids, const float* topk_weights,
                      void* out_bf16, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "moe_layer_forward";
  size_t off[MOE_LAYER_WORKSPACE_REGIONS + 1];
  int path = 0;
  int rc = layer_setup(fn, d, workspace, workspace_bytes, off, &path);
  if (rc || d->M == 0) return rc;
  if (!x_bf16 || !topk_ids || !topk_weights || !out_bf16)
    return fail(MOE_ERR_NULL, "%s: x, topk_ids, topk_weights or out is NULL", fn);
  if ((rc = check_aligned(fn, "x", x_bf16, 16)) || (rc = check_aligned(fn, "out", out_bf16, 8))) return rc;
  log_path_once(d, path);
  char* ws = static_cast<char*>(workspace);
  if (path == MOE_LAYER_PATH_SINGLE_PASS) {
    const moe::FusedLayerArgs a = single_pass_args(d, ws, off, x_bf16, topk_ids, topk_weights, out_bf16);
    if ((rc = hip_status(moe::launch_layer_partials(a, fmt_of(d->wdt), stream), fn))) return rc;
    return hip_status(moe::launch_blend_partials(a, stream), fn);
  }
  if (path == MOE_LAYER_PATH_NARROW) {
    moe::FusedLayerArgs a = single_pass_args(d, ws, off, x_bf16, topk_ids, topk_weights, out_bf16);
    a.act = reinterpret_cast<float*>(ws + off[8]);
    a.sh_act = d->S > 0 ? reinterpret_cast<float*>(ws + off[10]) : nullptr;
    return hip_status(moe::launch_narrow_layer(a, stream), fn);
  }
  const bool shared = d->S > 0;
  const int64_t n = d->M * d->top_k;
  moe_align_tables t = workspace_tables(ws, off);
  float* act = reinterpret_cast<float*>(ws + off[8]);
  float* expert_out = reinterpret_cast<float*>(ws + off[9]);
  float* sh_act = shared ? reinterpret_cast<float*>(ws + off[10]) : nullptr;
  float* sh_out = shared ? reinterpret_cast<float*>(ws + off[11]) : nullptr;

  if (n <= moe::kFusedAlignMaxSlots && moe::grouped_passes(d->M) == 1) {
    // few slots and one workgroup row per expert: every gate+up workgroup
    // aligns topk_ids itself (in LDS) and one writes the tables, which saves
    // the align launch and its latency
    if ((rc = moe_align_gate_up_silu(topk_ids, d->idt, x_bf16, d->wdt, &d->gate, &d->up, &t, act,
                                     shared ? &d->sh_gate : nullptr, shared ? &d->sh_up : nullptr, sh_act, d->M,
                                     d->H, d->I, d->S, d->E, d->top_k, d->BS, stream)))
      return rc;
  } else {
    // the blocks' expert counts of the two-launch align go to the expert_out
    // region, which only the down projection writes, later on the stream
    const size_t need = moe::align_workspace_bytes((int)n, d->E), room = off[10] - off[9];
    if ((rc = need <= room ? moe_align_ws(topk_ids, d->idt, d->M, d->top_k, d->E, d->BS, &t, expert_out, room, stream)
                           : moe_align(topk_ids, d->idt, d->M, d->top_k, d->E, d->BS, &t, stream)))
      return rc;
    if ((rc = moe_grouped_gate_up_silu(x_bf16, d->wdt, &d->gate, &d->up, &t, act, shared ? &d->sh_gate : nullptr,
                                       shared ? &d->sh_up : nullptr, sh_act, d->M, d->H, d->I, d->S, d->E, d->top_k,
                                       d->BS, stream)))
      return rc;
  }
  if ((rc = moe_grouped_down(act, d->wdt, &d->down, &t, expert_out, shared ? &d->sh_down : nullptr, sh_act, sh_out,
                             d->M, d->H, d->I, d->S, d->E, d->top_k, d->BS, stream)))
    return rc;
  return moe_blend(out_bf16, expert_out, topk_weights, t.token_to_perm, sh_out, x_bf16,
                   shared ? d->sh_expert_gate : nullptr, d->M, d->H, d->top_k, stream);
}

int moe_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, hipStream_t stream) {
  const char* fn = "moe_stream_read_probe";
  if (bytes % 16) return fail(MOE_ERR_SHAPE, "%s: bytes=%zu is not a multiple of 16", fn, bytes);
  if (blocks < 1 || blocks > 65536) return fail(MOE_ERR_SHAPE, "%s: blocks=%d outside [1, 65536]", fn, blocks);
  if (bytes == 0) return MOE_OK;
  if (!src || !sink) return fail(MOE_ERR_NULL, "%s: src or sink is NULL", fn);
  if (reinterpret_cast<uintptr_t>(src) % 16) return fail(MOE_ERR_SHAPE, "%s: src is not 16-byte aligned", fn);
  return hip_status(moe::launch_stream_read(src, bytes, sink, blocks, stream), fn);
}

int moe_router_topk(const void* x_bf16, const void* router_w_bf16, int64_t M, int32_t H, int32_t E, int32_t top_k,
                    float* logits, void* topk_ids, moe_index_dtype idt, float* topk_weights, hipStream_t stream) {
  const char* fn = "moe_router_topk";
  if (M < 0) return fail(MOE_ERR_SHAPE, "%s: M=%lld is negative", fn, (long long)M);
  if (M >= ((int64_t)1 << 20)) return fail(MOE_ERR_LIMIT, "%s: M=%lld reaches 2^20 rows", fn, (long long)M);
  if (H < 8 || H % 8) return fail(MOE_ERR_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if (E < 1) return fail(MOE_ERR_SHAPE, "%s: E=%d must be >= 1", fn, E);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_LIMIT, "%s: E=%d exceeds the %d experts the router handles", fn, E, MOE_MAX_EXPERTS);
  if (top_k < 1 || top_k > E || top_k > MOE_ROUTER_MAX_TOP_K)
    return fail(MOE_ERR_SHAPE, "%s: top_k=%d must be in [1, min(E, %d)]", fn, top_k, MOE_ROUTER_MAX_TOP_K);
  if (idt != MOE_IDX_I32 && idt != MOE_IDX_I64)
    return fail(MOE_ERR_SHAPE, "%s: unknown index dtype %d", fn, (int)idt);
  if (M == 0) return MOE_OK;
  if (!x_bf16 || !router_w_bf16 || !logits || !topk_ids || !topk_weights)
    return fail(MOE_ERR_NULL, "%s: x, router weight, logits, topk_ids or topk_weights is NULL", fn);
  int rc;
  if ((rc = check_aligned(fn, "x", x_bf16, 16)) || (rc = check_aligned(fn, "router weight", router_w_bf16, 16)))
    return rc;
  return hip_status(moe::launch_router(x_bf16, router_w_bf16, (int)M, H, E, top_k, logits, topk_ids,
                                       idt == MOE_IDX_I64, topk_weights, stream),
                    fn);
}

}  // extern "C"
