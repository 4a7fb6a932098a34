/*
 * moe_mi355x.h - C ABI of the MI355X (gfx950) MoE routing-align + grouped
 * expert FFN library (libmoe_mi355x.so).
 *
 * The path, restated from the pages that define it:
 *   1. align  - a deterministic on-device sort of the (token, k) slots by
 *      expert: per-expert counts, padding to a block size BS, the exclusive
 *      prefix of the padded counts, a stable within-expert rank, the
 *      block->expert map, token_to_perm and the ascending active-expert list
 *      (nbxtensor 0.0.1 wheel page, moe_align.py: module docstring and the
 *      three stage kernels; metrale fp8_moe_grouped.rs: moe_fp8_grouped_sort
 *      and Fp8GroupedSortOut);
 *   2. gate+up with SiLU and 3. down over the sorted slots, one workgroup
 *      column per active expert, each weight row streamed once for every row
 *      routed to that expert (fp8_moe_grouped.rs: module doc and the gate+up
 *      and down launchers);
 *   4. blend - each token's router-weighted sum of its slots' expert outputs,
 *      looked up through token_to_perm, in a fixed k order, plus the shared
 *      expert (fp8_moe_grouped.rs: moe_weighted_sum_blend_fp8_grouped;
 *      moe_decode_vec.py: moe_part_reduce_kernel's fixed-order sum).
 *
 * Conventions for every entry point:
 *   - All buffers are device memory owned by the caller.  The library never
 *     allocates, never synchronises and never reads device data on the host,
 *     so every call can be captured in a HIP graph and replayed for any routing.
 *   - Work is enqueued on `stream` (0 = the null stream) in call order.
 *   - Host-side argument checks come first: on failure the call returns a
 *     negative moe_status, records a message for moe_last_error() and
 *     launches nothing.  MOE_ERR_HIP reports a failed kernel launch.
 *   - M == 0 returns MOE_OK and launches nothing.
 *   - Slot ids outside [0, E) are dropped on the device: they are in no count
 *     or table, get token_to_perm = -1 and add nothing to the blend (the
 *     stage-3 kernel of moe_align.py skips them the same way).
 *   - Weight matrices are row-major [N, K] per expert (N output rows, K input
 *     columns) stacked over experts: gate/up [E, I, H], down [E, H, I]; the
 *     shared expert's are [S, H] and [H, S].  FP8 weights are OCP E4M3
 *     (e4m3fn) codes with one float32 scale per 128x128 block, row-major
 *     [E, N/128, K/128] (fp8_moe_grouped.rs, fp8_grouped_tc_shape_ok: FP8
 *     projections come in whole 128 blocks, the scale blocks), or, with the
 *     _ROWS weight dtypes, one float32 scale per output row, [E, N].  BF16
 *     weights take no scale.
 *   - Activations x are bf16 [M, H]; intermediates are float32; the output is
 *     bf16 [M, H], one round-to-nearest-even of the float32 blend sum.
 *   - Alignment: the kernels move weights (tiled or row-major), x, the router
 *     weight, act, sh_act, expert_out and sh_out 16 bytes per lane, and the
 *     bf16 output 8 bytes per lane.  Those pointers must be 16-byte (output:
 *     8-byte) aligned; any other is refused with MOE_ERR_SHAPE before any
 *     launch.  Ids, routing weights, block scales and the shared-expert gate
 *     vector need only their element alignment.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,      /* a required pointer is NULL                          */
  MOE_ERR_SHAPE = -2,     /* a size is negative, zero where it must not be, or
                             not a whole number of the blocks the kernels need   */
  MOE_ERR_LIMIT = -3,     /* E > MOE_MAX_EXPERTS, or a table would need >= 2^31
                             entries                                             */
  MOE_ERR_WORKSPACE = -4, /* workspace smaller than moe_layer_workspace_bytes()  */
  MOE_ERR_HIP = -5        /* the HIP runtime reported a launch failure           */
} moe_status;

typedef enum { MOE_IDX_I32 = 0, MOE_IDX_I64 = 1 } moe_index_dtype;

/* Expert weight element type and layout.  The row-major forms are [E, N, K];
 * the tiled forms are the same values reordered by moe_tile_weights() so that
 * every wave streams one contiguous run (see there).  Both layouts give
 * bit-identical results.  FP8 weights carry float32 scales: one per 128x128
 * block (the FP8 grouped GEMM page's block-wise scaling), or, in the _ROWS
 * forms, one per output row of each expert (the FP8 page's per-row scale of
 * its shared-expert weights, here for every expert).  A weight is the code's
 * e4m3fn value times its scale.
 * MXFP4 is the 4-bit expert format (the layer page's 4-bit grouped experts,
 * in the OCP microscaling form gfx950 converts natively): E2M1 codes, two per
 * byte, the lower nibble holding the lower k, so a row is K/2 bytes; one E8M0
 * scale byte per 32 consecutive k of a row, [E, N, K/32] uint8.  A weight is
 * the code's E2M1 value times 2^(scale byte - 127). */
typedef enum {
  MOE_W_BF16 = 0,                /* bf16, row-major [E, N, K]                  */
  MOE_W_FP8_E4M3 = 1,            /* e4m3fn codes, row-major [E, N, K], scales
                                    [E, N/128, K/128]                          */
  MOE_W_BF16_TILED = 2,          /* bf16, tiled by moe_tile_weights            */
  MOE_W_FP8_E4M3_TILED = 3,      /* e4m3fn codes, tiled; block scales as above */
  MOE_W_FP8_E4M3_ROWS = 4,       /* e4m3fn codes, row-major [E, N, K], scales
                                    [E, N] (16-byte aligned)                   */
  MOE_W_FP8_E4M3_ROWS_TILED = 5, /* e4m3fn codes, tiled; row scales as above   */
  MOE_W_MXFP4 = 6,               /* E2M1 codes, row-major [E, N, K/2] bytes;
                                    E8M0 scales [E, N, K/32] (4-byte aligned)  */
  MOE_W_MXFP4_TILED = 7          /* E2M1 codes, tiled; scales as above         */
} moe_weight_dtype;

/* Experts one align launch handles (fp8_moe_grouped.rs: the one-launch sort's
 * 1024-expert limit, FP8_GROUPED_SORT_MAX_EXPERTS). */
#define MOE_MAX_EXPERTS 1024

/* ---------------------------------------------------------------- sizing --
 * Pure host functions; no GPU needed.                                       */

/* Worst-case length of sorted_token_ids for n = M*top_k slots:
 * min(n*BS, n + E*(BS-1)) rounded up to a multiple of BS (moe_align.py,
 * module docstring).  block_expert_ids has moe_align_max_total(...)/BS
 * entries.  Returns -1 for a negative n or a non-positive E or BS. */
int64_t moe_align_max_total(int64_t n, int32_t E, int32_t BS);

/* Length of active_experts: min(n, E), the most distinct experts n slots can
 * reach; it does not depend on the routing (fp8_moe_grouped.rs,
 * fp8_grouped_active_cap).  Returns -1 for a negative n or E. */
int32_t moe_active_cap(int64_t n, int32_t E);

/* Text of the last failure on the calling thread ("" if none).  The pointer
 * stays valid until the thread's next failing call. */
const char* moe_last_error(void);

/* ABI version of this header (increases on any change). */
int32_t moe_abi_version(void);

/* ------------------------------------------------------------- align -- */

/* Alignment tables; all int32 device arrays allocated by the caller. */
typedef struct {
  int32_t* sorted_token_ids; /* [max_total]  flat slot i = t*top_k + k; the
                                sentinel n = M*top_k at every padding position */
  int32_t* block_expert_ids; /* [max_total/BS] owning expert of each BS block,
                                -1 for blocks at or past the total            */
  int32_t* expert_offsets;   /* [E+1] exclusive prefix of the padded counts;
                                expert_offsets[E] = total                     */
  int32_t* expert_counts;    /* [E] in-range slots per expert (unpadded)      */
  int32_t* token_to_perm;    /* [n] sorted position of slot i, -1 if dropped  */
  int32_t* active_experts;   /* [cap] experts with a slot, ascending, then -1 */
  int32_t* active_count;     /* [1] number of active experts                  */
  int32_t* total;            /* [1] padded total; lives only on the device    */
} moe_align_tables;

/* Sort the n = M*top_k slots of topk_ids ([M, top_k] row-major, int32 or
 * int64 per idt) by expert, stably (a slot's rank within its expert is the
 * number of earlier slots with the same id), with no atomics: the tables are
 * bit-identical run to run and equal to a host stable sort's.
 * Errors: MOE_ERR_NULL (topk_ids or a table pointer NULL with M > 0),
 * MOE_ERR_SHAPE (M < 0, top_k < 1, E < 1, BS < 1), MOE_ERR_LIMIT
 * (E > MOE_MAX_EXPERTS, n or max_total >= 2^31). */
int moe_align(const void* topk_ids, moe_index_dtype idt, int64_t M, int32_t top_k,
              int32_t E, int32_t BS, const moe_align_tables* out, hipStream_t stream);

/* Bytes of device workspace moe_align_ws needs for n = M*top_k slots over E
 * experts: 4*E per block of 1024 slots from 4096 slots on, else 0 (also 0 for
 * arguments moe_align would refuse). */
size_t moe_align_workspace_bytes(int64_t M, int32_t top_k, int32_t E);

/* moe_align with a caller-owned workspace for the per-block expert counts
 * (`workspace_bytes` >= moe_align_workspace_bytes(M, top_k, E), 16-byte
 * aligned; it may be NULL when that size is 0).  Without it the counts of the
 * blocks of 1024 slots must live in token_to_perm until the scatter overwrites
 * them, which takes three launches (count, one-workgroup scan, scatter); with
 * it, two: count, then a scatter in which every block forms the offsets and its
 * own bases from all blocks' counts.  The tables are bit-identical to
 * moe_align's (the same stable order; still no atomics), and the workspace
 * holds nothing after the call that the caller needs.  Below 4096 slots this
 * is moe_align (one workgroup), and so it is where E * G^2 (G blocks of 1024
 * slots) passes 256 * 512^2: every scatter block reads all blocks' counts,
 * which past that costs more than the three launches' single scan (measured
 * on MI355X at 256 experts: faster up to 512 blocks, slower from 576).  Errors as for moe_align, plus MOE_ERR_NULL
 * (workspace NULL when needed), MOE_ERR_WORKSPACE (too small), MOE_ERR_SHAPE
 * (misaligned). */
int moe_align_ws(const void* topk_ids, moe_index_dtype idt, int64_t M, int32_t top_k,
                 int32_t E, int32_t BS, const moe_align_tables* out, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------- weight tiling --
 * A one-time, load-time reordering of an expert weight tensor (the source pages
 * describe such a load-time repack for their lean tensor-core kernels:
 * metrale forward_nvfp4_grouped_decode.rs, Nvfp4GroupedKernels doc).  The tiled
 * copy holds, for each expert, 16-row tiles; in a tile, 128-deep chunks (K
 * zero-padded up to a multiple of 128); in a chunk, 1 KB fragments in which the
 * 16 bytes lane l of a wave feeds the matrix core sit at byte 16*l.  A wave
 * then reads its weights as one contiguous stream (on MI355X, ~1.3x the HBM
 * bandwidth of reading 16 row-major rows side by side).  Scales are unchanged. */

/* Bytes of the tiled copy of row-major weights of dtype `wdt` (MOE_W_BF16,
 * MOE_W_FP8_E4M3, MOE_W_FP8_E4M3_ROWS or MOE_W_MXFP4: the codes tile the same
 * way whatever their scales) and shape [E, N, K]: E * N * roundup(K, 128) *
 * element size (half a byte for MXFP4, whose 1 KB fragments hold two 512-byte
 * halves, each the 64-deep half of the chunk with lane l's 8 bytes at 8*l).
 * Returns 0 for an invalid shape (the projection rules of the grouped calls). */
size_t moe_tiled_weight_bytes(moe_weight_dtype wdt, int64_t E, int32_t N, int32_t K);

/* Write the tiled copy of `src` (row-major, dtype `wdt`) into `dst` (device,
 * moe_tiled_weight_bytes bytes, must not overlap src) on `stream`.  The result
 * is used with MOE_W_BF16_TILED, MOE_W_FP8_E4M3_TILED,
 * MOE_W_FP8_E4M3_ROWS_TILED or MOE_W_MXFP4_TILED. */
int moe_tile_weights(const void* src, void* dst, moe_weight_dtype wdt, int64_t E, int32_t N, int32_t K,
                     hipStream_t stream);

/* ---------------------------------------------------- grouped expert FFN -- */

/* One projection's weights: w is [E, N, K] (bf16 or e4m3fn codes; MXFP4:
 * [E, N, K/2] bytes), row-major or tiled as the call's weight dtype says;
 * scale is float32 [E, N/128, K/128] for block-scaled FP8, float32 [E, N] for
 * row-scaled FP8, uint8 E8M0 [E, N, K/32] for MXFP4, and ignored (may be NULL)
 * for BF16.  FP8 needs N and K in whole multiples of 128 either way; MXFP4
 * needs K a multiple of 128 and N of 16.  MXFP4 scale bytes from 2 to 252
 * give every weight exactly (its value is a bf16); outside that range (255 is
 * E8M0's NaN) the results are not specified. */
typedef struct {
  const void* w;
  const void* scale;
} moe_weight;

/* act[p, :] = silu(g) * u with g = W_gate[e] x[t], u = W_up[e] x[t] for every
 * sorted position p holding a slot of active expert e (t = slot / top_k);
 * act is float32 [max_total, I], rows indexed by sorted position; padding rows
 * are not written.  With a shared expert (sh_gate and sh_up non-NULL, S > 0)
 * the same launch writes sh_act[t, :] (float32 [M, S]) for every token.
 * `t` are the tables moe_align wrote for the same topk_ids.
 * Shapes: FP8 needs H, I, S multiples of 128; BF16 needs H multiple of 32 and
 * I, S multiples of 16; MXFP4 needs H a multiple of 128 and I, S of 16.
 * Errors as for moe_align, plus MOE_ERR_SHAPE for the block rules above. */
int moe_grouped_gate_up_silu(const void* x_bf16, moe_weight_dtype wdt, const moe_weight* gate,
                             const moe_weight* up, const moe_align_tables* t, float* act,
                             const moe_weight* sh_gate, const moe_weight* sh_up, float* sh_act,
                             int64_t M, int32_t H, int32_t I, int32_t S, int32_t E,
                             int32_t top_k, int32_t BS, hipStream_t stream);

/* Slot counts up to this use the one-launch alignment + gate+up below. */
#define MOE_FUSED_ALIGN_MAX_SLOTS 2048

/* moe_align followed by moe_grouped_gate_up_silu in ONE launch, for
 * n = M*top_k <= MOE_FUSED_ALIGN_MAX_SLOTS: every gate+up workgroup aligns
 * topk_ids itself in LDS (the same deterministic counts, scan and stable rank)
 * to find its expert and rows, and one workgroup writes all of `t`.  The
 * tables and act equal the two separate calls' bit for bit; the saving is the
 * align launch and the dependent table reads in front of the weight stream.
 * Errors: as for the two calls, plus MOE_ERR_LIMIT for n above the limit. */
int moe_align_gate_up_silu(const void* topk_ids, moe_index_dtype idt, const void* x_bf16, moe_weight_dtype wdt,
                           const moe_weight* gate, const moe_weight* up, const moe_align_tables* t, float* act,
                           const moe_weight* sh_gate, const moe_weight* sh_up, float* sh_act, int64_t M,
                           int32_t H, int32_t I, int32_t S, int32_t E, int32_t top_k, int32_t BS,
                           hipStream_t stream);

/* expert_out[p, :] = W_down[e] act[p, :] for every slot position p of active
 * expert e (float32 [max_total, H]; padding rows not written); with a shared
 * expert (sh_down non-NULL, S > 0) also sh_out[t, :] = W_sh_down sh_act[t, :]
 * (float32 [M, H]).  The depth is summed in 64-deep halves of 128-deep chunks,
 * ascending, from 0: each half's float32 product (times its block or row scale, FP8)
 * is rounded and then added, with no fused multiply-add across halves.  Shapes: FP8 needs H,
 * I, S multiples of 128; BF16 needs I, S multiples of 32 and H a multiple of 16;
 * MXFP4 needs I, S multiples of 128 and H of 16. */
int moe_grouped_down(const float* act, moe_weight_dtype wdt, const moe_weight* down,
                     const moe_align_tables* t, float* expert_out, const moe_weight* sh_down,
                     const float* sh_act, float* sh_out, int64_t M, int32_t H, int32_t I,
                     int32_t S, int32_t E, int32_t top_k, int32_t BS, hipStream_t stream);

/* out[t, :] = bf16( (sum over k = 0..top_k-1 in that order of
 * w[t*top_k+k] * expert_out[token_to_perm[t*top_k+k], :]) + g_t * sh_out[t, :] ),
 * float32 fused multiply-adds, a slot with token_to_perm < 0 skipped, sh_out
 * NULL for no shared expert; one round-to-nearest-even at the end.  The
 * shared term is added as is when sh_expert_gate is NULL; else it is scaled
 * by g_t = sigmoid(x[t] . sh_expert_gate) (bf16 x [M, H] and bf16 gate vector
 * [H], a float32 dot product in a fixed order; fp8_moe_grouped.rs: the blend
 * takes the layer input and the shared expert's gate weight, ungated when the
 * weight is absent).  A row's bits depend only on that token's inputs (not on
 * M).  H must be a multiple of 4; x must be given with a gate. */
int moe_blend(void* out_bf16, const float* expert_out, const float* topk_weights,
              const int32_t* token_to_perm, const float* sh_out, const void* x_bf16,
              const void* sh_expert_gate, int64_t M, int32_t H, int32_t top_k, hipStream_t stream);

/* ------------------------------------------------------------ whole layer -- */

/* The three ways moe_layer_forward runs.  A descriptor asks for one with its
 * `path` field; MOE_LAYER_PATH_AUTO (0) lets the library choose from the
 * descriptor's shapes (never from the routing, so a captured graph stays valid
 * for any routing): the narrow path for at most MOE_NARROW_AUTO_SLOTS slots
 * where it fits; else the single pass where it fits, except where the steps
 * measured faster on MI355X (MXFP4 and per-row FP8 scales at every width;
 * block-scaled FP8 where the slots exceed 6 times the rows of one pass of the
 * 4- and 8-row pass classes, e.g. 4, 7 and 8 tokens at top-8); else the
 * steps.  Every path gives the same bits, so the choice changes only time.
 * (The FP8 page picks its decode kernel pair the same way, from the shape and
 * a kill switch read once: metrale forward_nvfp4_grouped_decode.rs,
 * nvfp4_grouped_tc_enabled.)
 *  - MOE_LAYER_PATH_STEPS: align (fused into gate+up for at most
 *    MOE_FUSED_ALIGN_MAX_SLOTS slots when every expert fits one pass; from
 *    4096 slots the two-launch moe_align_ws, its block counts held in the
 *    expert_out region until the down projection overwrites it),
 *    gate+up+SiLU, down and blend, the same kernels the entry points above
 *    launch.  Runs every valid descriptor.
 *  - MOE_LAYER_PATH_SINGLE_PASS: tiled weights and at most
 *    MOE_FUSED_LAYER_MAX_SLOTS slots (decode width).  One launch aligns and, per
 *    active expert and 64-wide slice j of the intermediate, runs gate+up+SiLU
 *    into LDS and then the 64-deep slice j of down, writing float32 partial
 *    outputs part[j][slot][:]; a second launch forms each slot's expert output
 *    as the sum of its slices (j ascending, from 0) and blends.  The separate
 *    down projection sums the 64-deep halves of its chunks in the same order,
 *    so both paths give the same bits.  (The decomposition of the layer into gate+up then down
 *    per expert is metrale forward_nvfp4_grouped_decode.rs's; the per-slice
 *    split is this library's.)  Forcing it on a descriptor it does not fit
 *    (row-major weights, more slots, LDS) is refused with MOE_ERR_SHAPE.
 *  - MOE_LAYER_PATH_NARROW: tiled FP8 weights and at most
 *    MOE_NARROW_LAYER_MAX_SLOTS slots (a few tokens), within its LDS budget.
 *    Launch 1 aligns (one workgroup writes the tables) and runs gate+up+SiLU
 *    per (expert, 16-column tile) with the depth split over 8 waves: each
 *    wave leaves the MFMA sums of its 128-deep chunks in LDS and one thread
 *    per output runs the chunk chain in ascending order, writing act (float32
 *    [n, I] by slot; shared expert [M, S] by token) to the workspace.  Launch 2
 *    runs down and the blend per 16 rows of H, the 64-deep halves' scaled sums
 *    added in ascending order.  The same bits as the other two paths.  Forcing
 *    it on a descriptor it does not fit is refused with MOE_ERR_SHAPE.
 * Environment, read once per process:
 *  - MOE_FORCE_PATH=steps | single_pass | narrow replaces MOE_LAYER_PATH_AUTO in every
 *    descriptor (an explicit `path` wins); any other value is ignored;
 *  - MOE_LOG=1 prints one line to stderr the first time moe_layer_forward runs
 *    each path in the process, naming the path and the layer's shapes. */
typedef enum {
  MOE_LAYER_PATH_AUTO = 0,
  MOE_LAYER_PATH_STEPS = 1,
  MOE_LAYER_PATH_SINGLE_PASS = 2,
  MOE_LAYER_PATH_NARROW = 3
} moe_layer_path_kind;

/* Slot counts (M*top_k) the narrow path takes, and up to which AUTO picks it. */
#define MOE_NARROW_LAYER_MAX_SLOTS 32
#define MOE_NARROW_AUTO_SLOTS 24
typedef struct {
  int64_t M;          /* tokens                                       */
  int32_t H;          /* hidden size                                  */
  int32_t I;          /* routed expert intermediate size              */
  int32_t S;          /* shared expert intermediate size (0: none)    */
  int32_t E;          /* routed experts                               */
  int32_t top_k;
  int32_t BS;         /* alignment block size                         */
  moe_weight_dtype wdt;
  moe_index_dtype idt;
  moe_weight gate, up, down;            /* routed experts                  */
  moe_weight sh_gate, sh_up, sh_down;   /* shared expert (.w NULL if none) */
  const void* sh_expert_gate;           /* bf16 [H] gate vector of the shared
                                           expert's output (moe_blend), or NULL:
                                           ungated; only with S > 0      */
  moe_layer_path_kind path;             /* MOE_LAYER_PATH_AUTO (0: a zeroed
                                           descriptor) or a forced path   */
} moe_layer_desc;

#define MOE_FUSED_LAYER_MAX_SLOTS 256

/* Workspace regions of moe_layer_forward, in this order: sorted_token_ids,
 * block_expert_ids, expert_offsets, expert_counts, token_to_perm,
 * active_experts, active_count, total (the tables, int32), then float32:
 * act [max_total, I], expert_out [max_total, H], sh_act [M, S], sh_out [M, H]
 * (the steps path), part [ceil(I/64), M*top_k, H] and sh_part [ceil(S/64), M, H]
 * (the single-pass path).  The narrow path uses act as [M*top_k, I] by slot
 * and sh_act [M, S].  A region the chosen path (or a layer without a shared
 * expert) does not use has size 0. */
#define MOE_LAYER_WORKSPACE_REGIONS 14

/* Bytes of workspace moe_layer_forward needs for `d`, each region 256-byte
 * aligned.  Depends on the shapes only, never on the routing.  Returns 0 for
 * an invalid descriptor (moe_last_error says why). */
size_t moe_layer_workspace_bytes(const moe_layer_desc* d);

/* The moe_layer_path_kind (STEPS or SINGLE_PASS) moe_layer_forward takes for
 * `d`, or a negative moe_status for an invalid descriptor or a forced path
 * that does not fit it. */
int moe_layer_path(const moe_layer_desc* d);

/* The whole layer on `stream`: align, gate+up+SiLU, down, blend, with no host
 * synchronisation.  x is bf16 [M, H], topk_ids [M, top_k] (d->idt),
 * topk_weights float32 [M, top_k], out bf16 [M, H].  The workspace (device,
 * >= moe_layer_workspace_bytes(d), 256-byte aligned) holds the tables and the
 * chosen path's intermediates afterwards, laid out as
 * moe_layer_workspace_layout says.  Errors: as for the four steps, plus
 * MOE_ERR_WORKSPACE. */
int moe_layer_forward(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids,
                      const float* topk_weights, void* out_bf16, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_forward with its workspace in a device array the library owns,
 * MOE_NOALLOC_WORKSPACE_BYTES bytes on each GPU it runs on, held from the
 * module's load until the process ends.  The caller still passes x, topk_ids,
 * topk_weights and out.  The call allocates nothing; the array's device
 * address is looked up once per device, on the first call with that device
 * current.  Every call on one GPU shares that GPU's array and leaves its
 * tables and intermediates there (nothing in it has to start at zero), so calls
 * that overlap on one GPU (several streams or threads at once) race: serialize
 * them.  Errors: those of moe_layer_forward, plus MOE_ERR_WORKSPACE when
 * moe_layer_workspace_bytes(d) exceeds the array (64 MiB: the tiny, decode and
 * verify-width layers fit; the 7168-wide layer does not). */
#define MOE_NOALLOC_WORKSPACE_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids,
                              const float* topk_weights, void* out_bf16, hipStream_t stream);

/* The two launches of the single-pass path, callable one at a time (for
 * example to time each); moe_layer_forward on that path is exactly
 * moe_layer_partials followed by moe_layer_blend_partials on the same
 * workspace.  moe_layer_partials aligns topk_ids (writing the tables into the
 * workspace) and writes the float32 partial outputs part / sh_part;
 * moe_layer_blend_partials reads them with topk_ids and topk_weights (and x,
 * for the shared gate when d->sh_expert_gate is set; else x may be NULL) and
 * writes out (bf16 [M, H]).  Both return MOE_ERR_SHAPE when `d` does not take
 * MOE_LAYER_PATH_SINGLE_PASS; other errors as for moe_layer_forward. */
int moe_layer_partials(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);
int moe_layer_blend_partials(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids,
                             const float* topk_weights, void* out_bf16, const void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Byte offsets of the MOE_LAYER_WORKSPACE_REGIONS regions, in the order above;
 * offsets[MOE_LAYER_WORKSPACE_REGIONS] is the total size.  Returns MOE_OK or an
 * error for an invalid descriptor. */
int moe_layer_workspace_layout(const moe_layer_desc* d, size_t offsets[MOE_LAYER_WORKSPACE_REGIONS + 1]);

/* ---------------------------------------------------------------- router --
 * The step before the path: the per-row router that turns token activations
 * into the topk_ids / topk_weights every call above takes (metrale
 * forward_nvfp4_grouped_decode.rs, the decode layer's admission predicate: a
 * BF16 softmax gate with no correction bias, computed by a router GEMV over the
 * batch rows and a per-row top-k softmax).
 *
 *   logits[t][e] = sum_h W[e][h] * x[t][h]      x bf16 [M, H], W bf16 [E, H],
 *                                               float32 accumulation
 *   topk_ids[t]  = the top_k largest logits of row t, larger first; equal
 *                  logits go to the lower expert
 *   topk_weights[t][j] = softmax over the chosen logits (the full softmax over
 *                  E, renormalised over its top k: the two are equal)
 *
 * Writes logits (float32 [M, E], caller-owned device memory; also the hand-off
 * between the two launches), topk_ids ([M, top_k], int32 or int64 per idt) and
 * topk_weights (float32 [M, top_k]).  Requires H a multiple of 8 (>= 8),
 * 1 <= E <= MOE_MAX_EXPERTS, 1 <= top_k <= min(E, MOE_ROUTER_MAX_TOP_K),
 * M < 2^20; finite logits (a NaN logit leaves the choice unspecified).  Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_LIMIT (E or M too large), MOE_ERR_HIP.
 * M == 0 launches nothing. */
#define MOE_ROUTER_MAX_TOP_K 64
int moe_router_topk(const void* x_bf16, const void* router_w_bf16, int64_t M, int32_t H, int32_t E, int32_t top_k,
                    float* logits, void* topk_ids, moe_index_dtype idt, float* topk_weights, hipStream_t stream);

/* Measurement aid, not part of the layer: one launch that reads `bytes` of
 * device memory at `src` with 16-byte vector loads and does nothing else,
 * giving the plain HBM read rate for a buffer of that size against which the
 * layer's weight-stream bandwidth is judged.  `blocks` workgroups of 256
 * threads (1 <= blocks <= 65536) read it in 16 KB tiles, tile i by workgroup
 * i mod blocks; each wave XOR-folds what it read into one 32-bit word of
 * `sink` (device, at least 4 * blocks words, caller-owned), so the loads are
 * not dead.  `bytes` must be
 * a multiple of 16 and `src` 16-byte aligned.  Errors: MOE_ERR_NULL (src or
 * sink NULL with bytes > 0), MOE_ERR_SHAPE (bytes not a multiple of 16, src
 * misaligned, blocks out of range), MOE_ERR_HIP.  bytes == 0 launches
 * nothing. */
int moe_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
