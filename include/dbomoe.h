/*
 * dbomoe.h - C ABI of the Dual-Batch-Overlap (DBO) expert-parallel MoE layer
 * for AMD Instinct MI355X (gfx950), on one GPU's share of the work.
 *
 * The layer: a batch is split into two microbatches; each runs top-k routing,
 * a dispatch that counting-sorts its tokens into contiguous per-expert rows
 * (the single-GPU stand-in for the all-to-all dispatch), a grouped SwiGLU
 * expert FFN, and a combine that gathers, weights and sums each token's expert
 * outputs (stand-in for the all-to-all combine).  The two microbatches are
 * interleaved on a compute stream and a comm stream and joined by
 * per-microbatch events recorded before each yield.
 * Sources: "[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", Purpose
 * (split, two streams, yields, equal yield counts); "[Perf] Fix DBO overlap:
 * capture DeepEP event before yield", Purpose (event recorded before the
 * yield); "DeepEP HT: full decode CUDA graphs via worst-token dispatch", bot
 * reviews (device-side per-expert counts, worst-case capacity, reserved
 * workspace, aligned slices, loud errors, one id dtype).
 *
 * Conventions shared by every entry point
 *  - Pointers named x, w_*, out, ... are DEVICE pointers; structs passed by
 *    pointer (params, desc, opts) are HOST memory read during the call only.
 *  - The caller owns every buffer.  No entry point allocates or frees device
 *    memory; dbo_ctx owns only HIP events.
 *  - Work is enqueued on the given HIP stream(s) (hipStream_t passed as void*;
 *    NULL = the null stream) and the call returns without a host sync.
 *    Counts and offsets stay on the device.
 *  - All argument checks run before the first launch: on any error nothing is
 *    enqueued.  A failed launch returns MOE_ERR_HIP.
 *  - Every device pointer must be 16-byte aligned, workspaces 256-byte aligned
 *    (else MOE_ERR_MISALIGNED).
 *  - Expert ids are int32 everywhere; routing weights are fp32.
 *  - Layouts are row-major and contiguous unless stated.
 */
#ifndef DBOMOE_H
#define DBOMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* a size, range, NULL pointer or combination is invalid */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but not implemented (dtype combo, shape multiple) */
  MOE_ERR_MISALIGNED = -3,   /* pointer or row pitch alignment violated */
  MOE_ERR_WORKSPACE = -4,    /* workspace smaller than the *_workspace_size query */
  MOE_ERR_HIP = -5           /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3FN = 2 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* Routing parameters.  The pages fix no routing rule; this is the reading:
 * softmax top-k (selection on logits, ties -> lower expert index, slot j =
 * rank j) or sigmoid scores with optional group-limited selection (groups of
 * E/n_groups consecutive experts, group score = sum of the group_topn best
 * scores, keep topk_groups groups, ties -> lower index).  Weight of slot j:
 * softmax probability or sigmoid score of its expert, optionally divided by
 * the sum over the k slots, then multiplied by routed_scale. */
typedef struct {
  int32_t E;            /* routed experts, 1..256 */
  int32_t k;            /* experts per token, 1..16, k <= E */
  int32_t score;        /* moe_score */
  int32_t renormalize;  /* 0 or 1 */
  int32_t n_groups;     /* 1 = no group limit; else divides E, <= 64 */
  int32_t topk_groups;  /* groups kept, 1..n_groups */
  int32_t group_topn;   /* 1..4, <= E/n_groups */
  float routed_scale;   /* multiplies every weight */
} moe_route_params;

/* ---------------------------------------------------------------------------
 * moe_route_topk - router logits and top-k routing of T tokens.
 * The step before dispatch in each microbatch ("[Core/DBO][1/N]", Purpose:
 * compute, then dispatch on the comm stream).
 *   x          [T, H] activations, dtype act (MOE_F32 or MOE_BF16)
 *   w_router   [E, H] router weights, dtype act
 *   logit_bias [E] fp32 added to every logit, or NULL
 *   forced_ids [T, k] int32 experts to use instead of the top-k selection
 *              (uniform-random routing simulation), or NULL.  Weights are
 *              then taken at these ids.  Ids outside [0, E) get weight 0.
 *   logits_out [T, E] fp32 logits = x W_r^T + bias (the values the
 *              selection compared), or NULL
 *   topk_ids   [T, k] int32 output; topk_w [T, k] fp32 output
 *   ws         moe_route_workspace_size(T, H, E) bytes (split-K partial logits)
 * T == 0 enqueues nothing and returns MOE_OK.  H must be a multiple of 128.
 * ------------------------------------------------------------------------- */
size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E);
moe_status moe_route_topk(const void* x, moe_dtype act, int64_t T, int32_t H,
                          const void* w_router, const float* logit_bias,
                          const int32_t* forced_ids, const moe_route_params* params,
                          float* logits_out, int32_t* topk_ids, float* topk_w,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_dispatch - counting-sort dispatch of T tokens' k (token, slot) pairs to
 * the local experts [expert_begin, expert_end), the single-GPU stand-in for
 * the all-to-all dispatch ("[Core/DBO][1/N]", Purpose; per-expert counts stay
 * on the device and capacity is worst case, "DeepEP HT: full decode CUDA
 * graphs via worst-token dispatch", bot review 2).
 * Pairs are numbered p = t*k + j.  Local pairs are sorted by expert, stable
 * in p; M = number of local pairs <= T*k.
 *   counts       [E_loc] int32 out: pairs per local expert
 *   offsets      [E_loc+1] int32 out: exclusive scan of counts (offsets[E_loc] = M)
 *   tile_offsets [E_loc+1] int32 out: exclusive scan of ceil(counts/tile_m),
 *                or NULL (then tile_m is ignored)
 *   perm         [T*k] int32 out: perm[pos] = p for pos < M (rest untouched)
 *   inv          [T*k] int32 out: inv[p] = pos, or -1 for a non-local pair
 *   x_perm       [T*k, H] out, dtype act: x_perm[pos] = x[perm[pos] / k]
 *   ws           workspace of moe_dispatch_workspace_size(T, k, E_loc) bytes
 * Ids outside [0, E_total) are not dispatched (inv = -1) and set the device
 * error word read by moe_get_device_error(ws).  E_loc <= 1024.
 * ------------------------------------------------------------------------- */
size_t moe_dispatch_workspace_size(int64_t T, int32_t k, int32_t E_loc);
moe_status moe_dispatch(const void* x, moe_dtype act, int64_t T, int32_t H,
                        const int32_t* topk_ids, int32_t k, int32_t E_total,
                        int32_t expert_begin, int32_t expert_end, int32_t tile_m,
                        int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                        int32_t* perm, int32_t* inv, void* x_perm,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_dispatch_noalloc - moe_dispatch without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * outputs and errors as moe_dispatch, less ws / ws_bytes: the workspace is a
 * library-owned device array of moe_dispatch_noalloc_max_workspace() bytes
 * (8 MiB) on each GPU, held until the process ends.  A call whose
 * moe_dispatch_workspace_size(T, k, E_loc) exceeds that returns
 * MOE_ERR_WORKSPACE and enqueues nothing.  The call allocates and frees
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (on different streams, or from several threads without
 * ordering) race and must not be issued.  Out-of-range ids are skipped as in
 * moe_dispatch; their device error word stays in the shared array and is not
 * reported (use moe_dispatch where it is needed).
 * ------------------------------------------------------------------------- */
size_t moe_dispatch_noalloc_max_workspace(void);
moe_status moe_dispatch_noalloc(const void* x, moe_dtype act, int64_t T, int32_t H,
                                const int32_t* topk_ids, int32_t k, int32_t E_total,
                                int32_t expert_begin, int32_t expert_end, int32_t tile_m,
                                int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                                int32_t* perm, int32_t* inv, void* x_perm, void* stream);

/* ---------------------------------------------------------------------------
 * fp8 activations: per-row quantisation in groups of 128 columns.
 * The pages name a fused SiLU-mul + fp8 quantisation op that feeds an fp8
 * GEMM ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", CI
 * discussion) and give no rule.  Reading: a group of 128 consecutive columns
 * of a row is stored as E4M3 (fn) codes plus one E8M0 byte b (scale 2^(b-127));
 * b - 127 is the smallest e >= -127 with max|group| <= 448 * 2^e, and each
 * code is the round-to-nearest-even E4M3 value of x * 2^-e (exact scaling, so
 * the codes depend only on the values).  Real value = code value * 2^(b-127).
 * Inputs must be finite.
 *
 * moe_quant_fp8_rows - quantise x [n, K] bf16 (K % 128 == 0, else
 *   MOE_ERR_UNSUPPORTED) into q [n, K] codes and scale [n, K/128] bytes.
 *
 * moe_dispatch_fp8 - moe_dispatch (same arguments and outputs, act = bf16)
 *   whose row gather quantises each token row once and writes its codes to
 *   xq_perm [T*k, H] and its bytes to xq_scale [T*k, H/128].  H % 128 == 0.
 * ------------------------------------------------------------------------- */
moe_status moe_quant_fp8_rows(const void* x, int64_t n, int32_t K, uint8_t* q, uint8_t* scale, void* stream);
moe_status moe_dispatch_fp8(const void* x, int64_t T, int32_t H, const int32_t* topk_ids, int32_t k,
                            int32_t E_total, int32_t expert_begin, int32_t expert_end, int32_t tile_m,
                            int32_t* counts, int32_t* offsets, int32_t* tile_offsets, int32_t* perm,
                            int32_t* inv, uint8_t* xq_perm, uint8_t* xq_scale, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------
 * moe_dispatch_send / moe_dispatch_recv - moe_dispatch in two phases, the
 * send / receive-hook split of a low-latency dispatch ("[Core/DBO][2/N]
 * Dual-Batch Overlap add DeepEP High Throughput support and Prefill support",
 * review of modular_kernel.py: the dispatch returns a hook that the receiver
 * runs later; under DBO after a yield).
 *   send: topk_ids -> counts, offsets, tile_offsets, perm, inv (as
 *         moe_dispatch; same workspace and device error word); no row moves.
 *   recv: x [T, H] act and the send's inv [T*k] -> x_perm rows
 *         (x_perm[inv[t*k+j]] = x[t] for inv >= 0).  xq_scale NULL: x_perm is
 *         in act; else (act bf16, H % 128 == 0) x_perm receives E4M3 codes and
 *         xq_scale [T*k, H/128] the E8M0 bytes, as moe_dispatch_fp8.
 * send then recv on one stream equals moe_dispatch (moe_dispatch_fp8) bit for
 * bit.
 * ------------------------------------------------------------------------- */
moe_status moe_dispatch_send(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E_total,
                             int32_t expert_begin, int32_t expert_end, int32_t tile_m, int32_t* counts,
                             int32_t* offsets, int32_t* tile_offsets, int32_t* perm, int32_t* inv,
                             void* ws, size_t ws_bytes, void* stream);
moe_status moe_dispatch_recv(const void* x, moe_dtype act, int64_t T, int32_t H, int32_t k,
                             const int32_t* inv, void* x_perm, uint8_t* xq_scale, void* stream);

/* Device error word of a dispatch workspace (0 = none, 1 = an expert id was
 * out of range).  Synchronises `stream` and copies 4 bytes: debug use only. */
moe_status moe_get_device_error(const void* dispatch_ws, int32_t* code, void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_ffn - per-local-expert SwiGLU FFN on dispatched rows
 * (the expert GEMM + act-and-mul of "[Core/DBO][1/N]", performance
 * discussion).  Reading: W13 stacks gate rows [0, I) over up rows [I, 2I);
 * h = silu(x G^T) * (x U^T) (rounded to act); y = h W2^T.
 *   x_perm   [cap_rows, H] act; rows [offsets[e], offsets[e+1]) use expert e
 *   offsets  [E_loc+1] int32 device offsets from moe_dispatch, or NULL for a
 *            dense call (E_loc must be 1; all cap_rows rows use expert 0: the
 *            shared-expert MLP)
 *   w13      [E_loc, 2I, H], w2 [E_loc, H, I] of dtype wdt:
 *            MOE_F32 (with act MOE_F32), MOE_BF16 or MOE_FP8_E4M3FN (act bf16)
 *   w13_scale [E_loc, 2I/128, H/128], w2_scale [E_loc, H/128, I/128] fp32:
 *            per-128x128-block scales for fp8 (real W = code value * scale);
 *            must be NULL otherwise
 *   y_perm   [cap_rows, H] out, act; rows >= offsets[E_loc] untouched
 *   tile_m   0 = automatic; 32, 64 or 128 rows per tile; any other value
 *            MOE_ERR_INVALID_ARG
 *   ws       moe_ffn_workspace_size(cap_rows, I, act) bytes (holds h)
 * H % 128 == 0 and I % 64 == 0 (fp8: I % 128 == 0), else MOE_ERR_UNSUPPORTED.
 * fp8 weights: the 64- and 128-row tiles of routed experts (no dense group,
 * K <= 64 scale blocks) convert the codes exactly and apply each block scale
 * to the fp32 sum over its 128-wide K block: with a block accumulator (one
 * fma per block), or, when the launch has about 128 rows per expert or more,
 * with one accumulator kept in units of the current block's scale (rescaled
 * at each block, one fp32 rounding per block).  That form needs the partial
 * sums divided by a block scale to stay within the fp32 range (nonzero scales
 * of one 128-row block within about 2^80 of each other); zero scales are
 * allowed and contribute nothing.  The 32-row tiles and launches with a dense
 * group expand code value x scale to bf16 (rounded once) before the MFMAs.
 * ------------------------------------------------------------------------- */
size_t moe_ffn_workspace_size(int64_t cap_rows, int32_t I, moe_dtype act);
/* The row tile the automatic choice (tile_m = 0) takes for experts of about
 * rows_per_expert rows (dbo_moe_layer passes ceil(T*k/E)); rows1/I1 describe
 * a dense group run in the same launches (the shared experts of
 * dbo_moe_layer: rows1 = microbatch tokens, I1 = shared_I), 0/0 if none.
 * Returns 32, 64 or 128, or 0 for shapes moe_grouped_ffn rejects.
 * Pure host function. */
int32_t moe_ffn_auto_tile(moe_dtype act, moe_dtype wdt, int32_t H, int32_t I, int64_t rows_per_expert,
                          int64_t rows1, int32_t I1);
moe_status moe_grouped_ffn(const void* x_perm, moe_dtype act, int32_t H, int32_t I,
                           const int32_t* offsets, int32_t E_loc, int64_t cap_rows,
                           const void* w13, const void* w2, moe_dtype wdt,
                           const float* w13_scale, const float* w2_scale,
                           void* y_perm, int32_t tile_m, void* ws, size_t ws_bytes,
                           void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_ffn_fp8 - moe_grouped_ffn with fp8 activations and fp8 weights:
 * the fp8 expert path fed by the fused SiLU-mul + fp8 quantisation op
 * ("[Core/DBO][1/N]", CI discussion).
 *   xq_perm [cap_rows, H] E4M3 codes, xq_scale [cap_rows, H/128] E8M0 bytes
 *            (moe_dispatch_fp8 / moe_quant_fp8_rows)
 *   w13 [E_loc, 2I, H], w2 [E_loc, H, I] E4M3 codes with the fp32 128x128
 *            block scales w13_scale / w2_scale (both required, positive)
 *   y_perm   [cap_rows, H] bf16 out
 *   tile_m   0 (automatic), 64 or 128 rows per tile; else MOE_ERR_UNSUPPORTED
 *   ws       moe_ffn_fp8_workspace_size(cap_rows, I) bytes: h codes
 *            [cap_rows, I] then (256-byte aligned) h bytes [cap_rows, I/128]
 * h = silu(gate) * up is computed in fp32 and quantised as above (groups of
 * 128 of its I columns) before the down projection.  fp8 x fp8 MFMAs with
 * fp32 accumulation; each 128-wide K block's product is scaled by its weight
 * block scale as it is accumulated.  H % 256 == 0 and I % 128 == 0, else
 * MOE_ERR_UNSUPPORTED.  Same offsets / E_loc / dense rules as moe_grouped_ffn.
 * ------------------------------------------------------------------------- */
size_t moe_ffn_fp8_workspace_size(int64_t cap_rows, int32_t I);
moe_status moe_grouped_ffn_fp8(const uint8_t* xq_perm, const uint8_t* xq_scale, int32_t H, int32_t I,
                               const int32_t* offsets, int32_t E_loc, int64_t cap_rows,
                               const uint8_t* w13, const uint8_t* w2, const float* w13_scale,
                               const float* w2_scale, void* y_perm, int32_t tile_m, void* ws,
                               size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine - weighted gather-reduce, the single-GPU stand-in for the
 * all-to-all combine ("[Core/DBO][1/N]", Purpose).
 *   out[t] = sum_{j: inv[t*k+j] >= 0} topk_w[t, j] * y_perm[inv[t*k+j]]
 *            (+ shared_out[t]), summed in j order in fp32, one rounding to act.
 *   Tokens with no local expert get 0 (+ shared_out).
 *   y_perm [*, H] act; inv [T*k] int32; topk_w [T, k] fp32;
 *   shared_out [T, H] act or NULL; out [T, H] act (must not alias y_perm).
 * ------------------------------------------------------------------------- */
moe_status moe_combine(const void* y_perm, moe_dtype act, int64_t T, int32_t H, int32_t k,
                       const int32_t* inv, const float* topk_w, const void* shared_out,
                       void* out, void* stream);

/* ---------------------------------------------------------------------------
 * dbo_moe_layer - the whole layer under Dual-Batch Overlap.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t H, I;                 /* hidden size; intermediate size per routed expert */
  moe_dtype act;                /* activations and router weights: MOE_F32 or MOE_BF16 */
  moe_dtype wdt;                /* routed expert weights (see moe_grouped_ffn) */
  moe_route_params route;
  int32_t expert_begin;         /* local experts [expert_begin, expert_end) */
  int32_t expert_end;
  const void* w_router;         /* [E, H] act */
  const void* w13;              /* [E_loc, 2I, H] wdt */
  const void* w2;               /* [E_loc, H, I] wdt */
  const float* w13_scale;       /* fp8 scales or NULL */
  const float* w2_scale;
  int32_t shared_I;             /* 0 = no shared expert.  Several always-on shared
                                   experts are passed as ONE expert whose gate, up and
                                   down matrices are their concatenations (the sum of
                                   SwiGLU experts equals one SwiGLU expert with the
                                   intermediate dims stacked) */
  const void* shared_w13;       /* [2*shared_I, H] act */
  const void* shared_w2;        /* [H, shared_I] act */
  int32_t fp8_act;              /* 0, or 1: the routed experts run with fp8 activations
                                   (needs act MOE_BF16, wdt MOE_FP8_E4M3FN, H % 256 == 0,
                                   I % 128 == 0): the dispatch writes rows as
                                   moe_dispatch_fp8 does and the FFN is
                                   moe_grouped_ffn_fp8 (row tiles 64 or 128: ffn_tile_m
                                   0, 64 or 128, else MOE_ERR_UNSUPPORTED).  The shared
                                   experts keep act. */
} moe_layer_desc;

typedef enum {
  DBO_SCHED_UNSPLIT = 0,        /* one microbatch of T rows, compute stream only */
  DBO_SCHED_SERIAL = 1,         /* microbatch A fully, then B, compute stream only */
  DBO_SCHED_DBO = 2,            /* interleaved on two streams, events recorded before
                                   each yield (the fixed behaviour) */
  DBO_SCHED_DBO_LATE_EVENT = 3, /* diagnostic: events recorded after the yield, so a
                                   microbatch's comm also waits for the other
                                   microbatch's compute (the behaviour the fix removed) */
  DBO_SCHED_DBO_RECV_HOOK = 4   /* DBO with the dispatch in two phases: send (count,
                                   scan, rank), then a receive hook (the row gather) run
                                   after one more yield, the low-latency dispatch structure
                                   ("[Core/DBO][2/N] Dual-Batch Overlap add DeepEP High
                                   Throughput support and Prefill support", review of
                                   modular_kernel.py).  Four yields per microbatch */
} dbo_schedule;

typedef struct {
  int32_t schedule;             /* dbo_schedule */
  int32_t min_tokens_to_split;  /* T below this runs UNSPLIT (>= 2) */
  int32_t split_at;             /* rows of microbatch A; -1 = ceil(T/2) */
  int32_t comm_cu_budget;       /* 0 = none; else at most this many workgroups per
                                   dispatch/combine kernel (grid-stride loops), leaving
                                   compute units to the overlapping FFN */
  int32_t ffn_tile_m;           /* 0 = automatic (see moe_grouped_ffn) */
} dbo_opts;

typedef struct dbo_ctx dbo_ctx;

/* Context: the per-microbatch events (one caller thread per context). */
moe_status dbo_ctx_create(dbo_ctx** ctx);
void dbo_ctx_destroy(dbo_ctx* ctx);
/* Optional kernel timing: while enabled, each dbo_moe_layer call brackets
 * each microbatch's two expert GEMM kernels with timing events on the compute
 * stream, and its dispatch and combine kernels on the stream they run on (the
 * context remembers the last 128 timed calls; the events are created by the
 * first enable). */
moe_status dbo_ctx_set_timing(dbo_ctx* ctx, int32_t enable);
/* Elapsed ms of the expert GEMM kernels of the timed call `back` calls ago
 * (0 = the last), ms4 = {A gate/up, A down, B gate/up, B down}; zeros for a
 * microbatch that did not run or a call not remembered.  Waits for the end
 * events of that call. */
moe_status dbo_ctx_ffn_times(dbo_ctx* ctx, int32_t back, float* ms4);
/* The same for the comm-side steps: ms4 = {A dispatch, B dispatch, A combine,
 * B combine} (each step's kernels from the first launch to the last). */
moe_status dbo_ctx_comm_times(dbo_ctx* ctx, int32_t back, float* ms4);
/* Schedule bookkeeping of the last call: stats[0..5] = {schedule run, T0,
 * yields A, yields B, stages launched, events recorded}.  DBO issues 3 yields
 * per microbatch, the receive-hook schedule 4. */
moe_status dbo_ctx_last_stats(dbo_ctx* ctx, int64_t* stats6);

/* Workspace of one call with up to T_max tokens: two disjoint halves, one per
 * microbatch (microbatches never share buffers). */
size_t moe_layer_workspace_size(const moe_layer_desc* desc, int64_t T_max);

/* Byte offsets, inside the layer workspace, of microbatch mb's (0 = A, 1 = B;
 * UNSPLIT uses 0) intermediate buffers, for inspection after a call:
 * off[0..11] = {logits, topk_ids, topk_w, counts, offsets, tile_offsets, perm,
 * inv, x_perm, y_perm, shared_out, dispatch_ws}. */
moe_status moe_layer_workspace_layout(const moe_layer_desc* desc, int64_t T_max, int32_t mb,
                                      int64_t* off12);

/* Runs the layer on x [T, H] (act) into out [T, H] (act).  forced_ids [T, k]
 * or NULL, logit_bias [E] fp32 or NULL, as in moe_route_topk.  Inputs must be
 * ready in order with `compute`; out is complete in order with `compute` when
 * the enqueued work ends (both microbatches' comm work is joined back).
 * T == 0 enqueues nothing.  On an error mid-schedule, issuing stops, the comm
 * work already issued is joined into `compute`, and the status is returned. */
moe_status dbo_moe_layer(dbo_ctx* ctx, const moe_layer_desc* desc, const void* x, int64_t T,
                         const int32_t* forced_ids, const float* logit_bias, void* out,
                         const dbo_opts* opts, void* ws, size_t ws_bytes,
                         void* compute_stream, void* comm_stream);

const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* DBOMOE_H */
