/*
 * moe.h -- C ABI of libmoe.so, the MI355X (gfx950) fused MoE forward.
 *
 * The path (pages cited by title, sections as printed on each page):
 *   [FMF8]  "Fused MoE FP8: 8.09 -> 13.18 TFLOPS (1.63x)" (Croqtile tutorial): pipeline
 *           overview, problem table, "Baseline: 7 kernels" items 1-7, Phase 1 fusions.
 *   [H200]  "H200 MoE Grouped GEMM: routed-row accounting, online replay and SM90 tuning":
 *           compact routed rows, gated-up and down projections (BF16 grouped GEMM).
 *   [WEAVE] repost blog on the "Weave" paper: persistent kernel pulling
 *           (expert, token_begin, token_num) tasks from an atomic counter (sections 2.2, 4.2,
 *           4.3).
 *
 *   route -> count + layout (+ task list) -> quantise + sort + gather -> grouped GEMM ->
 *   routing-weighted combine to BF16.
 *
 * Conventions that hold for every entry point:
 *   - Every pointer argument is DEVICE memory owned by the caller, except where a comment
 *     says "host".  The library never allocates, frees or synchronises inside these calls,
 *     with one opt-in exception: moe_forward_ex with MOE_FWD_GRAPH captures the step on a
 *     stream of its own (created on first use) and instantiates and caches a graph per
 *     argument set.  moe_forward and every other entry point launch plain kernels only.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL means the null stream) and is
 *     asynchronous; calls made under stream capture are recorded like any other launch.
 *   - Arrays are row-major, last index contiguous.  bf16 travels as uint16_t bit patterns;
 *     FP8 is OCP E4M3FN (bias 7, max 448, 0x7F/0xFF NaN) as uint8_t.
 *   - k (top-k) is at most 64 and at most E; E is at most 1024.
 *   - Argument checks run on the host before any HIP call.  Return values: MOE_OK, or a
 *     negative status; nothing is thrown across the ABI.  Invalid arguments launch nothing.
 *   - topk_ids produced by moe_route are always in [0, E).  Ids supplied by a caller that lie
 *     outside [0, E) are skipped by every later stage (that route contributes nothing).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_E_INVAL (-1)  /* bad sizes, null pointer, unsupported combination         */
#define MOE_E_NOSPC (-2)  /* caller-provided buffer (tasks, workspace) is too small    */
#define MOE_E_HIP (-3)    /* a HIP launch or runtime call failed                       */
#define MOE_E_DEVICE (-4) /* no HIP device, or the current device is not gfx950        */

typedef void* moe_stream_t; /* hipStream_t */

/* Words of a grouped-GEMM task-counter buffer (`queue` arguments): per-XCD tickets, an exit
 * count and an error word.  Zero before first use; every launch leaves it zeroed. */
#define MOE_QUEUE_WORDS 16
/* Word of moe_forward's part 7 (the task counters) that the two-kernel small-batch step
 * sets to 1 when a wave of its GEMM stopped waiting for a routing wave and routed tokens
 * itself (informational: the output is complete and the same either way).  It stays set
 * until the caller clears it or a step that builds a layout resets the counters. */
#define MOE_QUEUE_HANDOFF_STATUS 10

/* Task schedules of the LDS-tiled grouped GEMMs (BF16, and FP8 with chunks of 65..256 rows)
 * ([WEAVE] sections 1.2, 2.2, 3.1 and 4.2):
 *   MOE_SCHED_DISPATCH   one workgroup per task; the hardware dispatcher hands workgroups to
 *                        CUs as they free up (in order, round robin over the 8 XCDs)
 *   MOE_SCHED_STATIC     one workgroup per CU, each walking a fixed share of its XCD's
 *                        tasks (the static big kernel)
 *   MOE_SCHED_QUEUE      one workgroup per CU pulling tasks from one atomic counter
 *   MOE_SCHED_QUEUE_XCD  one workgroup per CU pulling from its XCD's own counter over that
 *                        XCD's run of tasks, then from the other XCDs' counters
 * The queue forms need a MOE_QUEUE_WORDS counter buffer.  MOE_SCHED_AUTO is hardware
 * dispatch: on every workload measured it was the fastest or within noise of the fastest. */
#define MOE_SCHED_AUTO (-1)
#define MOE_SCHED_DISPATCH 0
#define MOE_SCHED_STATIC 1
#define MOE_SCHED_QUEUE 2
#define MOE_SCHED_QUEUE_XCD 3

/* One unit of grouped-GEMM work ([WEAVE] section 4.2): rows [row_begin, row_begin+row_count)
 * of expert `expert`'s segment, times the weight panel n_block (n_tile output columns). */
typedef struct moe_task {
    int32_t expert;
    int32_t row_begin;
    int32_t row_count;
    int32_t n_block;
} moe_task;

/* Grouped GEMM operand types. */
#define MOE_GEMM_FP8_B128 0 /* E4M3 operands, 1x128 activation / 128x128 weight fp32 scales */
#define MOE_GEMM_BF16 1     /* bf16 operands, no scales                                     */

/* Grouped GEMM epilogues (what is written for sorted row r, output column n). */
#define MOE_EPI_STORE_F32 0   /* out f32 [rows][N]: out[r][n]                              */
#define MOE_EPI_STORE_BF16 1  /* out bf16 [rows][N]: bf16(out[r][n]), round to nearest even */
#define MOE_EPI_ROUTE_F32 2   /* out f32 [M*k][N]: out[sorted_route_ids[r]][n], i.e. each
                                 routed row lands at its route id t*k+j for the combine   */
#define MOE_EPI_SWIGLU_BF16 3 /* BF16 mode only; out bf16 [rows][N/2]:
                                 bf16(silu(h[r][c]) * h[r][N/2+c]) for c < N/2             */

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(int status);

/* MOE_OK when the current HIP device is a gfx950; MOE_E_DEVICE otherwise. */
int moe_device_check(void);

/* ---- [WEAVE] section 3.1 (the gate, counted in the layer's forward): router projection ---
 * x bf16 [M][H] (the layer's hidden states), w_gate bf16 [E][H] -> logits f32 [M][E]:
 *   logits[t][e] = sum_h x[t][h] * w_gate[e][h]   (bf16 products, fp32 accumulation)
 * the input of moe_route / moe_forward.  H a multiple of 64, 1 <= E <= 1024, M*H < 2^40 and
 * ceil(M/16)*ceil(E/16) < 2^31 (else MOE_E_INVAL).  The fp32 sum is taken in a fixed order
 * (repeat calls give the same bits).  One launch on `stream`. */
int moe_router_logits(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                      float* logits, moe_stream_t stream);

/* ---- [FMF8] Baseline item 1 (Route): softmax with softcapping (tanh), then top-k --------
 * logits f32 [M][E].  For each token: the k experts with the largest raw logit, ties to the
 * lower index (-0 equals +0), written to topk_ids [M][k] in descending order; their weights
 * topk_weights [M][k] = softmax over c_j = softcap*tanh(logit_j/softcap) of the k selected
 * experts (renormalised to sum 1).  softcap <= 0 disables the cap (c = logit).  Logits must
 * be finite. */
int moe_route(const float* logits, int M, int E, int k, float softcap, int32_t* topk_ids,
              float* topk_weights, moe_stream_t stream);

/* moe_route plus the blockwise E4M3 quantisation of every token's row of x, once per token
 * ([FMF8] Baseline item 4 with the moe_quant_sort_gather rule below, without the sort and
 * the k copies): x bf16 [M][K] -> x_q E4M3 [M][K] and x_scales f32 [K/128][M] (scale of
 * token t, block b at x_scales[b*M + t]).  K a multiple of 128.  moe_grouped_gemm_gather
 * reads the routed rows from these by token.  One launch. */
int moe_route_quantize(const float* logits, const uint16_t* x, int M, int E, int k, int K,
                       float softcap, int32_t* topk_ids, float* topk_weights, uint8_t* x_q,
                       float* x_scales, moe_stream_t stream);

/* ---- [FMF8] Baseline items 2-3 + Fusion 3 (count and build layout), [WEAVE] 4.3 ---------
 * Host only (no HIP call): capacity that `tasks` needs for moe_build_layout, i.e.
 * (floor(M*k/chunk_rows) + min(E, M*k)) * n_blocks.  Returns -1 on bad arguments. */
int moe_max_tasks(int M, int k, int E, int n_blocks, int chunk_rows);

/* topk_ids s32 [M][k] ->
 *   counts s32 [E]       routes per expert
 *   offsets s32 [E+1]    exclusive prefix sum; offsets[E] = number of valid routes (M*k)
 *   cursors s32 [E]      = offsets[0..E-1]; moe_quant_sort_gather advances them
 *   tasks [max_tasks]    each expert's rows cut into chunks of at most chunk_rows rows,
 *                        each chunk crossed with n_blocks weight panels; full chunks first,
 *                        then the partial ones by decreasing row count (largest first)
 *   ntasks s32 [1]       number of tasks written
 *   queue u32 [MOE_QUEUE_WORDS]  reset to zero (the grouped GEMMs' task counters)
 *   sorted_route_ids s32 [M*k]   optional (NULL: not written): the routes in expert order,
 *                        sorted_route_ids[slot] = r for slot in [offsets[e], offsets[e+1])
 *                        of e = topk_ids[r]; the order inside a segment is unspecified
 *   route_slots s32 [M*k]        optional (only with sorted_route_ids): the inverse, -1 for
 *                        ids outside [0, E)
 * chunk_rows in [1, 1024]; max_tasks must be >= moe_max_tasks(...) (else MOE_E_NOSPC).
 * One workgroup of 1024 threads; the order of tasks with equal row counts is unspecified.
 * With sorted_route_ids set, do not also run moe_quant_sort_gather on the same cursors'
 * segments expecting the same slots (it takes its own). */
int moe_build_layout(const int32_t* topk_ids, int M, int k, int E, int n_blocks,
                     int chunk_rows, int32_t* counts, int32_t* offsets, int32_t* cursors,
                     moe_task* tasks, int max_tasks, int32_t* ntasks, uint32_t* queue,
                     int32_t* sorted_route_ids, int32_t* route_slots, moe_stream_t stream);

/* ---- [FMF8] Baseline items 4-5 + Fusion 2 (QSG: quantise, sort, gather) ------------------
 * x bf16 [M][K], K a multiple of 128.  Per token and 128-wide block b:
 *   amax = max|x|, scale = amax/448 (fp32, correctly rounded), inv = 1/scale (fp32,
 *   correctly rounded), code = E4M3(x*inv) rounded to nearest even, |y| >= 448 saturating to
 *   0x7E|sign, zeros keeping their sign; an all-zero block gets scale 0 and sign-only codes.
 * Each valid route r = t*k+j takes slot = atomicAdd(cursors[topk_ids[r]], 1) and writes
 *   sorted_route_ids[slot] = r, a_q[slot][0..K) = codes of token t,
 *   a_scales[b][slot] = scale of token t, block b   (a_scales is [K/128][M*k]),
 *   and, when route_slots [M*k] is not NULL, route_slots[r] = slot (-1 for an invalid id).
 * The order of routes inside one expert segment depends on atomic arrival order. */
int moe_quant_sort_gather(const uint16_t* x, int M, int K, const int32_t* topk_ids, int k,
                          int E, int32_t* cursors, int32_t* sorted_route_ids,
                          int32_t* route_slots, uint8_t* a_q, float* a_scales,
                          moe_stream_t stream);

/* ---- [WEAVE] Mixtral-like layer: sort + gather of bf16 rows (no quantisation) ---------
 * x bf16 [M][K] (K a multiple of 8).  Slots as in moe_quant_sort_gather: route r = t*k+j
 * with a valid id takes slot = atomicAdd(cursors[e], 1); sorted_route_ids[slot] = r,
 * route_slots[r] = slot (route_slots may be NULL; invalid ids get -1 and no row), and
 * a[slot][:] = x[t][:] (bf16 [M*k][K]).  Rows inside a segment come in arrival order. */
int moe_sort_gather_bf16(const uint16_t* x, int M, int K, const int32_t* topk_ids, int k,
                         int E, int32_t* cursors, int32_t* sorted_route_ids,
                         int32_t* route_slots, uint16_t* a, moe_stream_t stream);

/* ---- [FMF8] problem table (128x128 blockwise weights): weight preparation ---------------
 * w f32 [E][N][K] -> w_q E4M3 [E][N][K] and w_scales f32 [E][N/128][K/128], with the
 * activation rule above applied to every 128x128 block.  N, K multiples of 128. */
int moe_quantize_weights(const float* w, int E, int N, int K, uint8_t* w_q, float* w_scales,
                         moe_stream_t stream);

/* ---- [FMF8] Baseline item 6 (grouped GEMM) + [WEAVE] persistent atomic task queue -------
 * Output column tile of one task, per operand mode: 128 for MOE_GEMM_FP8_B128, 256 for
 * MOE_GEMM_BF16 (with MOE_EPI_SWIGLU_BF16 a task's 256 weight rows are 128 gate rows and
 * their 128 up rows, giving 128 output columns).  -1 for an unknown mode. */
int moe_gemm_n_tile(int mode);

/* For every task (e, r0, nr, nb) in tasks[0..*ntasks) and every row r in [r0, r0+nr),
 * column n in the task's panel [nb*n_tile, (nb+1)*n_tile):
 *   FP8_B128:  h[r][n] = sum_b a_scales[b][r] * w_scales[e][n/128][b] *
 *                        sum_{k in block b} e4m3(a[r][k]) * e4m3(w[e][n][k])   (fp32 accum)
 *   BF16:      h[r][n] = sum_k a[r][k] * w[e][n][k]                           (fp32 accum)
 * and the epilogue writes h (see MOE_EPI_*).  a is [rows][K] (u8 or bf16); w is [E][N][K].
 * a_scales/w_scales are ignored in BF16 mode.  sorted_route_ids [rows] is read only by
 * MOE_EPI_ROUTE_F32 (may be NULL otherwise).
 * BF16 mode ([H200] gated-up and down projections; [WEAVE] Mixtral-like layer): K a multiple
 * of 64, N a multiple of 256, chunk_rows <= 256; epilogues STORE_F32, STORE_BF16 and
 * SWIGLU_BF16, which writes out [rows][N/2] bf16 = bf16(silu(h[:, c]) * h[:, N/2 + c]) for
 * the task's 128 columns c (weight rows [0, N/2) are the gate, [N/2, N) the up projection).
 * One 256 x 256 output tile per task; `sched` (MOE_SCHED_*) picks how tiles reach
 * workgroups, the queue forms counting in queue (MOE_QUEUE_WORDS words, left zeroed).
 * Scheduling (FP8_B128): for chunk_rows <= 16 and K = 512, 1024 or 2048 the task list is
 * cut into one contiguous range of 16-column subtasks per workgroup, balanced inside the
 * workgroup by an LDS counter; queue is not used.  For chunk_rows in [65, 256] (K <= 8192) one workgroup
 * runs one task with both operands staged in LDS (grid = max_tasks rounded up to whole
 * chunks per XCD; workgroups past *ntasks exit at once; the panels of one chunk run on one
 * XCD); queue is not used.  Otherwise, with queue != NULL, a persistent grid pulls
 * task indices from queue[0] with atomics and the last workgroup to leave resets
 * queue[0..1] to zero, so the call can be repeated or graph-replayed; with queue == NULL
 * the same grid walks the task list with a fixed stride.  Tasks must come from
 * moe_build_layout for the same rows, E, n_tile and chunk_rows (FP8_B128: chunk_rows <= 256):
 * all n_blocks panels of one chunk consecutive.  Each task streams its expert's weight panel
 * once.  FP8_B128 takes sched = MOE_SCHED_AUTO only (its walk follows queue as above). */
int moe_grouped_gemm(int mode, const void* a, const float* a_scales, int rows, int K,
                     const void* w, const float* w_scales, int E, int N,
                     const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                     int chunk_rows, uint32_t* queue, int epilogue,
                     const int32_t* sorted_route_ids, void* out, int sched,
                     moe_stream_t stream);

/* ---- [FMF8] Baseline items 5-6 with the gather done on load ------------------------------
 * The grouped FP8 GEMM of moe_grouped_gemm (FP8_B128, MOE_EPI_ROUTE_F32) for chunk_rows in
 * [65, 256] and K <= 8192, reading sorted row r from token sorted_route_ids[r] / k of the
 * token-major codes x_q [M][K] and scales x_scales [K/128][M] (moe_route_quantize) instead
 * of from a sorted copy:
 *   rows[r_id][n] = sum_b x_scales[b][t] * w_scales[e][n/128][b] *
 *                   sum_{kk in block b} e4m3(x_q[t][kk]) * e4m3(w[e][n][kk]),
 * for every route r_id = sorted_route_ids[r] of a task's rows (t = r_id / k, e its expert),
 * rows f32 [M*k][N].  tasks from moe_build_layout (n_tile 128, the same chunk_rows) with its
 * sorted_route_ids.  An item is one chunk against two adjacent panels; `sched` (a
 * MOE_SCHED_* value) picks how items reach workgroups, the queue forms counting in `queue`
 * (MOE_QUEUE_WORDS words, zero before the first call, left zeroed; NULL is allowed for
 * MOE_SCHED_DISPATCH and MOE_SCHED_STATIC). */
/* ---- [FMF8] Baseline items 1-6 fused: the route inside the small-batch grouped GEMM ------
 * moe_route and moe_grouped_gemm_routed in one launch (the first kernel of moe_forward's
 * two-kernel step): logits f32 [M][E], x bf16 [M][K] -> topk_ids i32 and topk_weights f32
 * [M][k] (as moe_route writes them) and rows f32 [M*k][N] at route ids (as
 * moe_grouped_gemm_routed writes them).  Token t is routed by one wave of workgroup t % CUs,
 * which publishes each route in route_words [M*k] (caller-owned scratch, any content at the
 * call: a word left by an earlier call carries an older tag) as a tagged word; every
 * workgroup polls the words it reads, and a wave still missing words after a bounded number
 * of polls routes those tokens itself and sets *status to 1 (informational; the results are
 * the same).  The words are left tagged.  The tag changes with every call made through this
 * function, but a launch captured in a HIP graph replays with the tag it was captured with:
 * zero route_words between replays (moe_forward's combine does this for its own words).
 * Limits: those of moe_grouped_gemm_routed, and E <= 256, M at most 8 per CU, k <= 64;
 * MOE_E_INVAL otherwise. */
int moe_route_grouped_gemm(const float* logits, const uint16_t* x, int M, int E, int k, int K,
                           float softcap, const uint8_t* w_q, const float* w_scales, int N,
                           int32_t* topk_ids, float* topk_weights, uint32_t* route_words,
                           uint32_t* status, float* rows, moe_stream_t stream);

int moe_grouped_gemm_gather(const uint8_t* x_q, const float* x_scales, int M, int k, int K,
                            const uint8_t* w, const float* w_scales, int E, int N,
                            const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                            int chunk_rows, const int32_t* sorted_route_ids, float* rows,
                            uint32_t* queue, int sched, moe_stream_t stream);

/* ---- [FMF8] Baseline items 2-6 fused: grouped FP8 GEMM straight from routed ids ------------
 * The small-batch GEMM of moe_forward: K = 256, 512, 1024 or 2048, M*k <= 2048, N a multiple
 * of 128, and E at
 * most about three times the CU count (one CU's share of the E*N/16 weight slices may touch at
 * most four experts).  The weights are split evenly over one workgroup per CU, independent of
 * the routing; each workgroup finds its experts' routes in topk_ids [M][k] (ascending route
 * id), quantises those rows of x bf16 [M][K] with the moe_quant_sort_gather rule straight into
 * its MFMA tiles, and streams each of its weight slices once per 64 routed rows of the expert.
 * Writes rows f32 [M*k][N] at route ids (rows[t*k+j] = the GEMM row of route (t, j); rows of
 * invalid ids are not written).  counts [E] and offsets [E+1] are optional (both NULL or
 * both set): when set, a second small kernel writes them as moe_build_layout would.
 * w_q / w_scales as for moe_grouped_gemm.  MOE_E_INVAL outside the limits above. */
int moe_grouped_gemm_routed(const uint16_t* x, const int32_t* topk_ids, int M, int k, int E,
                            int K, const uint8_t* w_q, const float* w_scales, int N,
                            float* rows, int32_t* counts, int32_t* offsets,
                            moe_stream_t stream);

/* ---- [FMF8] Baseline item 7 (scatter, routing-weighted) ---------------------------------
 * rows f32 [M*k][N] are the GEMM rows.  Route r = t*k+j reads row route_slots[r] (rows in
 * sorted order, MOE_EPI_STORE_F32 + the slots recorded by moe_quant_sort_gather), or row r
 * itself when route_slots is NULL (MOE_EPI_ROUTE_F32).
 *   out[t][n] = bf16( sum_{j: topk_ids[t][j] valid} topk_weights[t][j] * row(t*k+j)[n] )
 * summed in fp32 in j order and rounded to nearest even once.  N a multiple of 4. */
int moe_scatter(const float* rows, const int32_t* route_slots, const float* topk_weights,
                const int32_t* topk_ids, int M, int k, int E, int N, uint16_t* out,
                moe_stream_t stream);

/* ---- whole step: route -> layout -> QSG -> FP8 grouped GEMM -> combine -------------------
 * Workspace (device, caller-owned) of at least moe_forward_workspace_bytes(...) bytes. */
size_t moe_forward_workspace_bytes(int M, int E, int k, int K, int N);

/* Byte offset inside the workspace of one intermediate, for inspection in tests:
 * 0 topk_ids, 1 topk_weights, 2 counts, 3 offsets, 4 cursors, 5 tasks, 6 ntasks, 7 queue,
 * 8 sorted_route_ids, 9 a_q, 10 a_scales, 11 GEMM rows (at route ids), 12 route_slots,
 * 13 x_q (token-major codes), 14 x_scales.  -1 on bad arguments. */
int64_t moe_forward_workspace_offset(int M, int E, int k, int K, int N, int which);

/* logits f32 [M][E], x bf16 [M][K], w_q E4M3 [E][N][K], w_scales f32 [E][N/128][K/128]
 * -> out bf16 [M][N].  K, N multiples of 128.
 * The five stages are enqueued on `stream` as plain kernel launches, with no host
 * synchronisation (moe_forward_ex can replay a cached HIP graph instead). */
int moe_forward(const float* logits, const uint16_t* x, const uint8_t* w_q,
                const float* w_scales, int M, int E, int k, int K, int N, float softcap,
                uint16_t* out, void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* moe_forward with explicit options: chunk_rows (0 = 16 while M*k/E <= 16, else 128 for
 * K <= 8192 or 64), flags bit 0 = replay
 * a HIP graph captured once per (shape, softcap, pointers, options) instead of launching the
 * kernels (ignored while the caller's stream is being captured), bit 1 = fixed-stride task
 * walk instead of the atomic queue (grouped GEMM forms that walk a queue). */
#define MOE_FWD_GRAPH 1
#define MOE_FWD_STATIC_GRID 2
/* bit 2: always run the five staged kernels (route, layout, moe_quant_sort_gather, grouped
 * GEMM, combine).  Without it:
 *  - a small batch (the limits of moe_grouped_gemm_routed, chunk_rows 16) runs the grouped
 *    GEMM straight from the routed ids (layout, sort/gather and quantisation inside it; fp32
 *    rows at route ids) and the combine, with the route inside that GEMM where E <= 256 and
 *    M <= 8 per CU (two kernels, see bit 7), else as a kernel of its own before it (three);
 *    the workspace then holds topk_ids, topk_weights and the GEMM rows (parts 0, 1 and 11),
 *    and on the two-kernel path the route words in part 12;
 *  - chunk_rows in [65, 256] (K <= 8192) runs four: moe_route_quantize, the layout with the
 *    sorted route ids over many workgroups (one launch; each segment in ascending route id),
 *    the moe_grouped_gemm_gather GEMM and the combine; the workspace then holds no a_q,
 *    a_scales or route_slots (parts 9, 10, 12) but the token-major x_q and x_scales (13,
 *    14). */
#define MOE_FWD_STAGED 4
/* bits 3-5: the task schedule of the tiled gathering GEMM, MOE_FWD_SCHED(MOE_SCHED_...);
 * 0 picks the default.  The queue forms use workspace part 7 as their counters. */
#define MOE_FWD_SCHED(s) (((s) + 1) << 3)
#define MOE_FWD_SCHED_MASK (7 << 3)
/* bit 6: the combine as the pages' scatter-add ([FMF8] Fusion 1): the gathering GEMM adds
 * w_tj * h of every routed row into fp32 token rows [M][N] (part 11, zeroed by the route
 * kernel) with float atomics, and a last kernel rounds them to bf16.  The fp32 sums then
 * follow atomic arrival order, so repeat calls may differ in the last bf16 bit.  Valid only on
 * the gathering path (chunk_rows in [65, 256], K <= 8192, not STAGED) with hardware
 * dispatch. */
#define MOE_FWD_ATOMIC_COMBINE 64
/* The small-batch path with E <= 256 and at most 8 tokens per CU runs two kernels by
 * default: the route moves into the grouped GEMM ([FMF8] "Baseline: 7 kernels" item 1 fused
 * with items 2-6).  Token t is routed by one wave of workgroup t % CUs, which writes topk_ids
 * and topk_weights and publishes each route as a word tagged for this call in part 12
 * (route_slots, unused on this path).  Every workgroup polls the route words it reads; a
 * wave whose words are still missing after a bounded number of polls routes those tokens
 * itself (see MOE_QUEUE_HANDOFF_STATUS), so the result never depends on another workgroup
 * being resident.  The combine clears the words.  Same results as three kernels.
 * bit 7: run the route as a kernel of its own instead (three kernels).
 * bit 8: on the two-kernel path, route without the handoff: every wave routes the tokens it
 * reads itself (the late-routing-wave fallback on every wave; slower, for tests). */
#define MOE_FWD_ROUTE_KERNEL 128
#define MOE_FWD_ROUTE_SELF 256
int moe_forward_ex(const float* logits, const uint16_t* x, const uint8_t* w_q,
                   const float* w_scales, int M, int E, int k, int K, int N, float softcap,
                   uint16_t* out, void* workspace, size_t workspace_bytes, int chunk_rows,
                   int flags, moe_stream_t stream);

/* Number of kernels moe_forward_ex launches for these arguments: 2 (small batch, route
 * inside the GEMM), 3 (small batch with the route as a kernel), 4 (the gathering path) or 5
 * (the staged one);
 * MOE_E_INVAL for arguments moe_forward_ex rejects. */
int moe_forward_kernels(int M, int E, int k, int K, int N, int chunk_rows, int flags);

/* ---- the whole step for callers that cannot allocate ----------------------------------
 * For code that may not call hipMalloc or take a workspace from an allocator (HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  moe_forward with the
 * library's own scratch in place of the caller's workspace: a 16 MiB device array that each
 * GPU the library runs on holds from its first use until the process ends, enough for every
 * shape whose moe_forward_workspace_bytes(...) is at most 16 MiB (the M=128, E=256, top-8,
 * K=2048, N=512 layer needs 4.4 MiB).  Larger shapes return MOE_E_NOSPC and launch nothing.
 * Same kernels, same default options and same results as moe_forward; plain launches on
 * `stream`, no allocation, no host synchronisation.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU (other streams, other threads) race, so a
 * caller serialises them on one stream.  Each call clears what it needs cleared itself. */
int moe_forward_noalloc(const float* logits, const uint16_t* x, const uint8_t* w_q,
                        const float* w_scales, int M, int E, int k, int K, int N, float softcap,
                        uint16_t* out, moe_stream_t stream);

/* ---- [WEAVE] / [H200] Mixtral-like expert FFN layer, BF16 --------------------------------
 * route (softcap, top-k) -> layout over many workgroups (chunk_rows rows per task, 0 = 256;
 * sorted route ids, route -> slot, both task lists) -> gated-up grouped GEMM reading each
 * routed row straight from x (gathered on load) with the SwiGLU epilogue -> down grouped GEMM
 * (fp32 rows) -> routing-weighted combine:
 *   act[r] = bf16(silu(x[t] . w_up[e][0:F]^T) * (x[t] . w_up[e][F:2F]^T)),
 *   y[t] = bf16( sum_j w_tj * act[r_j] . w_down[e_j]^T )      (fp32 accumulation)
 * logits f32 [M][E], x bf16 [M][H], w_up bf16 [E][2F][H] (gate rows then up rows),
 * w_down bf16 [E][H][F] -> out bf16 [M][H].  H a multiple of 256, F of 128.  Workspace of
 * moe_ffn_workspace_bytes(...) bytes; parts (for inspection): 0 topk_ids, 1 topk_weights,
 * 2 counts, 3 offsets, 4 cursors, 5 up tasks, 6 down tasks, 7 ntasks, 8 sorted_route_ids,
 * 9 route_slots, 10 act, 11 down rows, 12 task counters (MOE_QUEUE_WORDS per GEMM).  Five
 * plain launches on `stream`, no host
 * synchronisation.  flags: only MOE_FWD_SCHED(...) bits, the schedule of both BF16 GEMMs
 * (0: the default). */
size_t moe_ffn_workspace_bytes(int M, int E, int k, int H, int F);
int64_t moe_ffn_workspace_offset(int M, int E, int k, int H, int F, int which);
int moe_ffn_forward(const float* logits, const uint16_t* x, const uint16_t* w_up,
                    const uint16_t* w_down, int M, int E, int k, int H, int F, float softcap,
                    uint16_t* out, void* workspace, size_t workspace_bytes, int chunk_rows,
                    int flags, moe_stream_t stream);

/* ---- [FMF8] comparison section, "vLLM full MLP" reference, in FP8 ----------------------
 * The activation step of the expert MLP: for each of `rows` rows of h f32 [rows][2I] (gate
 * columns 0..I-1, up columns I..2I-1; device memory), act = silu(g) * u in fp32 with
 * silu(g) = g / (1 + e^-g), then the QSG quantiser per 128 columns (scale = amax/448, code =
 * e4m3(act * (1/scale)), an all-zero block gets scale 0) into a_q E4M3 [rows][I] and
 * a_scales f32 [I/128][rows] (transposed, as moe_quant_sort_gather writes them).  I a
 * positive multiple of 128.  One launch on `stream`. */
int moe_swiglu_quant(const float* h, int rows, int I, uint8_t* a_q, float* a_scales,
                     moe_stream_t stream);

/* The whole expert MLP layer in FP8:
 *   route (softcap, top-k) -> layouts of both GEMMs -> x quantised, sorted and gathered
 *   (moe_quant_sort_gather) -> gate+up grouped FP8 GEMM (fp32 rows, sorted order) ->
 *   moe_swiglu_quant -> down grouped FP8 GEMM (fp32 rows at route ids) -> routing-weighted
 *   combine:
 *   h1 = x_q[t] (*) w1[e]  (block-scaled, [2I] per route),  act_q = quant(silu(g) * u),
 *   y[t] = bf16( sum_j w_tj * act_q[r_j] (*) w2[e_j] )
 * logits f32 [M][E], x bf16 [M][H], w1_q E4M3 [E][2I][H] with w1_scales f32
 * [E][2I/128][H/128] (gate rows then up rows), w2_q E4M3 [E][H][I] with w2_scales f32
 * [E][H/128][I/128] -> out bf16 [M][H].  H and I positive multiples of 128; chunk_rows as in
 * moe_forward_ex (0 picks it from the batch).  Workspace of moe_mlp_workspace_bytes(...)
 * bytes; parts (for inspection): 0 topk_ids, 1 topk_weights, 2 counts, 3 offsets, 4 cursors,
 * 5 gate+up tasks, 6 down tasks, 7 ntasks (gate+up, down) at +0 and the two GEMMs' task
 * counters (MOE_QUEUE_WORDS each) at +64,
 * 8 sorted_route_ids, 9 route_slots, 10 x codes (sorted), 11 x scales, 12 gate+up rows f32
 * [M*k][2I], 13 act codes [M*k][I], 14 act scales [I/128][M*k], 15 down rows f32 [M*k][H]
 * at route ids.  Seven plain launches on `stream` (one layout pass writes both task lists),
 * no host synchronisation.  Small batches (the small-batch FP8 GEMM of moe_grouped_gemm_routed
 * applies to both projections: H and I in {256, 512, 1024, 2048}, chunk_rows 16) take three:
 * the gate+up GEMM from the routed ids with the route inside it (as moe_route_grouped_gemm;
 * route words in part 9, its status word at word MOE_QUEUE_HANDOFF_STATUS of the first task
 * counters in part 7; a separate route kernel first where E > 256 or M is above 8 per CU:
 * four) with rows at route ids in part 12 -> the down GEMM from the same ids, forming
 * silu(g) * u of each of its rows from part 12 and requantising it per 128 columns in its
 * tile build as moe_swiglu_quant would (those codes and scales also land in parts 13-14, in
 * route order) -> combine.  That path writes no counts, offsets, tasks or sorted ids (parts
 * 2-8 and 10-11 unused). */
size_t moe_mlp_workspace_bytes(int M, int E, int k, int H, int I);
/* Number of kernels moe_mlp_forward launches for these arguments (3, 4 or 7); MOE_E_INVAL for
 * arguments it rejects, MOE_E_DEVICE without a gfx950 device. */
int moe_mlp_forward_kernels(int M, int E, int k, int H, int I, int chunk_rows);
int64_t moe_mlp_workspace_offset(int M, int E, int k, int H, int I, int which);
int moe_mlp_forward(const float* logits, const uint16_t* x, const uint8_t* w1_q,
                    const float* w1_scales, const uint8_t* w2_q, const float* w2_scales, int M,
                    int E, int k, int H, int I, float softcap, uint16_t* out, void* workspace,
                    size_t workspace_bytes, int chunk_rows, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
