// moe_internal.h -- host-side launchers of the gfx950 kernels (arguments already checked by
// the C ABI layer in api.hip).  Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Device facts the launchers size grids with (cached per device by api.hip).
struct DeviceInfo {
    int cu_count;
};
const DeviceInfo& device_info();

// logits f32 [M][E] = x bf16 [M][H] . w_gate bf16 [E][H]^T (H a multiple of 64)
hipError_t launch_router_logits(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                                float* logits, hipStream_t s);

hipError_t launch_route(const float* logits, int M, int E, int k, float softcap,
                        int32_t* ids, float* weights, hipStream_t s);

// route + per-token quantisation of x (token-major codes [M][K], scales [K/128][M]); with
// acc != nullptr also zeroes the fp32 accumulator rows acc [M][acc_n] (acc_n % 4 == 0)
hipError_t launch_route_quantize(const float* logits, const uint16_t* x, int M, int E, int k,
                                 int K, float softcap, int32_t* ids, float* weights,
                                 uint8_t* x_q, float* x_scales, hipStream_t s,
                                 float* acc = nullptr, int acc_n = 0);

// the layout with the sorted route ids (ascending route id inside each segment) over many
// workgroups, one launch, E <= 1024; optionally route -> slot and a second task list over the
// same chunks (n_blocks2 panels)
hipError_t launch_layout_sorted_wide(const int32_t* ids, int M, int k, int E, int n_blocks,
                                     int chunk_rows, int32_t* counts, int32_t* offsets,
                                     int32_t* cursors, moe_task* tasks, int32_t* ntasks,
                                     uint32_t* queue, int32_t* sorted_route_ids,
                                     hipStream_t s, int32_t* route_slots = nullptr,
                                     int n_blocks2 = 0, moe_task* tasks2 = nullptr,
                                     int32_t* ntasks2 = nullptr, uint32_t* queue2 = nullptr);

// sorted_route_ids / route_slots may be null (then the routes are not sorted)
hipError_t launch_layout(const int32_t* ids, int M, int k, int E, int n_blocks, int chunk_rows,
                         int32_t* counts, int32_t* offsets, int32_t* cursors, moe_task* tasks,
                         int max_tasks, int32_t* ntasks, uint32_t* queue,
                         int32_t* sorted_route_ids, int32_t* route_slots, hipStream_t s);

// one layout pass writing two task lists over the same chunks (n_blocks and n_blocks2 panels)
hipError_t launch_layout2(const int32_t* ids, int M, int k, int E, int chunk_rows,
                          int32_t* counts, int32_t* offsets, int32_t* cursors, int n_blocks,
                          moe_task* tasks, int32_t* ntasks, uint32_t* queue, int n_blocks2,
                          moe_task* tasks2, int32_t* ntasks2, uint32_t* queue2, hipStream_t s);

hipError_t launch_qsg(const uint16_t* x, int M, int K, const int32_t* ids, int k, int E,
                      int32_t* cursors, int32_t* sorted_route_ids, int32_t* route_slots,
                      uint8_t* a_q, float* a_scales, hipStream_t s);

// bf16 sort/gather (K a multiple of 8)
hipError_t launch_gather_bf16(const uint16_t* x, int M, int K, const int32_t* ids, int k, int E,
                              int32_t* cursors, int32_t* sorted_route_ids,
                              int32_t* route_slots, uint16_t* a, hipStream_t s);

hipError_t launch_quantize_weights(const float* w, int E, int N, int K, uint8_t* w_q,
                                   float* w_scales, hipStream_t s);

hipError_t launch_gemm_fp8(const uint8_t* a, const float* a_scales, int rows, int K,
                           const uint8_t* w, const float* w_scales, int E, int N,
                           const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                           int chunk_rows, uint32_t* queue, int epilogue,
                           const int32_t* sorted_route_ids, void* out, hipStream_t s);

// contiguous-range form for tasks of at most 16 routed rows and K = 2048
bool gemm_fp8_range_applies(int K, int chunk_rows);
hipError_t launch_gemm_fp8_range(const uint8_t* a, const float* a_scales, int rows, int K,
                                 const uint8_t* w, const float* w_scales, int N,
                                 const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                                 int epilogue, const int32_t* sorted, void* out, hipStream_t s);

// tiled form for chunks of 65..256 routed rows (both operands staged in LDS)
bool gemm_fp8_tile_applies(int K, int chunk_rows);
hipError_t launch_gemm_fp8_tile(const uint8_t* a, const float* a_scales, int rows, int K,
                                const uint8_t* w, const float* w_scales, int N,
                                const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                                int chunk_rows, int epilogue, const int32_t* sorted, void* out,
                                hipStream_t s);
// the same with sorted row r read from token sorted[r] / k of x_q [M][K] (scales [K/128][M]);
// fp32 rows written at route ids
// (sched: MOE_SCHED_DISPATCH / STATIC / QUEUE / QUEUE_XCD; the queue forms use `queue`,
// MOE_QUEUE_WORDS zeroed words, which they leave zeroed)
hipError_t launch_gemm_fp8_tile_gather(const uint8_t* x_q, const float* x_scales, int M, int k,
                                       int K, const uint8_t* w, const float* w_scales, int N,
                                       const moe_task* tasks, const int32_t* ntasks,
                                       int max_tasks, int chunk_rows, const int32_t* sorted,
                                       float* rows_out, int sched, uint32_t* queue,
                                       hipStream_t s);
// the same GEMM with the scatter-add epilogue of the pages: every routed row h is added as
// w[r] * h into acc [M][N] (fp32 atomics; acc zeroed beforehand), hardware dispatch
hipError_t launch_gemm_fp8_tile_gather_atomic(const uint8_t* x_q, const float* x_scales, int M,
                                              int k, int K, const uint8_t* w,
                                              const float* w_scales, int N,
                                              const moe_task* tasks, const int32_t* ntasks,
                                              int max_tasks, int chunk_rows,
                                              const int32_t* sorted, const float* weights,
                                              float* acc, hipStream_t s);
// out bf16 [M][N] = bf16(acc) (round to nearest even)
hipError_t launch_acc_to_bf16(const float* acc, int M, int N, uint16_t* out, hipStream_t s);

// small-batch forward GEMM with the layout, sort/gather and quantisation folded in: weight
// slices split evenly over one workgroup per CU, fp32 rows at route ids ([M*k][N])
bool forward_fused_applies(int M, int k, int E, int K, int N, int chunk_rows);
hipError_t launch_gemm_fp8_fused(const uint16_t* x, const int32_t* ids, int M, int k, int E,
                                 int K, const uint8_t* w, const float* w_scales, int N,
                                 float* rows_out, hipStream_t s);
// The same GEMM as the FP8 MLP's down projection: the A rows are silu(g) * u of the fp32
// gate+up rows h [M*k][2K] at route ids, requantised per 128 columns in the tile build (as
// moe_swiglu_quant would); those codes [M*k][K] and scales [K/128][M*k] also go to a_q / a_s
// when a_q is set.  rows_out [M*k][N] at route ids.
hipError_t launch_gemm_fp8_fused_act(const float* h, const int32_t* ids, int M, int k, int E,
                                     int K, const uint8_t* w, const float* w_scales, int N,
                                     float* rows_out, uint8_t* a_q, float* a_s, hipStream_t s);
// The same GEMM with the route inside (moe_route folded in): writes ids and weights, hands
// the routes over through tagged words handoff [M*k] (untagged at launch; cleared by the
// combine) and sets *status to 1 if a workgroup's wait gave up.  Applies where
// fused_route_applies also holds.
bool fused_route_applies(int M, int k, int E);
hipError_t launch_gemm_fp8_fused_route(const float* logits, const uint16_t* x, int M, int k,
                                       int E, int K, float softcap, const uint8_t* w,
                                       const float* w_scales, int N, int32_t* ids,
                                       float* weights, uint32_t* handoff, uint32_t* status,
                                       float* rows_out, bool self_route, hipStream_t s);

// per-expert counts [E] and exclusive offsets [E+1] of the routed ids (E <= 1024)
hipError_t launch_counts(const int32_t* ids, int M, int k, int E, int32_t* counts,
                         int32_t* offsets, hipStream_t s);

// BF16 grouped GEMM (256 x 256 tiles; STORE_F32, STORE_BF16, SWIGLU_BF16)
// (with sorted != nullptr, A row s is row sorted[s] / kr of a: gathered on load)
// (sched: MOE_SCHED_*; AUTO picks hardware dispatch; the queue forms count in `queue`)
hipError_t launch_gemm_bf16(const uint16_t* a, int K, const uint16_t* w, int N,
                            const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                            int epilogue, void* out, hipStream_t s,
                            const int32_t* sorted = nullptr, int kr = 1,
                            int sched = MOE_SCHED_AUTO, uint32_t* queue = nullptr);

// silu(g) * u requantised per 128 columns (the FP8 expert MLP's activation step)
hipError_t launch_swiglu_quant(const float* h, int R, int I, uint8_t* a_q, float* a_scales,
                               hipStream_t s);

// clear: clear_n words set to zero by the same launch (the route-fused GEMM's flags)
hipError_t launch_scatter(const float* rows, const int32_t* route_slots, const float* weights,
                          const int32_t* ids, int M, int k, int E, int N, uint16_t* out,
                          hipStream_t s, uint32_t* clear = nullptr, int clear_n = 0);

}  // namespace moe
