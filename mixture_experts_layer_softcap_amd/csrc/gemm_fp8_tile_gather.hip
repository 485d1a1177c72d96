// gemm_fp8_tile_gather.hip -- launchers of the LDS-tiled grouped FP8 GEMM (kernel in
// gemm_fp8_tile.h) that gathers each routed row from the token-major codes on load: the
// forward's larger batches (chunks of 65..256 routed rows), fp32 rows at route ids, under one
// of the four task schedules (hardware dispatch, static persistent walk, one atomic queue,
// per-XCD atomic queues).
#include "gemm_fp8_tile.h"

namespace moe {
namespace {

// The persistent schedules are built for 128-row chunks only: with 256-row chunks the walk
// around the tile body does not fit the register file (the compiler spills ~2000 VGPRs).
template <int BM, int KBC>
hipError_t launch_sched(int sched, const uint8_t* x_q, const float* x_scales, int M, int k,
                        int K, const uint8_t* w, const float* w_scales, int N,
                        const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                        const int32_t* sorted, float* rows_out, uint32_t* queue,
                        hipStream_t s) {
#define MOE_TILE_ARGS x_q, x_scales, M, K, w, w_scales, N, tasks, ntasks, max_tasks, sorted, \
                      rows_out, k, queue, s
    if constexpr (BM > 128) {                      // (the API rejects other schedules first)
        (void)sched;
        return launch_tile<BM, MOE_EPI_ROUTE_F32, KBC, true, MOE_SCHED_DISPATCH>(MOE_TILE_ARGS);
    } else {
        switch (sched) {
            case MOE_SCHED_STATIC:
                return launch_tile<BM, MOE_EPI_ROUTE_F32, KBC, true, MOE_SCHED_STATIC>(
                    MOE_TILE_ARGS);
            case MOE_SCHED_QUEUE:
                return launch_tile<BM, MOE_EPI_ROUTE_F32, KBC, true, MOE_SCHED_QUEUE>(
                    MOE_TILE_ARGS);
            case MOE_SCHED_QUEUE_XCD:
                return launch_tile<BM, MOE_EPI_ROUTE_F32, KBC, true, MOE_SCHED_QUEUE_XCD>(
                    MOE_TILE_ARGS);
            default:
                return launch_tile<BM, MOE_EPI_ROUTE_F32, KBC, true, MOE_SCHED_DISPATCH>(
                    MOE_TILE_ARGS);
        }
    }
#undef MOE_TILE_ARGS
}

}  // namespace

hipError_t launch_gemm_fp8_tile_gather(const uint8_t* x_q, const float* x_scales, int M, int k,
                                       int K, const uint8_t* w, const float* w_scales, int N,
                                       const moe_task* tasks, const int32_t* ntasks,
                                       int max_tasks, int chunk_rows, const int32_t* sorted,
                                       float* rows_out, int sched, uint32_t* queue,
                                       hipStream_t s) {
    if (max_tasks <= 0) return hipSuccess;
    if (sched != MOE_SCHED_DISPATCH && !queue && sched != MOE_SCHED_STATIC)
        return hipErrorInvalidValue;
    if (chunk_rows <= 128) {
        if (K == 2048)
            return launch_sched<128, 16>(sched, x_q, x_scales, M, k, K, w, w_scales, N, tasks,
                                         ntasks, max_tasks, sorted, rows_out, queue, s);
        return launch_sched<128, 0>(sched, x_q, x_scales, M, k, K, w, w_scales, N, tasks,
                                    ntasks, max_tasks, sorted, rows_out, queue, s);
    }
    if (K == 2048)
        return launch_sched<256, 16>(sched, x_q, x_scales, M, k, K, w, w_scales, N, tasks,
                                     ntasks, max_tasks, sorted, rows_out, queue, s);
    return launch_sched<256, 0>(sched, x_q, x_scales, M, k, K, w, w_scales, N, tasks, ntasks,
                                max_tasks, sorted, rows_out, queue, s);
}

hipError_t launch_gemm_fp8_tile_gather_atomic(const uint8_t* x_q, const float* x_scales, int M,
                                              int k, int K, const uint8_t* w,
                                              const float* w_scales, int N,
                                              const moe_task* tasks, const int32_t* ntasks,
                                              int max_tasks, int chunk_rows,
                                              const int32_t* sorted, const float* weights,
                                              float* acc, hipStream_t s) {
    if (max_tasks <= 0) return hipSuccess;
#define MOE_TILE_ARGS x_q, x_scales, M, K, w, w_scales, N, tasks, ntasks, max_tasks, sorted, acc, \
                      k, nullptr, s, weights
    if (chunk_rows <= 128) {
        if (K == 2048)
            return launch_tile<128, kEpiAtomicAdd, 16, true, MOE_SCHED_DISPATCH>(MOE_TILE_ARGS);
        return launch_tile<128, kEpiAtomicAdd, 0, true, MOE_SCHED_DISPATCH>(MOE_TILE_ARGS);
    }
    if (K == 2048)
        return launch_tile<256, kEpiAtomicAdd, 16, true, MOE_SCHED_DISPATCH>(MOE_TILE_ARGS);
    return launch_tile<256, kEpiAtomicAdd, 0, true, MOE_SCHED_DISPATCH>(MOE_TILE_ARGS);
#undef MOE_TILE_ARGS
}

}  // namespace moe
