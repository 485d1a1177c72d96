// gemm_fp8_tile.hip -- launchers of the LDS-tiled grouped FP8 GEMM (kernel in gemm_fp8_tile.h)
// on sorted FP8 rows: chunks of 65..256 routed rows, the fp32 / bf16 / route-id epilogues,
// one workgroup per item under hardware dispatch.
#include "gemm_fp8_tile.h"

namespace moe {
namespace {

template <int BM, int EPI>
hipError_t launch_epi(const uint8_t* a, const float* a_scales, int rows, int K,
                      const uint8_t* w, const float* w_scales, int N, const moe_task* tasks,
                      const int32_t* ntasks, int max_tasks, const int32_t* sorted, void* out,
                      hipStream_t s) {
    if (K == 2048)
        return launch_tile<BM, EPI, 16, false, MOE_SCHED_DISPATCH>(
            a, a_scales, rows, K, w, w_scales, N, tasks, ntasks, max_tasks, sorted, out, 1,
            nullptr, s);
    return launch_tile<BM, EPI, 0, false, MOE_SCHED_DISPATCH>(
        a, a_scales, rows, K, w, w_scales, N, tasks, ntasks, max_tasks, sorted, out, 1, nullptr,
        s);
}

template <int BM>
hipError_t launch_bm(const uint8_t* a, const float* a_scales, int rows, int K, const uint8_t* w,
                     const float* w_scales, int N, const moe_task* tasks,
                     const int32_t* ntasks, int max_tasks, int epilogue, const int32_t* sorted,
                     void* out, hipStream_t s) {
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            return launch_epi<BM, MOE_EPI_STORE_BF16>(a, a_scales, rows, K, w, w_scales, N,
                                                      tasks, ntasks, max_tasks, sorted, out, s);
        case MOE_EPI_ROUTE_F32:
            return launch_epi<BM, MOE_EPI_ROUTE_F32>(a, a_scales, rows, K, w, w_scales, N,
                                                     tasks, ntasks, max_tasks, sorted, out, s);
        default:
            return launch_epi<BM, MOE_EPI_STORE_F32>(a, a_scales, rows, K, w, w_scales, N,
                                                     tasks, ntasks, max_tasks, sorted, out, s);
    }
}

}  // namespace

bool gemm_fp8_tile_applies(int K, int chunk_rows) {
    return chunk_rows > 64 && chunk_rows <= 256 && K / 128 <= kMaxKB;
}

hipError_t launch_gemm_fp8_tile(const uint8_t* a, const float* a_scales, int rows, int K,
                                const uint8_t* w, const float* w_scales, int N,
                                const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                                int chunk_rows, int epilogue, const int32_t* sorted, void* out,
                                hipStream_t s) {
    if (max_tasks <= 0) return hipSuccess;
    if (chunk_rows <= 128)
        return launch_bm<128>(a, a_scales, rows, K, w, w_scales, N, tasks, ntasks, max_tasks,
                              epilogue, sorted, out, s);
    return launch_bm<256>(a, a_scales, rows, K, w, w_scales, N, tasks, ntasks, max_tasks,
                          epilogue, sorted, out, s);
}

}  // namespace moe
