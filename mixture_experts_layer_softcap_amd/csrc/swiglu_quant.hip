// swiglu_quant.hip -- the activation step of the FP8 expert MLP ([FMF8] comparison section,
// the "vLLM full MLP" reference: gate+up projection, SiLU gating, down projection): from the
// gate+up GEMM's fp32 rows h [R][2I] (gate columns first), act = silu(g) * u in fp32,
// requantised per 128 columns with the QSG rule (scale = amax/448, E4M3 of act times the
// reciprocal) into codes [R][I] and scales [I/128][R], rows kept in their (expert-sorted)
// order so the down GEMM reads them as its A operand.
//
// One wave per 512 columns of a row (swiglu_quant_piece).  HBM-bound: 8*I bytes read, I +
// I/32 written per row.  The FP8 MLP's small-batch path runs the same pieces in the layout's
// launch (layout.hip).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void swiglu_quant_kernel(
    const float* __restrict__ h, int R, int I, uint8_t* __restrict__ a_q,
    float* __restrict__ a_scales) {
    const long long item = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    swiglu_quant_piece(h, R, I, a_q, a_scales, item, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_swiglu_quant(const float* h, int R, int I, uint8_t* a_q, float* a_scales,
                               hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const long long waves = (long long)R * ((I + 511) / 512);
    const long long grid = (waves + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL(swiglu_quant_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, h, R,
                       I, a_q, a_scales);
    return hipGetLastError();
}

}  // namespace moe
