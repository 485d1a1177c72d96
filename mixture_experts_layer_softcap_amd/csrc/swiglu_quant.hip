// swiglu_quant.hip -- the activation step of the FP8 expert MLP ([FMF8] comparison section,
// the "vLLM full MLP" reference: gate+up projection, SiLU gating, down projection): from the
// gate+up GEMM's fp32 rows h [R][2I] (gate columns first), act = silu(g) * u in fp32,
// requantised per 128 columns with the QSG rule (scale = amax/448, E4M3 of act times the
// reciprocal) into codes [R][I] and scales [I/128][R], rows kept in their (expert-sorted)
// order so the down GEMM reads them as its A operand.
//
// One wave per 512 columns of a row: lane l holds columns [8l, 8l+8) of the piece, so a
// 128-column block is an aligned group of 16 lanes (I is a multiple of 128: a group lies
// wholly inside or outside the row).  HBM-bound: 8*I bytes read, I + I/32 written per row.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void swiglu_quant_kernel(
    const float* __restrict__ h, int R, int I, uint8_t* __restrict__ a_q,
    float* __restrict__ a_scales) {
    const int lane = threadIdx.x & 63;
    const int pieces = (I + 511) >> 9;
    const long long item = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (item >= (long long)R * pieces) return;
    const int r = (int)(item / pieces);
    const int c = (int)(item % pieces) * 512 + lane * 8;
    const bool valid = c < I;
    float v[8];
    if (valid) {
        const float* hr = h + (size_t)r * 2 * I;
        const float4 g0 = *reinterpret_cast<const float4*>(hr + c);
        const float4 g1 = *reinterpret_cast<const float4*>(hr + c + 4);
        const float4 u0 = *reinterpret_cast<const float4*>(hr + I + c);
        const float4 u1 = *reinterpret_cast<const float4*>(hr + I + c + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    const Quant8 q = quantise8_f32(v, valid);
    if (valid) {
        *reinterpret_cast<uint2*>(a_q + (size_t)r * I + c) = q.codes;
        if ((lane & 15) == 0) a_scales[(size_t)(c >> 7) * R + r] = q.scale;
    }
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
