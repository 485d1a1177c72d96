// route.hip -- softcapped softmax routing with top-k selection
// ([FMF8] "Baseline: 7 kernels", item 1 Route; pipeline overview: topk_ids feed the layout,
// topk_weights feed the combine).
//
// One wave64 per token, E/64 logits per lane held in registers.  Selection runs on the raw
// fp32 logit (softcap and softmax are strictly increasing, so the top-k is the same), ordered
// by its monotone 32-bit image and, between equal logits, by the lower expert index: k rounds
// of a wave-wide maximum of the image (DPP row shifts and row broadcasts, no LDS), then one
// ballot per register for the lowest-index holder of that maximum, which is retired.  tanh
// and exp run only for the k winners, on lanes 0..k-1.
//
// With QUANT the token's row of x is also quantised once, with the rule of the
// quantise-sort-gather stage ([FMF8] Baseline items 4-5: amax per 128-value block, scale =
// amax/448, E4M3 of x times the reciprocal), into token-major codes [M][K] and scales
// [K/128][M]: the grouped GEMM then gathers each routed row from there by its token instead
// of reading a sorted copy of it (one copy per token, not one per route).  Routing and
// quantisation are independent, so they run in different waves (grid row 0 routes, rows
// 1..kQuantSplit quantise one slice of K each): a wave's serial chain, not bandwidth, sets
// this kernel's time.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;   // tokens (waves) per workgroup at most
constexpr int kQuantSplit = 2;   // waves quantising one token's row, each a slice of K

// One wave per token; blockDim.x / 64 tokens per workgroup (one while the batch is smaller than
// four per CU, so small batches spread over the CUs).
template <int VPL, bool QUANT>
__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(
    const float* __restrict__ logits, int M, int E, int k, float softcap,
    int32_t* __restrict__ ids, float* __restrict__ weights, const uint16_t* __restrict__ x,
    int K, uint8_t* __restrict__ x_q, float* __restrict__ x_scales, float* __restrict__ acc,
    int acc_n) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (QUANT && blockIdx.y > 0) {
        // quantisation of token t's slice blockIdx.y - 1 of K
        if (t >= M) return;
        if (acc && blockIdx.y == 1) {
            // the token's fp32 accumulator row that the grouped GEMM adds its routes into
            for (int n = lane * 4; n < acc_n; n += 256)
                *reinterpret_cast<float4*>(acc + (size_t)t * acc_n + n) =
                    make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        const int per = (K / 128 + kQuantSplit - 1) / kQuantSplit * 128;
        const int k_lo = (blockIdx.y - 1) * per;
        quantise_token_slice(x, M, K, t, k_lo, min(K, k_lo + per), x_q, x_scales, lane);
        return;
    }
    if (t >= M) return;
    float val[VPL];
    route_load_row<VPL>(logits + (size_t)t * E, E, lane, val);
    int my_e;
    float my_w;
    route_select<VPL>(val, E, k, softcap, lane, my_e, my_w);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        weights[(size_t)t * k + lane] = my_w;
    }
}

template <int VPL>
hipError_t launch_vpl(const float* logits, int M, int E, int k, float softcap, int32_t* ids,
                      float* weights, const uint16_t* x, int K, uint8_t* x_q, float* x_scales,
                      float* acc, int acc_n, hipStream_t s) {
    const int per = M >= kRouteWaves * device_info().cu_count ? kRouteWaves : 1;
    const int grid = (M + per - 1) / per;
    if (x_q)
        hipLaunchKernelGGL((route_kernel<VPL, true>), dim3(grid, 1 + kQuantSplit),
                           dim3(64 * per), 0, s, logits, M, E, k, softcap, ids, weights, x, K, x_q,
                           x_scales, acc, acc_n);
    else
        hipLaunchKernelGGL((route_kernel<VPL, false>), dim3(grid), dim3(64 * per), 0, s,
                           logits, M, E, k, softcap, ids, weights, x, K, x_q, x_scales, acc,
                           acc_n);
    return hipGetLastError();
}

hipError_t launch_route_any(const float* logits, int M, int E, int k, float softcap,
                            int32_t* ids, float* weights, const uint16_t* x, int K,
                            uint8_t* x_q, float* x_scales, float* acc, int acc_n, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define MOE_ROUTE_ARGS logits, M, E, k, softcap, ids, weights, x, K, x_q, x_scales, acc, acc_n, s
    if (E <= 64) return launch_vpl<1>(MOE_ROUTE_ARGS);
    if (E <= 128) return launch_vpl<2>(MOE_ROUTE_ARGS);
    if (E <= 256) return launch_vpl<4>(MOE_ROUTE_ARGS);
    if (E <= 512) return launch_vpl<8>(MOE_ROUTE_ARGS);
    return launch_vpl<16>(MOE_ROUTE_ARGS);
#undef MOE_ROUTE_ARGS
}

}  // namespace

hipError_t launch_route(const float* logits, int M, int E, int k, float softcap, int32_t* ids,
                        float* weights, hipStream_t s) {
    return launch_route_any(logits, M, E, k, softcap, ids, weights, nullptr, 0, nullptr,
                            nullptr, nullptr, 0, s);
}

hipError_t launch_route_quantize(const float* logits, const uint16_t* x, int M, int E, int k,
                                 int K, float softcap, int32_t* ids, float* weights,
                                 uint8_t* x_q, float* x_scales, hipStream_t s, float* acc,
                                 int acc_n) {
    return launch_route_any(logits, M, E, k, softcap, ids, weights, x, K, x_q, x_scales, acc,
                            acc_n, s);
}

}  // namespace moe
