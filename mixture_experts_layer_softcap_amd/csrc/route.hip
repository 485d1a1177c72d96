// route.hip -- softcapped softmax routing with top-k selection
// ([FMF8] "Baseline: 7 kernels", item 1 Route; pipeline overview: topk_ids feed the layout,
// topk_weights feed the combine).
//
// One wave64 per token, E/64 logits per lane held in registers.  Selection runs on the raw
// fp32 logit (softcap and softmax are strictly increasing, so the top-k is the same) as k
// rounds of a wave-wide argmax over a 64-bit key: the high word orders the float, the low
// word holds 0xFFFFFFFF - e so equal logits resolve to the lower expert index.  tanh and exp
// run only for the k winners, on lanes 0..k-1.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int M,
                                                    int E, int k, float softcap,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= M) return;
    const float* row = logits + (size_t)t * E;

    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? route_key(row[e], e) : 0ull;   // 0 sorts below every valid key
    }

    int my_e = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off);
            best = o > best ? o : best;
        }
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        // retire the winner in the lane that holds it
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + 64 * i == e) key[i] = 0ull;
        if (lane == j) {
            my_e = e;
            my_l = row[e];
        }
    }

    const bool active = lane < k;
    float c = my_l;
    if (softcap > 0.0f) c = softcap * tanhf(my_l / softcap);
    const float c0 = __shfl(c, 0);                         // the largest selected value
    const float ex = active ? expf(c - c0) : 0.0f;
    const float sum = wave_sum(ex);
    if (active) {
        ids[(size_t)t * k + lane] = my_e;
        weights[(size_t)t * k + lane] = ex / sum;
    }
}

template <int VPL>
hipError_t launch_vpl(const float* logits, int M, int E, int k, float softcap, int32_t* ids,
                      float* weights, hipStream_t s) {
    const int grid = (M + 3) / 4;
    hipLaunchKernelGGL(route_kernel<VPL>, dim3(grid), dim3(256), 0, s, logits, M, E, k,
                       softcap, ids, weights);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int M, int E, int k, float softcap, int32_t* ids,
                        float* weights, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (E <= 64) return launch_vpl<1>(logits, M, E, k, softcap, ids, weights, s);
    if (E <= 128) return launch_vpl<2>(logits, M, E, k, softcap, ids, weights, s);
    if (E <= 256) return launch_vpl<4>(logits, M, E, k, softcap, ids, weights, s);
    if (E <= 512) return launch_vpl<8>(logits, M, E, k, softcap, ids, weights, s);
    return launch_vpl<16>(logits, M, E, k, softcap, ids, weights, s);
}

}  // namespace moe
