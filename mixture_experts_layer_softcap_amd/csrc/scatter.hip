// scatter.hip -- routing-weighted combine of the routed GEMM rows back to BF16 token rows
// ([FMF8] "Baseline: 7 kernels" item 7 and Fusion 1: token = route_id / TOPK,
// weight = topk_weights[token, route_id % TOPK], output[token] += weight * row).
//
// The GEMM writes its fp32 rows with plain 16-byte stores (in sorted order, or at the route
// id), and the scatter-add becomes a gather-sum per token:
// out[t] = bf16(sum_j w[t][j] * row(t*k+j)), summed in fp32 in j order.  No float atomics,
// no zero-initialised accumulator, and the result does not depend on the order of rows
// inside an expert segment.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// The k routes of a token are read in groups of kGroup: every load of a group (ids, weights,
// slots, rows) is issued before any is used, so a group costs one round trip (two with a slot
// table), whatever the ids hold; indices past k or behind an invalid id are clamped and their
// terms skipped.
constexpr int kGroup = 8;

template <bool SLOTS>
__global__ __launch_bounds__(kThreads) void scatter_kernel(
    const float* __restrict__ rows, const int32_t* __restrict__ route_slots,
    const float* __restrict__ weights, const int32_t* __restrict__ ids, int M, int k, int E,
    int N, uint16_t* __restrict__ out) {
    const int quads = N >> 2;
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (size_t)M * quads) return;
    const int t = (int)(idx / quads);
    const int n = (int)(idx % quads) * 4;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        int e[kGroup];
        float wv[kGroup];
        size_t row[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const size_t r = (size_t)t * k + min(j0 + u, k - 1);
            e[u] = ids[r];
            wv[u] = weights[r];
            row[u] = r;
            if (SLOTS) {
                const int sl = route_slots[r];          // -1 behind an invalid id
                row[u] = sl < 0 ? 0 : (size_t)sl;
            }
        }
        float4 v[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
            v[u] = *reinterpret_cast<const float4*>(rows + row[u] * N + n);
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if (j0 + u < k && (unsigned)e[u] < (unsigned)E) {
                acc.x += wv[u] * v[u].x;
                acc.y += wv[u] * v[u].y;
                acc.z += wv[u] * v[u].z;
                acc.w += wv[u] * v[u].w;
            }
        }
    }
    uint2 o;
    o.x = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    o.y = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(out + (size_t)t * N + n) = o;
}

}  // namespace

hipError_t launch_scatter(const float* rows, const int32_t* route_slots, const float* weights,
                          const int32_t* ids, int M, int k, int E, int N, uint16_t* out,
                          hipStream_t s) {
    const size_t work = (size_t)M * (N / 4);
    if (work == 0) return hipSuccess;
    const unsigned grid = (unsigned)((work + kThreads - 1) / kThreads);
    if (route_slots)
        hipLaunchKernelGGL(scatter_kernel<true>, dim3(grid), dim3(kThreads), 0, s, rows,
                           route_slots, weights, ids, M, k, E, N, out);
    else
        hipLaunchKernelGGL(scatter_kernel<false>, dim3(grid), dim3(kThreads), 0, s, rows,
                           route_slots, weights, ids, M, k, E, N, out);
    return hipGetLastError();
}

}  // namespace moe
