// scatter.hip -- routing-weighted combine of the routed GEMM rows back to BF16 token rows
// ([FMF8] "Baseline: 7 kernels" item 7 and Fusion 1: token = route_id / TOPK,
// weight = topk_weights[token, route_id % TOPK], output[token] += weight * row).
//
// The GEMM writes its fp32 rows with plain stores (in sorted order, or at the route id), and
// the scatter-add becomes a gather-sum per token:
// out[t] = bf16(sum_j w[t][j] * row(t*k+j)), summed in fp32 in j order.  No float atomics,
// no zero-initialised accumulator, and the result does not depend on the order of rows
// inside an expert segment.
#include "moe_device.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kThreads = 256;

// The k routes of a token are read in groups of G (2, 4 or 8, the smallest that holds k, else
// 8): every load of a group (ids, weights, slots, rows) is issued before any is used, so a
// group costs one round trip (two with a slot table), whatever the ids hold; indices past k or
// behind an invalid id are clamped and their terms skipped.
//
// CPT output columns per thread (4, 2 or 1): small batches use narrower threads so the grid
// covers every CU (a CU's requests in flight, not the bytes, bound this kernel).
template <bool SLOTS, int CPT, int kGroup>
__global__ __launch_bounds__(kThreads) void scatter_kernel(
    const float* __restrict__ rows, const int32_t* __restrict__ route_slots,
    const float* __restrict__ weights, const int32_t* __restrict__ ids, int M, int k, int E,
    int N, uint16_t* __restrict__ out, uint32_t* __restrict__ clear, int clear_n) {
    typedef float vec __attribute__((ext_vector_type(CPT)));
    const int groups = N / CPT;
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    // words the step's GEMM has finished with that must start at zero in the next step
    if (clear && idx < (size_t)clear_n) clear[idx] = 0u;
    if (idx >= (size_t)M * groups) return;
    const int t = (int)(idx / groups);
    const int n = (int)(idx % groups) * CPT;
    vec acc = (vec)0.0f;
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
        vec v[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) v[u] = *reinterpret_cast<const vec*>(rows + row[u] * N + n);
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
            if (j0 + u < k && (unsigned)e[u] < (unsigned)E) acc += wv[u] * v[u];
    }
    if constexpr (CPT == 4) {
        uint2 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        *reinterpret_cast<uint2*>(out + (size_t)t * N + n) = o;
    } else if constexpr (CPT == 2) {
        *reinterpret_cast<uint32_t*>(out + (size_t)t * N + n) =
            f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
    } else {
        out[(size_t)t * N + n] = (uint16_t)f32_to_bf16(acc[0]);
    }
}

template <bool SLOTS, int CPT>
hipError_t launch_cpt(const float* rows, const int32_t* route_slots, const float* weights,
                      const int32_t* ids, int M, int k, int E, int N, uint16_t* out,
                      unsigned grid, uint32_t* clear, int clear_n, hipStream_t s) {
    if (k <= 2)
        hipLaunchKernelGGL((scatter_kernel<SLOTS, CPT, 2>), dim3(grid), dim3(kThreads), 0, s,
                           rows, route_slots, weights, ids, M, k, E, N, out, clear, clear_n);
    else if (k <= 4)
        hipLaunchKernelGGL((scatter_kernel<SLOTS, CPT, 4>), dim3(grid), dim3(kThreads), 0, s,
                           rows, route_slots, weights, ids, M, k, E, N, out, clear, clear_n);
    else
        hipLaunchKernelGGL((scatter_kernel<SLOTS, CPT, 8>), dim3(grid), dim3(kThreads), 0, s,
                           rows, route_slots, weights, ids, M, k, E, N, out, clear, clear_n);
    return hipGetLastError();
}

template <bool SLOTS>
hipError_t launch_slots(const float* rows, const int32_t* route_slots, const float* weights,
                        const int32_t* ids, int M, int k, int E, int N, uint16_t* out,
                        uint32_t* clear, int clear_n, hipStream_t s) {
    // widest threads that still give one workgroup per CU
    const size_t cus = (size_t)device_info().cu_count;
    int cpt = 4;
    while (cpt > 1 && (N % cpt || (size_t)M * (N / cpt) < cus * kThreads)) cpt >>= 1;
    const size_t work = (size_t)M * (N / cpt);
    const unsigned grid = (unsigned)((std::max(work, (size_t)clear_n) + kThreads - 1) / kThreads);
    if (cpt == 4)
        return launch_cpt<SLOTS, 4>(rows, route_slots, weights, ids, M, k, E, N, out, grid, clear,
                                      clear_n, s);
    if (cpt == 2)
        return launch_cpt<SLOTS, 2>(rows, route_slots, weights, ids, M, k, E, N, out, grid, clear,
                                      clear_n, s);
    return launch_cpt<SLOTS, 1>(rows, route_slots, weights, ids, M, k, E, N, out, grid, clear,
                                      clear_n, s);
}

}  // namespace

hipError_t launch_scatter(const float* rows, const int32_t* route_slots, const float* weights,
                          const int32_t* ids, int M, int k, int E, int N, uint16_t* out,
                          hipStream_t s, uint32_t* clear, int clear_n) {
    if ((size_t)M * N == 0) return hipSuccess;
    if (route_slots)
        return launch_slots<true>(rows, route_slots, weights, ids, M, k, E, N, out, clear,
                                  clear_n, s);
    return launch_slots<false>(rows, route_slots, weights, ids, M, k, E, N, out, clear, clear_n,
                               s);
}

namespace {

// out[i] = bf16(acc[i]) for the accumulator rows of the scatter-add form, 8 per thread
__global__ __launch_bounds__(kThreads) void acc_to_bf16_kernel(const float* __restrict__ acc,
                                                               size_t n8,
                                                               uint16_t* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n8) return;
    const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
    uint4 o;
    o.x = f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16);
    o.y = f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16);
    o.z = f32_to_bf16(b.x) | (f32_to_bf16(b.y) << 16);
    o.w = f32_to_bf16(b.z) | (f32_to_bf16(b.w) << 16);
    reinterpret_cast<uint4*>(out)[i] = o;
}

}  // namespace

hipError_t launch_acc_to_bf16(const float* acc, int M, int N, uint16_t* out, hipStream_t s) {
    const size_t n8 = (size_t)M * N / 8;        // N a multiple of 128
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(acc_to_bf16_kernel, dim3((unsigned)((n8 + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, acc, n8, out);
    return hipGetLastError();
}

}  // namespace moe
