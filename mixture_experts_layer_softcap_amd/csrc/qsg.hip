// qsg.hip -- blockwise FP8 E4M3 quantisation fused with the sort/gather into
// expert-contiguous rows ([FMF8] "Baseline: 7 kernels" items 4-5; Fusion 2 QSG; Phase 3
// vectorised copy and batched quantisation; Phase 5 load pipelining, parallel slot
// assignment; compiler-flag table: transposed activation scales [K_BLOCKS, routes]).
//
// One workgroup of 256 threads per token; a thread owns 8 consecutive bf16 (one 16-byte
// load), so a 128-wide block is one aligned group of 16 lanes and its amax is four xor
// shuffles -- no LDS and no barrier in the quantiser.  Lanes 0..k-1 take the k slots with
// global atomics on the expert cursors while the row loads are in flight; one barrier
// publishes the slots, then every thread stores its 8 codes to each of the k sorted rows.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSpan = kThreads * 8;  // elements of one row covered per pass

__global__ __launch_bounds__(kThreads) void qsg_kernel(
    const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ ids, int k, int E,
    int32_t* __restrict__ cursors, int32_t* __restrict__ sorted_route_ids,
    int32_t* __restrict__ route_slots, uint8_t* __restrict__ a_q, float* __restrict__ a_scales) {
    __shared__ int s_slot[64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t R = (size_t)M * k;
    const uint16_t* xrow = x + (size_t)t * K;

    // first pass's row data is requested before the slot atomics and the barrier
    int k0 = tid * 8;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (k0 < K) raw = *reinterpret_cast<const uint4*>(xrow + k0);

    if (tid < k) {
        const int r = t * k + tid;
        const int e = ids[r];
        int slot = -1;
        if ((unsigned)e < (unsigned)E) {
            slot = atomicAdd(&cursors[e], 1);
            sorted_route_ids[slot] = r;
        }
        s_slot[tid] = slot;
        if (route_slots) route_slots[r] = slot;
    }
    __syncthreads();

    for (;;) {
        const bool valid = k0 < K;
        const Quant8 q = quantise8(raw, valid);
        if (valid) {
            for (int j = 0; j < k; ++j) {
                const int slot = s_slot[j];
                if (slot < 0) continue;
                *reinterpret_cast<uint2*>(a_q + (size_t)slot * K + k0) = q.codes;
                if ((tid & 15) == 0) a_scales[(size_t)(k0 >> 7) * R + slot] = q.scale;
            }
        }
        k0 += kSpan;
        if (k0 - tid * 8 >= K) break;
        raw = make_uint4(0u, 0u, 0u, 0u);
        if (k0 < K) raw = *reinterpret_cast<const uint4*>(xrow + k0);
    }
}

// The bf16 form of the same sort/gather ([WEAVE] Mixtral-like layer: rows are gathered into
// expert-contiguous order without quantisation): slots as above, then every thread copies
// its 16 bytes of the token's row to each of the k sorted rows.
__global__ __launch_bounds__(kThreads) void gather_bf16_kernel(
    const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ ids, int k, int E,
    int32_t* __restrict__ cursors, int32_t* __restrict__ sorted_route_ids,
    int32_t* __restrict__ route_slots, uint16_t* __restrict__ a) {
    __shared__ int s_slot[64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* xrow = x + (size_t)t * K;
    if (tid < k) {
        const int r = t * k + tid;
        const int e = ids[r];
        int slot = -1;
        if ((unsigned)e < (unsigned)E) {
            slot = atomicAdd(&cursors[e], 1);
            sorted_route_ids[slot] = r;
        }
        s_slot[tid] = slot;
        if (route_slots) route_slots[r] = slot;
    }
    __syncthreads();
    for (int k0 = tid * 8; k0 < K; k0 += kSpan) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xrow + k0);
        for (int j = 0; j < k; ++j) {
            const int slot = s_slot[j];
            if (slot >= 0) *reinterpret_cast<uint4*>(a + (size_t)slot * K + k0) = raw;
        }
    }
}

}  // namespace

hipError_t launch_gather_bf16(const uint16_t* x, int M, int K, const int32_t* ids, int k, int E,
                              int32_t* cursors, int32_t* sorted_route_ids,
                              int32_t* route_slots, uint16_t* a, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_bf16_kernel, dim3(M), dim3(kThreads), 0, s, x, M, K, ids, k, E,
                       cursors, sorted_route_ids, route_slots, a);
    return hipGetLastError();
}

hipError_t launch_qsg(const uint16_t* x, int M, int K, const int32_t* ids, int k, int E,
                      int32_t* cursors, int32_t* sorted_route_ids, int32_t* route_slots,
                      uint8_t* a_q, float* a_scales, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(qsg_kernel, dim3(M), dim3(kThreads), 0, s, x, M, K, ids, k, E, cursors,
                       sorted_route_ids, route_slots, a_q, a_scales);
    return hipGetLastError();
}

}  // namespace moe
