// layout.hip -- per-expert counts, exclusive prefix sum, write cursors and the grouped-GEMM
// task list in one workgroup ([FMF8] "Baseline: 7 kernels" items 2-3, Fusion 3 count and
// build layout, Phase 5 parallel prefix scan and pipelined topk_ids loads; [WEAVE] section
// 4.3 task-list construction: histogram, prefix sum, per-expert chunks).
//
// 1024 threads: ids are loaded four per thread before the LDS histogram atomics; the scan is
// a wave64 shuffle scan plus a cross-wave scan of the 16 wave totals.  Tasks: the full
// chunk_rows-row chunks of every expert first (expert order), then each expert's partial
// chunk placed by a counting sort on its row count, largest first; every chunk is crossed
// with the n_blocks weight panels (consecutive entries share the chunk).  The persistent
// queue counter is reset here so the captured step needs no memset node.  Optionally the
// routes are also sorted by expert ([FMF8] Baseline item 5's slot assignment, here with LDS
// atomics on per-expert cursors rather than global ones): sorted_route_ids[slot] = route and
// route_slots[route] = slot, a slot's order inside its expert segment being arbitrary.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Exclusive block scan of one int per thread; returns the exclusive prefix and the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_inclusive_scan(v);
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kWaves ? s_wsum[lane] : 0;
        const int winc = wave_inclusive_scan(w);
        if (lane < kWaves) s_wsum[lane] = winc - w;        // exclusive wave base
        if (lane == kWaves - 1) s_wsum[kWaves] = winc;    // block total
    }
    __syncthreads();
    const int excl = inc - v + s_wsum[wave];
    total = s_wsum[kWaves];
    __syncthreads();                                      // s_wsum may be reused
    return excl;
}

__global__ __launch_bounds__(kThreads) void layout_kernel(
    const int32_t* __restrict__ ids, int R, int E, int n_blocks, int chunk,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ cursors,
    moe_task* __restrict__ tasks, int32_t* __restrict__ ntasks, uint32_t* __restrict__ queue,
    int32_t* __restrict__ sorted_route_ids, int32_t* __restrict__ route_slots) {
    // one histogram per wave over its own contiguous range of routes: the LDS atomics of a
    // busy expert are spread over 16 counters instead of queueing on one
    __shared__ int s_hw[kWaves][kThreads];
    __shared__ int s_hist[kThreads];      // number of experts whose partial chunk has size s
    __shared__ int s_wsum[kWaves + 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int span = (R + kWaves - 1) / kWaves;
    const int r_lo = min(R, wave * span), r_hi = min(R, r_lo + span);

#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_hw[w][tid] = 0;
    s_hist[tid] = 0;
    __syncthreads();

    for (int base = r_lo; base < r_hi; base += 4 * 64) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = base + u * 64 + lane;
            v[u] = r < r_hi ? ids[r] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if ((unsigned)v[u] < (unsigned)E) atomicAdd(&s_hw[wave][v[u]], 1);
    }
    __syncthreads();

    int c = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c += s_hw[w][tid];
    }
    const int full = c / chunk;
    const int tail = c - full * chunk;
    int total_rows, total_full;
    const int row0 = block_exclusive_scan(c, s_wsum, total_rows);
    const int full0 = block_exclusive_scan(full, s_wsum, total_full);

    if (tail > 0) atomicAdd(&s_hist[tail], 1);
    __syncthreads();
    // descending scan over partial-chunk sizes: thread i looks at size chunk-1-i
    const int size = chunk - 1 - tid;
    const int h = size >= 1 ? s_hist[size] : 0;
    int total_tails;
    const int larger = block_exclusive_scan(h, s_wsum, total_tails);
    if (size >= 1) s_hist[size] = larger;                 // first position of size `size`
    __syncthreads();

    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = row0;
        cursors[tid] = row0;
        // each wave's first slot inside the expert's segment (waves in route order)
        int run = row0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int h = s_hw[w][tid];
            s_hw[w][tid] = run;
            run += h;
        }
        if (tid == E - 1) offsets[E] = row0 + c;
        for (int i = 0; i < full; ++i) {
            const int p = full0 + i;
            for (int nb = 0; nb < n_blocks; ++nb)
                *reinterpret_cast<int4*>(&tasks[(size_t)p * n_blocks + nb]) =
                    make_int4(tid, row0 + i * chunk, chunk, nb);
        }
        if (tail > 0) {
            const int p = total_full + atomicAdd(&s_hist[tail], 1);
            for (int nb = 0; nb < n_blocks; ++nb)
                *reinterpret_cast<int4*>(&tasks[(size_t)p * n_blocks + nb]) =
                    make_int4(tid, row0 + full * chunk, tail, nb);
        }
    }
    if (tid == 0) {
        ntasks[0] = (total_full + total_tails) * n_blocks;
        queue[0] = 0u;
        queue[1] = 0u;
    }
    if (sorted_route_ids) {
        __syncthreads();                                  // s_hw holds the wave cursors
        for (int base = r_lo; base < r_hi; base += 4 * 64) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = base + u * 64 + lane;
                v[u] = r < r_hi ? ids[r] : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = base + u * 64 + lane;
                if (r >= r_hi) continue;
                int slot = -1;
                if ((unsigned)v[u] < (unsigned)E) {
                    slot = atomicAdd(&s_hw[wave][v[u]], 1);
                    sorted_route_ids[slot] = r;
                }
                if (route_slots) route_slots[r] = slot;
            }
        }
    }
}

// Per-expert counts and exclusive offsets alone (the layout kernel without the task list).
__global__ __launch_bounds__(kThreads) void counts_kernel(const int32_t* __restrict__ ids, int R,
                                                          int E, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets) {
    __shared__ int s_cnt[kThreads];
    __shared__ int s_wsum[kWaves + 1];
    const int tid = threadIdx.x;
    s_cnt[tid] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kThreads) {
        const int e = ids[r];
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    const int c = tid < E ? s_cnt[tid] : 0;
    int total;
    const int o = block_exclusive_scan(c, s_wsum, total);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = o;
        if (tid == E - 1) offsets[E] = o + c;
    }
}

}  // namespace

hipError_t launch_layout(const int32_t* ids, int M, int k, int E, int n_blocks, int chunk_rows,
                         int32_t* counts, int32_t* offsets, int32_t* cursors, moe_task* tasks,
                         int max_tasks, int32_t* ntasks, uint32_t* queue,
                         int32_t* sorted_route_ids, int32_t* route_slots, hipStream_t s) {
    (void)max_tasks;  // capacity checked on the host against moe_max_tasks
    hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(kThreads), 0, s, ids, M * k, E, n_blocks,
                       chunk_rows, counts, offsets, cursors, tasks, ntasks, queue,
                       sorted_route_ids, route_slots);
    return hipGetLastError();
}

hipError_t launch_counts(const int32_t* ids, int M, int k, int E, int32_t* counts,
                         int32_t* offsets, hipStream_t s) {
    hipLaunchKernelGGL(counts_kernel, dim3(1), dim3(kThreads), 0, s, ids, M * k, E, counts,
                       offsets);
    return hipGetLastError();
}

}  // namespace moe
