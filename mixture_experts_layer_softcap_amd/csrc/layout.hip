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

// chunks whose tasks are written from an LDS table, consecutive threads on consecutive tasks
constexpr int kChunkTable = 4096;

// The task list of expert counts c (thread e holds c_e and its exclusive prefix row0): full
// chunk_rows-row chunks first (expert order), then the partial chunks by a counting sort on
// their row count, largest first, each crossed with the n_blocks panels; also offsets[E+1],
// cursors = offsets, ntasks, and the queue reset.  Every thread of the workgroup calls it.
// Up to kChunkTable chunks, each expert's thread only files its chunks in LDS and the whole
// workgroup then writes the tasks in order (every store instruction covers 1 KiB of the
// list); beyond that, each expert's thread writes its own tasks.
__device__ void write_tasks(int c, int row0, int E, int n_blocks, int chunk,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ cursors,
                            moe_task* __restrict__ tasks, int32_t* __restrict__ ntasks,
                            uint32_t* __restrict__ queue, int* s_hist, int* s_wsum) {
    __shared__ int2 s_chunks[kChunkTable];        // (row_begin, expert | rows << 16)
    const int tid = threadIdx.x;
    const int full = c / chunk;
    const int tail = c - full * chunk;
    int total_full;
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
    const int nchunks = total_full + total_tails;
    if (tid < E) {
        offsets[tid] = row0;
        cursors[tid] = row0;
        if (tid == E - 1) offsets[E] = row0 + c;
    }
    if (nchunks <= kChunkTable) {                         // uniform over the workgroup
        if (tid < E) {
            for (int i = 0; i < full; ++i)
                s_chunks[full0 + i] = make_int2(row0 + i * chunk, tid | (chunk << 16));
            if (tail > 0)
                s_chunks[total_full + atomicAdd(&s_hist[tail], 1)] =
                    make_int2(row0 + full * chunk, tid | (tail << 16));
        }
        __syncthreads();
        const int T = nchunks * n_blocks;
        for (int t = tid; t < T; t += kThreads) {
            const int p = t / n_blocks;
            const int2 ci = s_chunks[p];
            *reinterpret_cast<int4*>(&tasks[t]) =
                make_int4(ci.y & 0xFFFF, ci.x, ci.y >> 16, t - p * n_blocks);
        }
    } else if (tid < E) {
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
        ntasks[0] = nchunks * n_blocks;
#pragma unroll
        for (int i = 0; i < MOE_QUEUE_WORDS; ++i) queue[i] = 0u;
    }
}

__device__ __forceinline__ void layout_body(
    const int32_t* __restrict__ ids, int R, int E, int n_blocks, int chunk,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ cursors,
    moe_task* __restrict__ tasks, int32_t* __restrict__ ntasks, uint32_t* __restrict__ queue,
    int32_t* __restrict__ sorted_route_ids, int32_t* __restrict__ route_slots, int n_blocks2,
    moe_task* __restrict__ tasks2, int32_t* __restrict__ ntasks2, uint32_t* __restrict__ queue2) {
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

    // a wave's ids stay in registers for the sort (kHeld per lane; a larger range is read again)
    constexpr int kHeld = 32;
    int held[kHeld];
#pragma unroll
    for (int u = 0; u < kHeld; ++u) {
        const int r = r_lo + u * 64 + lane;
        held[u] = r < r_hi ? ids[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kHeld; ++u)
        if ((unsigned)held[u] < (unsigned)E) atomicAdd(&s_hw[wave][held[u]], 1);
    for (int base = r_lo + kHeld * 64; base < r_hi; base += 4 * 64) {
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
    int total_rows;
    const int row0 = block_exclusive_scan(c, s_wsum, total_rows);
    write_tasks(c, row0, E, n_blocks, chunk, offsets, cursors, tasks, ntasks, queue, s_hist,
                s_wsum);
    if (tasks2) {
        // a second task list over the same chunks, n_blocks2 panels each
        __syncthreads();
        s_hist[tid] = 0;
        __syncthreads();
        write_tasks(c, row0, E, n_blocks2, chunk, offsets, cursors, tasks2, ntasks2, queue2,
                    s_hist, s_wsum);
    }
    if (tid < E) {
        counts[tid] = c;
        // each wave's first slot inside the expert's segment (waves in route order)
        int run = row0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int h = s_hw[w][tid];
            s_hw[w][tid] = run;
            run += h;
        }
    }
    if (sorted_route_ids) {
        __syncthreads();                                  // s_hw holds the wave cursors
        auto place = [&](int r, int e) __attribute__((always_inline)) {
            if (r >= r_hi) return;
            int slot = -1;
            if ((unsigned)e < (unsigned)E) {
                slot = atomicAdd(&s_hw[wave][e], 1);
                sorted_route_ids[slot] = r;
            }
            if (route_slots) route_slots[r] = slot;
        };
#pragma unroll
        for (int u = 0; u < kHeld; ++u) place(r_lo + u * 64 + lane, held[u]);
        for (int base = r_lo + kHeld * 64; base < r_hi; base += 4 * 64) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = base + u * 64 + lane;
                v[u] = r < r_hi ? ids[r] : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) place(base + u * 64 + lane, v[u]);
        }
    }
}

__global__ __launch_bounds__(kThreads) void layout_kernel(
    const int32_t* __restrict__ ids, int R, int E, int n_blocks, int chunk,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ cursors,
    moe_task* __restrict__ tasks, int32_t* __restrict__ ntasks, uint32_t* __restrict__ queue,
    int32_t* __restrict__ sorted_route_ids, int32_t* __restrict__ route_slots, int n_blocks2,
    moe_task* __restrict__ tasks2, int32_t* __restrict__ ntasks2, uint32_t* __restrict__ queue2) {
    layout_body(ids, R, E, n_blocks, chunk, counts, offsets, cursors, tasks, ntasks, queue,
                sorted_route_ids, route_slots, n_blocks2, tasks2, ntasks2, queue2);
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

// ---- the same layout over many workgroups (the forward's larger batches) ------------------
// A single workgroup is bound by its own CU's requests in flight; here every workgroup takes
// the kThreads routes of its chunk, one per thread, in one launch with no exchange between
// workgroups.  Each workgroup histograms ALL routes' ids in LDS, and separately those of the
// chunks before its own: the expert totals (hence offsets, the task list, and for workgroup 0
// counts, cursors, ntasks and the queue reset as layout_kernel writes them) and the chunk's
// first slot inside every expert segment follow locally, with no global atomics and nothing to
// clear beforehand.  Inside the chunk a route's rank among the routes of its expert is stable:
// wave ballots find the lanes holding the same id, and the per-wave counts are prefixed in
// wave order.  Every segment therefore holds its routes in ascending route id, the order of
// the serial counting sort ([FMF8] Baseline item 5).

struct WideLayoutOut {
    int32_t* counts;
    int32_t* offsets;
    int32_t* cursors;
    moe_task* tasks;
    int32_t* ntasks;
    uint32_t* queue;
    int32_t* sorted_route_ids;
    int32_t* route_slots;                         // may be null
    int n_blocks, chunk;
    moe_task* tasks2;                             // a second task list, or null
    int32_t* ntasks2;
    uint32_t* queue2;
    int n_blocks2;
};

// Everything after the histograms: route r of this chunk has id e; s_all and s_before hold
// the whole batch's and the earlier chunks' counts (their atomics issued before the call),
// s_wcnt [kWaves][E] is zero, s_hist zero; `writer`: this workgroup writes counts, offsets,
// cursors and the task lists.
__device__ __forceinline__ void wide_place(int e, int r, int R, int E, bool writer,
                                           const WideLayoutOut& o, int* s_all, int* s_before,
                                           int* s_first, int* s_hist, int* s_wsum,
                                           int* s_wcnt) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // stable rank inside the wave: lanes whose value v (E for a route past R or an invalid id)
    // agrees with this lane's in every bit
    const int v = (unsigned)e < (unsigned)E ? e : E;
    const int nbits = 32 - __clz(E);
    uint64_t same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (v >> b) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    const int rank_w = __popcll(same & ((1ull << lane) - 1ull));
    if (v < E && rank_w == 0) s_wcnt[wave * E + v] = __popcll(same);
    __syncthreads();
    if (tid < E) {                                // prefix of the wave counts, in wave order
        int run = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int t = s_wcnt[w * E + tid];
            s_wcnt[w * E + tid] = run;
            run += t;
        }
    }
    const int c = tid < E ? s_all[tid] : 0;
    int total_rows;
    const int row0 = block_exclusive_scan(c, s_wsum, total_rows);
    if (tid < E) s_first[tid] = row0 + s_before[tid];
    if (writer) {
        if (tid < E) o.counts[tid] = c;
        write_tasks(c, row0, E, o.n_blocks, o.chunk, o.offsets, o.cursors, o.tasks, o.ntasks,
                    o.queue, s_hist, s_wsum);
        if (o.tasks2) {                           // a second list over the same chunks
            __syncthreads();
            s_hist[tid] = 0;
            __syncthreads();
            write_tasks(c, row0, E, o.n_blocks2, o.chunk, o.offsets, o.cursors, o.tasks2,
                        o.ntasks2, o.queue2, s_hist, s_wsum);
        }
    }
    __syncthreads();
    if (r < R) {
        const int slot = v < E ? s_first[v] + s_wcnt[wave * E + v] + rank_w : -1;
        if (slot >= 0) o.sorted_route_ids[slot] = r;
        if (o.route_slots) o.route_slots[r] = slot;
    }
}

__global__ __launch_bounds__(kThreads) void layout_wide_kernel(const int32_t* __restrict__ ids,
                                                               int R, int E, WideLayoutOut o) {
    __shared__ int s_all[kThreads];               // routes per expert, whole batch
    __shared__ int s_before[kThreads];            // routes per expert in the chunks before this one
    __shared__ int s_first[kThreads];             // this chunk's first slot in each segment
    __shared__ int s_hist[kThreads];
    __shared__ int s_wsum[kWaves + 1];
    __shared__ int s_wcnt[kWaves * kThreads];     // [wave][expert]: count, then wave prefix
    const int tid = threadIdx.x;
    const int cb = blockIdx.x * kThreads;         // the chunk's first route
    const int r = cb + tid;
    // this route's id and the first batch of the whole-batch histogram's ids go out together,
    // ahead of the LDS clearing (kU loads in flight per thread ahead of their LDS atomics)
    constexpr int kU = 8;
    const int e = r < R ? ids[r] : -1;
    int q[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int rr = u * kThreads + tid;
        q[u] = rr < R ? ids[rr] : -1;
    }
    s_all[tid] = 0;
    s_before[tid] = 0;
    s_hist[tid] = 0;
    for (int i = tid; i < kWaves * E; i += kThreads) s_wcnt[i] = 0;
    __syncthreads();
    // histograms of the whole batch and of the routes before this chunk
    for (int r0 = 0;;) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if ((unsigned)q[u] < (unsigned)E) {
                atomicAdd(&s_all[q[u]], 1);
                if (r0 + u * kThreads + tid < cb) atomicAdd(&s_before[q[u]], 1);
            }
        }
        r0 += kU * kThreads;
        if (r0 >= R) break;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int rr = r0 + u * kThreads + tid;
            q[u] = rr < R ? ids[rr] : -1;
        }
    }
    wide_place(e, r, R, E, blockIdx.x == 0, o, s_all, s_before, s_first, s_hist, s_wsum,
               s_wcnt);
}

}  // namespace

hipError_t launch_layout(const int32_t* ids, int M, int k, int E, int n_blocks, int chunk_rows,
                         int32_t* counts, int32_t* offsets, int32_t* cursors, moe_task* tasks,
                         int max_tasks, int32_t* ntasks, uint32_t* queue,
                         int32_t* sorted_route_ids, int32_t* route_slots, hipStream_t s) {
    (void)max_tasks;  // capacity checked on the host against moe_max_tasks
    hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(kThreads), 0, s, ids, M * k, E, n_blocks,
                       chunk_rows, counts, offsets, cursors, tasks, ntasks, queue,
                       sorted_route_ids, route_slots, 0, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_layout2(const int32_t* ids, int M, int k, int E, int chunk_rows,
                          int32_t* counts, int32_t* offsets, int32_t* cursors, int n_blocks,
                          moe_task* tasks, int32_t* ntasks, uint32_t* queue, int n_blocks2,
                          moe_task* tasks2, int32_t* ntasks2, uint32_t* queue2, hipStream_t s) {
    hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(kThreads), 0, s, ids, M * k, E, n_blocks,
                       chunk_rows, counts, offsets, cursors, tasks, ntasks, queue, nullptr,
                       nullptr, n_blocks2, tasks2, ntasks2, queue2);
    return hipGetLastError();
}

hipError_t launch_layout_sorted_wide(const int32_t* ids, int M, int k, int E, int n_blocks,
                                     int chunk_rows, int32_t* counts, int32_t* offsets,
                                     int32_t* cursors, moe_task* tasks, int32_t* ntasks,
                                     uint32_t* queue, int32_t* sorted_route_ids, hipStream_t s,
                                     int32_t* route_slots, int n_blocks2, moe_task* tasks2,
                                     int32_t* ntasks2, uint32_t* queue2) {
    const int R = M * k;
    if (R == 0) return hipSuccess;
    const unsigned grid = (unsigned)((R + kThreads - 1) / kThreads);
    const WideLayoutOut o{counts,  offsets, cursors,   tasks,      ntasks,  queue,  sorted_route_ids,
                          route_slots, n_blocks, chunk_rows, tasks2, ntasks2, queue2, n_blocks2};
    hipLaunchKernelGGL(layout_wide_kernel, dim3(grid), dim3(kThreads), 0, s, ids, R, E, o);
    return hipGetLastError();
}

hipError_t launch_counts(const int32_t* ids, int M, int k, int E, int32_t* counts,
                         int32_t* offsets, hipStream_t s) {
    hipLaunchKernelGGL(counts_kernel, dim3(1), dim3(kThreads), 0, s, ids, M * k, E, counts,
                       offsets);
    return hipGetLastError();
}

}  // namespace moe
