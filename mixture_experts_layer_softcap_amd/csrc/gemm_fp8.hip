// gemm_fp8.hip -- grouped FP8 GEMM against 128x128 block-scaled expert weights, with the
// persistent atomic task queue and the routed-row epilogue
// ([FMF8] "Baseline: 7 kernels" item 6 and its listing (empty experts skipped, per-K-block
// scaling, zero-filled partial tiles); Phase 4 grid swap; Phase 5 scale-load overlap;
// "Future compiler improvements" rescale-accumulator discussion; [WEAVE] sections 2.2 and
// 4.2: a fixed grid pulls (expert, token_begin, token_num) tasks from an atomic counter).
//
// gfx950 design.  At the pages' small-batch shape every expert holds ~4 routed rows, so the
// op streams ~256 MiB of FP8 weights once and is bound by HBM, not by the matrix cores.
//  * MFMA: V_MFMA_F32_16X16X128_F8F6F4 with the weights as the 16-row A side (16 output
//    columns n) and up to 16 routed rows as the B side.  One instruction spans exactly one
//    128-wide scale block, so the block scaling is one fp32 FMA per output:
//    acc += (sa[row] * sb) * mfma(w_block, a_block, 0).
//  * Each lane feeds 32 bytes of k to the MFMA.  A and B are loaded with the same byte->k
//    assignment (lane group g = lane/16 takes bytes [16g,16g+16) and [64+16g,64+16g+16) of
//    the block), so the dot product is correct whatever order the hardware uses inside the
//    instruction, and each wave load reads 16 rows x 64 contiguous bytes.
//  * Workgroup = 8 waves = one 128-column weight panel of one task; wave w owns columns
//    [16w, 16w+16).  Waves never exchange data: the B rows come straight from L2/L1.
//  * Each wave keeps a ring of D (task, k-block) units in flight in registers and walks the
//    units of all its tasks as one stream, so the next task's weight loads are in flight
//    while the current task finishes and writes its epilogue.
//  * Scheduling: a persistent grid; with a queue, workgroups take task indices from an
//    atomic counter two tasks ahead (published through LDS at each task boundary); without
//    one they walk the list with a fixed stride.  The last workgroup out resets the queue.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

struct TaskP {
    int valid;
    int e, rb, rc, nb;
};

template <int CG>
struct Slot {
    uint4 w0, w1;
    uint4 b0[CG], b1[CG];
    float sa[CG];
    float sb;
};

__device__ __forceinline__ v8i pack(uint4 lo, uint4 hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// Task descriptors are wave-uniform: the index goes through readfirstlane so the descriptor
// (and the weight block scales) come through the scalar cache, whose counter is separate
// from the vector loads in flight -- waiting for a descriptor never drains the weight ring.
__device__ __forceinline__ TaskP load_task(const int4* __restrict__ tasks, int idx, int nt) {
    idx = __builtin_amdgcn_readfirstlane(idx);
    TaskP p;
    p.valid = idx < nt;
    if (p.valid) {
        const int4 t = tasks[idx];
        p.e = t.x; p.rb = t.y; p.rc = t.z; p.nb = t.w;
    } else {
        // a safe stand-in (expert 0, panel 0, routed row 0): the issue side keeps loading
        // through it after the last task so that every unit issues the same loads; those
        // units are never consumed
        p.e = 0; p.rb = 0; p.rc = 1; p.nb = 0;
    }
    return p;
}

struct Ctx {
    const uint8_t* __restrict__ a;
    const float* __restrict__ a_scales;
    const uint8_t* __restrict__ w;
    const float* __restrict__ w_scales;
    int rows, K, N, KB;
    int wave, j, g;
};

template <int CG>
__device__ __forceinline__ void issue(const Ctx& C, Slot<CG>& s, const TaskP& p, int kb) {
    const int n = p.nb * 128 + C.wave * 16 + C.j;
    const uint8_t* wp = C.w + ((size_t)p.e * C.N + n) * C.K + kb * 128 + C.g * 16;
    s.w0 = *reinterpret_cast<const uint4*>(wp);
    s.w1 = *reinterpret_cast<const uint4*>(wp + 64);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        // Lanes of routed rows past the task re-load row rb (always valid).  Their values
        // only reach MFMA output column j, which the epilogue never stores, so they need no
        // masking; keeping the loads unconditional gives every unit the same number of vector
        // memory operations, which lets the compiler wait for exactly the unit it consumes.
        const int r = c * 16 + C.j;
        const int row = p.rb + (r < p.rc ? r : 0);
        const uint8_t* ap = C.a + (size_t)row * C.K + kb * 128 + C.g * 16;
        s.b0[c] = *reinterpret_cast<const uint4*>(ap);
        s.b1[c] = *reinterpret_cast<const uint4*>(ap + 64);
        s.sa[c] = C.a_scales[(size_t)kb * C.rows + row];
    }
    s.sb = C.w_scales[((size_t)p.e * (C.N >> 7) + p.nb) * C.KB + kb];
}

template <int CG>
__device__ __forceinline__ void consume(const Slot<CG>& s, v4f (&acc)[CG]) {
    const v8i wa = pack(s.w0, s.w1);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        const v8i xb = pack(s.b0[c], s.b1[c]);
        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
        const v4f h = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, zero, 0, 0, 0,
                                                                        0, 0, 0);
        const float f = s.sa[c] * s.sb;
        acc[c] += f * h;
    }
}

template <int CG>
__device__ __forceinline__ void load_routes(const Ctx& C, const int32_t* __restrict__ sorted,
                                            const TaskP& p, int (&route)[CG]) {
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        const int r = c * 16 + C.j;
        route[c] = sorted[p.rb + (r < p.rc ? r : 0)];
    }
}

// C layout of the 16x16 MFMA: lane (j = lane%16, g = lane/16) holds rows 4g..4g+3 of column
// j.  Rows are weight columns n, columns are routed rows, so a lane owns 4 consecutive n of
// one routed row and writes them as one 16-byte (f32) or 8-byte (bf16) store.
template <int EPI, int CG>
__device__ __forceinline__ void epilogue(const Ctx& C, void* __restrict__ out,
                                         const TaskP& p, const v4f (&acc)[CG],
                                         const int (&route)[CG]) {
    const int n0 = p.nb * 128 + C.wave * 16 + C.g * 4;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        const int r = c * 16 + C.j;
        if (r >= p.rc) continue;
        const size_t row = EPI == MOE_EPI_ROUTE_F32 ? (size_t)route[c] : (size_t)(p.rb + r);
        if (EPI == MOE_EPI_STORE_BF16) {
            uint2 v;
            v.x = f32_to_bf16(acc[c][0]) | (f32_to_bf16(acc[c][1]) << 16);
            v.y = f32_to_bf16(acc[c][2]) | (f32_to_bf16(acc[c][3]) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * C.N + n0) = v;
        } else {
            const float4 v = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
            *reinterpret_cast<float4*>(static_cast<float*>(out) + row * C.N + n0) = v;
        }
    }
}

// Task sequence of one workgroup: position 0 is task blockIdx.x; later positions are
// blockIdx.x + i*G (fixed stride, DYN = false) or G + a ticket from the atomic queue
// (DYN = true).  In queue mode a ninth "scheduler" wave owns the queue: it fetches tickets
// ahead and publishes position i+1 in LDS before the barrier that ends position i-1, so the
// eight compute waves never wait on an atomic (a returning atomic would make them wait for
// their whole ring of weight loads).
template <int D, int CG, int EPI, bool DYN>
__global__ __launch_bounds__(DYN ? kThreads + 64 : kThreads)
__attribute__((amdgpu_waves_per_eu(DYN ? 3 : 2, DYN ? 3 : 2)))
void gemm_fp8_kernel(const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
                     const uint8_t* __restrict__ w, const float* __restrict__ w_scales,
                     const int4* __restrict__ tasks, const int32_t* __restrict__ ntasks,
                     uint32_t* __restrict__ queue, const int32_t* __restrict__ sorted_route_ids,
                     void* __restrict__ out, int rows, int K, int N) {
    __shared__ int s_tick[3];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nt = *ntasks;
    const int G = gridDim.x;
    const int first = blockIdx.x;
    const bool any = first < nt;

    if (DYN && wave == kWaves) {
        // ---- scheduler wave ----------------------------------------------------------
        if (any) {
            uint32_t pend = 0;
            if (lane == 0) {
                const uint32_t t = atomicAdd(&queue[0], 2u);
                s_tick[1] = (int)min((uint32_t)G + t, (uint32_t)nt);
                pend = min((uint32_t)G + t + 1u, (uint32_t)nt);
            }
            __syncthreads();                                   // B0: position 1 known
            for (int ci = 0;; ++ci) {
                if (lane == 0) s_tick[(ci + 2) % 3] = (int)pend;
                __syncthreads();                               // end of position ci
                if (s_tick[(ci + 1) % 3] >= nt) break;         // compute waves stop too
                if (lane == 0)
                    pend = (s_tick[(ci + 2) % 3] < nt)
                               ? min((uint32_t)G + atomicAdd(&queue[0], 1u), (uint32_t)nt)
                               : (uint32_t)nt;
            }
        }
    } else if (any) {
        // ---- compute waves -----------------------------------------------------------
        Ctx C{a, a_scales, w, w_scales, rows, K, N, K >> 7, wave, lane & 15, lane >> 4};
        const int KB = C.KB;
        auto task_no = [&](int i) -> int {
            if (i == 0) return first;
            return DYN ? s_tick[i % 3] : first + i * G;
        };

        TaskP pc = load_task(tasks, first, nt);  // consume side
        TaskP pi = pc;                           // issue side
        int ii = 0, ikb = 0;                     // issue cursor (sequence position, k-block)
        int ckb = 0;                             // consume cursor k-block
        bool published = !DYN;

        Slot<CG> ring[D];
        v4f acc[CG];
        int route[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            route[c] = 0;
        }
        auto advance_issue = [&]() {
            if (++ikb == KB) {
                if (!published) {
                    __syncthreads();                           // B0
                    published = true;
                }
                ikb = 0;
                ++ii;
                pi = load_task(tasks, task_no(ii), nt);
            }
        };

        // the first D units of task 0 go out before anything waits
#pragma unroll
        for (int s = 0; s < D; ++s) {
            issue<CG>(C, ring[s], pi, ikb);
            advance_issue();
        }
        if (!published) {
            __syncthreads();                                   // B0
            published = true;
        }
        if (EPI == MOE_EPI_ROUTE_F32) load_routes<CG>(C, sorted_route_ids, pc, route);
        for (;;) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                consume<CG>(ring[s], acc);
                if (++ckb == KB) {
                    epilogue<EPI, CG>(C, out, pc, acc, route);
#pragma unroll
                    for (int c = 0; c < CG; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                    ckb = 0;
                    if (DYN) __syncthreads();                  // end of this position
                    pc = pi;                                   // issue side is already there
                    if (!pc.valid) break;
                    if (EPI == MOE_EPI_ROUTE_F32)
                        load_routes<CG>(C, sorted_route_ids, pc, route);
                }
                issue<CG>(C, ring[s], pi, ikb);
                if (pi.valid) advance_issue();
            }
            if (!pc.valid) break;
        }
    }

    if (DYN) {
        // every wave of the workgroup gets here; the last workgroup out resets the queue
        __syncthreads();
        if (threadIdx.x == 0) {
            if (atomicAdd(&queue[1], 1u) == gridDim.x - 1u) {
                queue[0] = 0u;
                queue[1] = 0u;
            }
        }
    }
}

struct LaunchArgs {
    const uint8_t* a;
    const float* a_scales;
    const uint8_t* w;
    const float* w_scales;
    const moe_task* tasks;
    const int32_t* ntasks;
    uint32_t* queue;
    const int32_t* sorted_route_ids;
    void* out;
    int rows, K, N, epilogue;
};

template <int D, int CG, int EPI>
hipError_t launch_dce(const LaunchArgs& A, int grid, hipStream_t s) {
    const int4* t = reinterpret_cast<const int4*>(A.tasks);
    if (A.queue) {
        hipLaunchKernelGGL((gemm_fp8_kernel<D, CG, EPI, true>), dim3(grid), dim3(kThreads + 64),
                           0, s, A.a, A.a_scales, A.w, A.w_scales, t, A.ntasks, A.queue,
                           A.sorted_route_ids, A.out, A.rows, A.K, A.N);
    } else {
        hipLaunchKernelGGL((gemm_fp8_kernel<D, CG, EPI, false>), dim3(grid), dim3(kThreads), 0,
                           s, A.a, A.a_scales, A.w, A.w_scales, t, A.ntasks, A.queue,
                           A.sorted_route_ids, A.out, A.rows, A.K, A.N);
    }
    return hipGetLastError();
}

template <int D, int CG>
hipError_t launch_dc(const LaunchArgs& A, int grid, hipStream_t s) {
    switch (A.epilogue) {
        case MOE_EPI_STORE_BF16: return launch_dce<D, CG, MOE_EPI_STORE_BF16>(A, grid, s);
        case MOE_EPI_ROUTE_F32: return launch_dce<D, CG, MOE_EPI_ROUTE_F32>(A, grid, s);
        default: return launch_dce<D, CG, MOE_EPI_STORE_F32>(A, grid, s);
    }
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* a, const float* a_scales, int rows, int K,
                           const uint8_t* w, const float* w_scales, int E, int N,
                           const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                           int chunk_rows, uint32_t* queue, int epilogue,
                           const int32_t* sorted_route_ids, void* out, hipStream_t s) {
    (void)E;
    if (max_tasks <= 0) return hipSuccess;
    if (gemm_fp8_range_applies(K, chunk_rows))
        return launch_gemm_fp8_range(a, a_scales, rows, K, w, w_scales, N, tasks, ntasks,
                                     max_tasks, epilogue, sorted_route_ids, out, s);
    if (gemm_fp8_tile_applies(K, chunk_rows))
        return launch_gemm_fp8_tile(a, a_scales, rows, K, w, w_scales, N, tasks, ntasks,
                                    max_tasks, chunk_rows, epilogue, sorted_route_ids, out, s);
    LaunchArgs A{a, a_scales, w, w_scales, tasks, ntasks, queue, sorted_route_ids, out,
                 rows, K, N, epilogue};
    int grid = device_info().cu_count;      // one 8-wave workgroup per CU
    if (grid > max_tasks) grid = max_tasks;
    const int KB = K / 128;
    // ring depth D may not exceed the k-blocks of one task (the issue side then runs at most
    // one task ahead); column groups CG cover the task's routed rows 16 at a time
    const int cg = (chunk_rows + 15) / 16;
    if (cg <= 1) {
        if (KB >= 8) return launch_dc<8, 1>(A, grid, s);
        if (KB >= 4) return launch_dc<4, 1>(A, grid, s);
        if (KB >= 2) return launch_dc<2, 1>(A, grid, s);
        return launch_dc<1, 1>(A, grid, s);
    }
    if (cg == 2) {
        if (KB >= 4) return launch_dc<4, 2>(A, grid, s);
        if (KB >= 2) return launch_dc<2, 2>(A, grid, s);
        return launch_dc<1, 2>(A, grid, s);
    }
    // four column groups: a depth-4 ring fits only without the scheduler wave
    if (KB >= 4 && !queue) return launch_dc<4, 4>(A, grid, s);
    if (KB >= 2) return launch_dc<2, 4>(A, grid, s);
    return launch_dc<1, 4>(A, grid, s);
}

}  // namespace moe
