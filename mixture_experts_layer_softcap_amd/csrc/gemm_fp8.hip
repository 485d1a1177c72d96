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

struct Args {
    const uint8_t* a;        // [rows][K]
    const float* a_scales;   // [K/128][rows]
    const uint8_t* w;        // [E][N][K]
    const float* w_scales;   // [E][N/128][K/128]
    const moe_task* tasks;
    const int32_t* ntasks;
    uint32_t* queue;         // NULL: fixed-stride walk
    const int32_t* sorted_route_ids;
    void* out;
    int rows, K, N, epilogue;
};

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

__device__ __forceinline__ TaskP load_task(const Args& A, int idx, int nt) {
    TaskP p;
    p.valid = idx < nt;
    if (p.valid) {
        const int4 t = *reinterpret_cast<const int4*>(&A.tasks[idx]);
        p.e = t.x; p.rb = t.y; p.rc = t.z; p.nb = t.w;
    } else {
        p.e = p.rb = p.rc = p.nb = 0;
    }
    return p;
}

template <int CG>
__device__ __forceinline__ void issue(const Args& A, Slot<CG>& s, const TaskP& p, int kb,
                                      int wave, int j, int g) {
    if (!p.valid) return;
    const int KB = A.K >> 7;
    const int n = p.nb * 128 + wave * 16 + j;
    const uint8_t* wp = A.w + ((size_t)p.e * A.N + n) * A.K + kb * 128 + g * 16;
    s.w0 = *reinterpret_cast<const uint4*>(wp);
    s.w1 = *reinterpret_cast<const uint4*>(wp + 64);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        const int r = c * 16 + j;
        uint4 b0 = make_uint4(0u, 0u, 0u, 0u), b1 = b0;
        float sa = 0.0f;
        if (r < p.rc) {  // rows past the task are zero-filled, never read
            const uint8_t* ap = A.a + (size_t)(p.rb + r) * A.K + kb * 128 + g * 16;
            b0 = *reinterpret_cast<const uint4*>(ap);
            b1 = *reinterpret_cast<const uint4*>(ap + 64);
            sa = A.a_scales[(size_t)kb * A.rows + p.rb + r];
        }
        s.b0[c] = b0;
        s.b1[c] = b1;
        s.sa[c] = sa;
    }
    s.sb = A.w_scales[((size_t)p.e * (A.N >> 7) + p.nb) * KB + kb];
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

// C layout of the 16x16 MFMA: lane (j = lane%16, g = lane/16) holds rows 4g..4g+3 of column
// j.  Rows are weight columns n, columns are routed rows, so a lane owns 4 consecutive n of
// one routed row and writes them as one 16-byte (f32) or 8-byte (bf16) store.
template <int CG>
__device__ __forceinline__ void epilogue(const Args& A, const TaskP& p, const v4f (&acc)[CG],
                                         const int (&route)[CG], int wave, int j, int g) {
    const int n0 = p.nb * 128 + wave * 16 + g * 4;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        const int r = c * 16 + j;
        if (r >= p.rc) continue;
        const size_t row = A.epilogue == MOE_EPI_ROUTE_F32 ? (size_t)route[c] : (size_t)(p.rb + r);
        if (A.epilogue == MOE_EPI_STORE_BF16) {
            uint2 v;
            v.x = f32_to_bf16(acc[c][0]) | (f32_to_bf16(acc[c][1]) << 16);
            v.y = f32_to_bf16(acc[c][2]) | (f32_to_bf16(acc[c][3]) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(A.out) + row * A.N + n0) = v;
        } else {
            float4 v = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
            *reinterpret_cast<float4*>(static_cast<float*>(A.out) + row * A.N + n0) = v;
        }
    }
}

template <int D, int CG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_fp8_kernel(Args A) {
    __shared__ int s_tick[3];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int KB = A.K >> 7;
    const int nt = *A.ntasks;
    const bool dyn = A.queue != nullptr;
    const int G = gridDim.x;

    // task sequence of this workgroup: index i -> task number
    uint32_t pending = 0;
    if (dyn) {
        if (threadIdx.x == 0) {
            const uint32_t a = atomicAdd(&A.queue[0], 2u);
            s_tick[0] = (int)min(a, (uint32_t)nt);
            s_tick[1] = (int)min(a + 1u, (uint32_t)nt);
            pending = (a + 1u < (uint32_t)nt) ? atomicAdd(&A.queue[0], 1u) : (uint32_t)nt;
        }
        __syncthreads();
    }
    auto task_no = [&](int i) -> int {
        return dyn ? s_tick[i % 3] : (int)blockIdx.x + i * G;
    };

    TaskP pc = load_task(A, task_no(0), nt);     // consume side
    TaskP pi = pc;                               // issue side
    int ii = 0, ikb = 0;                         // issue cursor (task seq index, k-block)
    int ci = 0, ckb = 0;                         // consume cursor

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
            ikb = 0;
            ++ii;
            pi = load_task(A, task_no(ii), nt);
        }
    };

    if (pc.valid) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            issue<CG>(A, ring[s], pi, ikb, wave, j, g);
            advance_issue();
        }
        if (A.epilogue == MOE_EPI_ROUTE_F32) {
#pragma unroll
            for (int c = 0; c < CG; ++c)
                if (c * 16 + j < pc.rc) route[c] = A.sorted_route_ids[pc.rb + c * 16 + j];
        }
        for (;;) {
            bool done = false;
#pragma unroll
            for (int s = 0; s < D; ++s) {
                if (!done) {
                    consume<CG>(ring[s], acc);
                    if (++ckb == KB) {
                        epilogue<CG>(A, pc, acc, route, wave, j, g);
#pragma unroll
                        for (int c = 0; c < CG; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                        ckb = 0;
                        ++ci;
                        if (dyn) {
                            // publish task ci+1 (fetched one task ago), fetch task ci+2
                            if (threadIdx.x == 0) s_tick[(ci + 1) % 3] = (int)pending;
                            __syncthreads();
                            if (threadIdx.x == 0)
                                pending = (pc.valid && s_tick[(ci + 1) % 3] < nt)
                                              ? atomicAdd(&A.queue[0], 1u)
                                              : (uint32_t)nt;
                        }
                        pc = pi;                 // the issue side is already in task ci
                        if (!pc.valid) {
                            done = true;
                        } else if (A.epilogue == MOE_EPI_ROUTE_F32) {
#pragma unroll
                            for (int c = 0; c < CG; ++c)
                                if (c * 16 + j < pc.rc)
                                    route[c] = A.sorted_route_ids[pc.rb + c * 16 + j];
                        }
                    }
                    if (!done) {
                        issue<CG>(A, ring[s], pi, ikb, wave, j, g);
                        if (pi.valid) advance_issue();
                    }
                }
            }
            if (done) break;
        }
    }

    if (dyn) {
        __syncthreads();
        if (threadIdx.x == 0) {
            if (atomicAdd(&A.queue[1], 1u) == gridDim.x - 1u) {
                A.queue[0] = 0u;
                A.queue[1] = 0u;
            }
        }
    }
}

template <int D, int CG>
hipError_t launch_dc(const Args& A, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_fp8_kernel<D, CG>), dim3(grid), dim3(kThreads), 0, s, A);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* a, const float* a_scales, int rows, int K,
                           const uint8_t* w, const float* w_scales, int E, int N,
                           const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                           int chunk_rows, uint32_t* queue, int epilogue,
                           const int32_t* sorted_route_ids, void* out, hipStream_t s) {
    (void)E;
    if (max_tasks <= 0) return hipSuccess;
    Args A{a, a_scales, w, w_scales, tasks, ntasks, queue, sorted_route_ids, out,
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
    if (KB >= 4) return launch_dc<4, 4>(A, grid, s);
    if (KB >= 2) return launch_dc<2, 4>(A, grid, s);
    return launch_dc<1, 4>(A, grid, s);
}

}  // namespace moe
