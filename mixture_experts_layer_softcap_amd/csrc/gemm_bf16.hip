// gemm_bf16.hip -- grouped BF16 GEMM for large routed-row counts ([H200] gated-up and down
// projections over compact routed rows; [WEAVE] Mixtral-like layer, sections 2.2 and 4.2
// for the task list).  h[r][n] = sum_k a[r][k] * w[e][n][k], bf16 operands, fp32 accumulate.
//
// Tile.  One workgroup computes a 256-row x 256-column tile of one task (expert e, sorted rows
// [rb, rb+rc) with rc <= 256, 256-column panel nb) and walks K in steps of 64.  Four waves
// in a 2 x 2 layout each own 128 rows x 128 columns: 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane (AGPRs), one wave per SIMD.  The
// weights are the MFMA's A side (32 output columns), the routed rows its B side (32 rows),
// so a lane holds, for one routed row, runs of 4 consecutive output columns.  Per 16-wide k
// step a wave reads 8 operand fragments for 16 MFMAs.
//
// Operands.  Both tiles go from global memory straight into LDS with global_load_lds_dwordx4:
// one instruction moves 8 whole 128-byte row segments (64 k values of 8 rows), each 16-byte
// chunk c of row r stored at position c ^ ((r/2) % 8), so the DMA reads whole cache lines and
// the MFMA fragment reads are free of LDS bank conflicts.  The routed rows have two stages
// of 32 KiB and the weights three (all 160 KiB of LDS): the weight DMA runs two k steps
// ahead, the row DMA one; one barrier per k step publishes a stage and frees the oldest.  The
// DMA instructions go out between the first half of the current stage's MFMAs, and each 16-wide
// step's fragments are read during the previous step's MFMAs.  Every stage is a __shared__
// object of its own, read by plain element indexing, and the k loop is unrolled over the six
// (row stage, weight stage) phases: the compiler then tells a DMA into one stage from reads
// of another and places each wait for exactly the data a read needs.
// Rows past rc repeat row rb + rc - 1 (never stored).  With a sorted route list the A rows
// are gathered on load: sorted row s is token row sorted[s] / k of the layer input, so no
// expert-sorted copy of the input is written first.
//
// Order.  Workgroups go round-robin over the 8 XCDs; each XCD takes one contiguous run of the
// chunk-major task list, regrouped so that the tiles it runs together cover a few chunks x a
// few panels (fewer distinct operand slices per k step in its L2).  How tiles reach
// workgroups is one of the MOE_SCHED_* schedules: hardware dispatch of one workgroup per tile,
// a static persistent walk of the XCD's run, one atomic queue over the regrouped list, or
// per-XCD atomic queues over each XCD's run ([WEAVE] sections 1.2, 2.2 and 4.2).
//
// Epilogues.  STORE_F32 / STORE_BF16 write h; SWIGLU_BF16 computes a 128-column block of
// act = bf16(silu(g) * u) from the gate columns [nb*128, nb*128+128) and the up columns
// [N/2 + nb*128, ...) of the same task (each wave holds 64 gate columns and their up columns).
#include "moe_device.h"
#include "moe_internal.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most VM vector-memory operations of this wave are outstanding and all its LDS
// operations are done, then barrier.  LDS DMA decrements vmcnt once its data is in LDS, so
// the stage it waits for is visible to every wave after the barrier.
template <int VM>
__device__ __forceinline__ void barrier_after_vmcnt() {
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

using T = std::true_type;
template <int I>
using IC = std::integral_constant<int, I>;

// Position of the tile a workgroup runs for slot q of XCD x's run of the task list (nt tasks,
// nbk per chunk): the run is regrouped into groups of gch chunks, taken pw panels at a time.
struct TileOrder {
    int nt, nbk, per_xcd, pw, gch;
    // task of position t of the (regrouped) list, t < nt
    __device__ int task_at(int t) const {
        const int grp = t / (gch * nbk);
        const int gc = min(gch, nt / nbk - grp * gch);
        int i = t - grp * gch * nbk;
        const int pb = i / (gc * pw);
        const int pwb = min(pw, nbk - pb * pw);
        i -= pb * gc * pw;
        return (grp * gch + i / pwb) * nbk + pb * pw + i % pwb;
    }
    __device__ int xcd_count(int x) const { return max(0, min(per_xcd, nt - x * per_xcd)); }
};

template <int EPI, int SCHED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
                      const int4* __restrict__ tasks, const int32_t* __restrict__ ntasks,
                      void* __restrict__ out, int K, int N, int pw, int gch,
                      const int32_t* __restrict__ sorted, int kr, uint32_t* __restrict__ queue) {
    // routed rows: 2 stages x 256 rows x 128 bytes; weights: three stages
    __shared__ uint4 sA0[kBM * 8], sA1[kBM * 8];
    __shared__ uint4 sW0[kBN * 8], sW1[kBN * 8], sW2[kBN * 8];
    auto stA = [&](auto bi) __attribute__((always_inline)) -> uint4* {
        if constexpr (decltype(bi)::value == 0) return sA0;
        else return sA1;
    };
    auto stW = [&](auto bi) __attribute__((always_inline)) -> uint4* {
        if constexpr (decltype(bi)::value == 0) return sW0;
        else if constexpr (decltype(bi)::value == 1) return sW1;
        else return sW2;
    };
    const int nt = *ntasks;
    const int nbk = N / kBN;                    // tasks per chunk (both epilogue layouts)
    const TileOrder ord{nt, nbk, (nt + 7) >> 3, pw, gch};
    const int xcd = (int)(blockIdx.x & 7);
    const int slot = (int)(blockIdx.x >> 3);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int j = lane & 31, h = lane >> 5;
    const int nk = K / kBK;
    const int dl = lane >> 3;                   // row within a DMA instruction

    // Fragment positions (uint4 elements), per 16-wide k step st: row j of a 32-row group, chunk
    // 2st + h at its swizzled position; A groups 4wm.., W groups of this wave ((4wn..) or, for
    // SwiGLU, gate groups 2wn, 2wn+1 and up groups 4+2wn, 5+2wn)
    const int wg0 = EPI == MOE_EPI_SWIGLU_BF16 ? 2 * wn : 4 * wn;
    const int wg2 = EPI == MOE_EPI_SWIGLU_BF16 ? 4 + 2 * wn : 4 * wn + 2;
    int pa[4], pw0[4], pw2[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int in_row = j * 8 + ((2 * st + h) ^ ((j >> 1) & 7));
        pa[st] = (4 * wm) * 256 + in_row;
        pw0[st] = wg0 * 256 + in_row;
        pw2[st] = wg2 * 256 + in_row;
    }

    // one 256 x 256 tile: task (e, rb, rc, nb)
    auto run_tile = [&](int task) __attribute__((always_inline)) {
        const int4 td = tasks[task];
        const int e = td.x, rb = td.y, rc = td.z, nb = td.w;
        // Operand tiles in LDS, per stage: [256 rows][128 bytes] for A and for W (the stage's 64
        // k values of each row), the 16-byte chunk c of row r stored at position c ^ ((r/2) % 8).
        // A DMA instruction moves 8 whole 128-byte row segments (lane l: row l/8, position l%8);
        // every line it touches is read in full.  The LDS serves a 16-byte read for 16 lanes per
        // clock over 64 four-byte banks, i.e. two 128-byte rows side by side: an MFMA fragment
        // read (lanes j..j+15 of one half h: rows g*32 + j, one chunk 2s + h) then has rows of
        // equal parity at 8 distinct positions, so it is free of bank conflicts.
        const uint16_t* srcA[8];
        const uint16_t* srcW[8];
        // A row of tile row r: sorted row rb + r, or with a sorted route list the token row it
        // was routed from (the eight lookups issued together)
        int arow[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) arow[i] = rb + min(wave * 64 + i * 8 + dl, rc - 1);
        if (sorted) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = sorted[arow[i]];
#pragma unroll
            for (int i = 0; i < 8; ++i) arow[i] = v[i] / kr;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wave * 64 + i * 8 + dl;   // tile row moved by this lane
            const int dc = (lane & 7) ^ ((r >> 1) & 7);   // global 16-byte chunk this lane moves
            srcA[i] = a + (size_t)arow[i] * K + dc * 8;
            int wr;
            if (EPI == MOE_EPI_SWIGLU_BF16)
                wr = r < 128 ? nb * 128 + r : N / 2 + nb * 128 + (r - 128);
            else
                wr = nb * kBN + r;
            srcW[i] = w + ((size_t)e * N + wr) * K + dc * 8;
        }

        f32x16 acc[4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

        struct Frag {
            uint4 a[4], w[4];
        };
        auto read_frags = [&](Frag& f, const uint4* A, const uint4* W, int st)
                              __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) f.a[i] = A[pa[st] + i * 256];
            f.w[0] = W[pw0[st]];
            f.w[1] = W[pw0[st] + 256];
            f.w[2] = W[pw2[st]];
            f.w[3] = W[pw2[st] + 256];
        };

        // One k step: stage (BA, BW) holds k step kt; the fragments of 16-wide step st+1 are
        // read while the MFMAs of step st run, and the next k step's 16 DMA instructions (A of
        // kt+1 into stage NA, W of kt+2 into stage NW) go out one after every second MFMA of
        // the step's first half, from the first on: a wave issues in order, and a burst of DMA
        // instructions stalls it on the memory pipeline long enough to hold back its MFMAs,
        // while DMA issued late in the step leaves its latency to the next barrier (one per
        // fourth MFMA over the whole step measured 3-7 % slower, one per third 1-3 % slower).
        auto step = [&](auto ba, auto bw, auto na, auto nw, int kt)
                        __attribute__((always_inline)) {
            // A(kt) and W(kt) have landed; W(kt+1) (the newest 8) may still be in flight.  Past
            // the end the DMA repeats the last stage into a free buffer (never read).
            barrier_after_vmcnt<8>();
            const uint4* A = stA(ba);
            const uint4* W = stW(bw);
            uint4* dA = stA(na);
            uint4* dW = stW(nw);
            const int k0A = min(kt + 1, nk - 1) * kBK, k0W = min(kt + 2, nk - 1) * kBK;
            Frag f[2];
            read_frags(f[0], A, W, 0);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const Frag& c = f[st & 1];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(c.w[ni]), as_bf16x8(c.a[mi]), acc[mi][ni], 0, 0, 0);
                        // the next 16-wide step's fragments are read behind this step's 4th
                        // MFMA: the compiler waits for all outstanding LDS reads before the
                        // next step's first MFMA, by which time 12 MFMAs have covered them
                        if (st < 3 && mi == 0 && ni == 3) read_frags(f[(st + 1) & 1], A, W, st + 1);
                        const int m = st * 16 + mi * 4 + ni;     // MFMA index in the step
                        if (m % 2 == 0 && m / 2 < 16) {
                            const int q = m / 2;                 // DMA slot 0..15
                            if (q < 8)
                                __builtin_amdgcn_global_load_lds(
                                    srcA[q] + k0A, (lds_void*)(dA + (wave * 64 + q * 8) * 8), 16,
                                    0, 0);
                            else
                                __builtin_amdgcn_global_load_lds(
                                    srcW[q - 8] + k0W,
                                    (lds_void*)(dW + (wave * 64 + (q - 8) * 8) * 8), 16, 0, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        };

        // Weights run two steps ahead (three stages), routed rows one (two stages): k step kt
        // reads A stage kt%2 and W stage kt%3 and refills A stage (kt+1)%2 and W stage
        // (kt+2)%3.  The six phases of (kt%2, kt%3) are unrolled so that every stage is named
        // at compile time; a remainder of nk%6 steps runs the first phases behind run-time
        // guards.
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(srcA[i], (lds_void*)(sA0 + (wave * 64 + i * 8) * 8),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(srcW[i], (lds_void*)(sW0 + (wave * 64 + i * 8) * 8),
                                             16, 0, 0);
        {
            const int k1 = min(1, nk - 1) * kBK;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_global_load_lds(srcW[i] + k1,
                                                 (lds_void*)(sW1 + (wave * 64 + i * 8) * 8), 16,
                                                 0, 0);
        }
        int kt = 0;
        for (; kt + 6 <= nk; kt += 6) {
            step(IC<0>{}, IC<0>{}, IC<1>{}, IC<2>{}, kt);
            step(IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{}, kt + 1);
            step(IC<0>{}, IC<2>{}, IC<1>{}, IC<1>{}, kt + 2);
            step(IC<1>{}, IC<0>{}, IC<0>{}, IC<2>{}, kt + 3);
            step(IC<0>{}, IC<1>{}, IC<1>{}, IC<0>{}, kt + 4);
            step(IC<1>{}, IC<2>{}, IC<0>{}, IC<1>{}, kt + 5);
        }
        if (kt < nk) step(IC<0>{}, IC<0>{}, IC<1>{}, IC<2>{}, kt);
        if (kt + 1 < nk) step(IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{}, kt + 1);
        if (kt + 2 < nk) step(IC<0>{}, IC<2>{}, IC<1>{}, IC<1>{}, kt + 2);
        if (kt + 3 < nk) step(IC<1>{}, IC<0>{}, IC<0>{}, IC<2>{}, kt + 3);
        if (kt + 4 < nk) step(IC<0>{}, IC<1>{}, IC<1>{}, IC<0>{}, kt + 4);
        // no DMA may still write this workgroup's LDS when it stores or takes the next tile
        barrier_after_vmcnt<0>();

        // C layout of the 32x32 MFMA: lane (j, h) holds column j (routed row) and, in register
        // r, output row 8*(r/4) + 4*h + r%4 of the 32-row weight group
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int m = (4 * wm + mi) * 32 + j;
            if (m >= rc) continue;
            const size_t row = (size_t)(rb + m);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = 8 * q + 4 * h;       // 4 consecutive output columns
                if (EPI == MOE_EPI_SWIGLU_BF16) {
                    const int Nh = N / 2;
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        uint32_t p[2];
#pragma unroll
                        for (int c = 0; c < 4; c += 2) {
                            float v[2];
#pragma unroll
                            for (int d = 0; d < 2; ++d) {
                                const float g = acc[mi][ni][4 * q + c + d];
                                const float u = acc[mi][ni + 2][4 * q + c + d];
                                v[d] = g / (1.0f + __expf(-g)) * u;
                            }
                            p[c / 2] = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
                        }
                        const int n = nb * 128 + (2 * wn + ni) * 32 + nl;
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * Nh + n) =
                            make_uint2(p[0], p[1]);
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const int n = nb * kBN + (4 * wn + ni) * 32 + nl;
                        const f32x16& c = acc[mi][ni];
                        if (EPI == MOE_EPI_STORE_BF16) {
                            const uint32_t p0 =
                                f32_to_bf16(c[4 * q]) | (f32_to_bf16(c[4 * q + 1]) << 16);
                            const uint32_t p1 =
                                f32_to_bf16(c[4 * q + 2]) | (f32_to_bf16(c[4 * q + 3]) << 16);
                            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * N + n) =
                                make_uint2(p0, p1);
                        } else {
                            *reinterpret_cast<float4*>(static_cast<float*>(out) + row * N + n) =
                                make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
                        }
                    }
                }
            }
        }
    };

    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs, so workgroup b
    // runs on XCD b%8; each XCD takes one contiguous run of the (chunk-major) task list, so the
    // tiles running together on an XCD share routed-row chunks and weight panels, and walk K
    // in near lockstep, out of that XCD's L2.  Inside a run, gch consecutive chunks (same
    // expert where possible) are taken pw panels at a time: the ~32 tiles an XCD runs together
    // then cover gch chunks x pw panels, so each k step asks its L2 for gch + pw distinct
    // slices instead of ~3 + N/256.
    if constexpr (SCHED == MOE_SCHED_DISPATCH) {
        if (slot >= ord.per_xcd) return;
        const int t = xcd * ord.per_xcd + slot;
        if (t >= nt) return;
        run_tile(ord.task_at(t));
    } else {
        const int cus_x = (int)(gridDim.x >> 3);
        int victim = 0;                            // QUEUE_XCD: the run being drained
        auto next_ticket = [&]() -> int {          // thread 0 only; a list position or -1
            if (SCHED == MOE_SCHED_QUEUE) {
                const int t = (int)atomicAdd(&queue[0], 1u);
                return t < nt ? t : -1;
            }
            for (; victim < 8; ++victim) {
                const int x = (xcd + victim) & 7;
                const int n = ord.xcd_count(x);
                if (n <= 0) continue;
                const int t = (int)atomicAdd(&queue[x], 1u);
                if (t < n) return x * ord.per_xcd + t;
            }
            return -1;
        };
        // A ticket is published in the first word of weight stage 2: all 160 KiB of LDS hold
        // operand stages, and stage 2 is idle between two tiles (the next tile first writes
        // it after its first barrier, which every wave reaches only after reading the ticket).
        auto publish = [&]() -> int {
            if (threadIdx.x == 0) sW2[0].x = (uint32_t)next_ticket();
            __syncthreads();
            return (int)sW2[0].x;
        };
        int cur;
        if (SCHED == MOE_SCHED_STATIC)
            cur = slot < ord.xcd_count(xcd) ? xcd * ord.per_xcd + slot : -1;
        else
            cur = publish();
        int iter = 0;
        while (cur >= 0) {
            run_tile(ord.task_at(cur));
            ++iter;
            if (SCHED == MOE_SCHED_STATIC) {
                const int q = slot + iter * cus_x;
                cur = q < ord.xcd_count(xcd) ? xcd * ord.per_xcd + q : -1;
            } else {
                cur = publish();
            }
            if (iter > nt && cur >= 0) {              // cannot happen with a sound counter
                if (SCHED != MOE_SCHED_STATIC && threadIdx.x == 0) atomicOr(&queue[9], 1u);
                break;
            }
        }
        if (SCHED != MOE_SCHED_STATIC && threadIdx.x == 0) {
            if (atomicAdd(&queue[8], 1u) == gridDim.x - 1u) {
#pragma unroll
                for (int i = 0; i < 9; ++i) atomicExch(&queue[i], 0u);
            }
        }
    }
}

template <int EPI>
hipError_t launch_epi(int sched, unsigned grid, const uint16_t* a, const uint16_t* w,
                      const int4* t, const int32_t* ntasks, void* out, int K, int N, int pw,
                      int gch, const int32_t* sorted, int kr, uint32_t* queue, hipStream_t s) {
#define MOE_BF16_ARGS a, w, t, ntasks, out, K, N, pw, gch, sorted, kr, queue
    switch (sched) {
        case MOE_SCHED_STATIC:
            hipLaunchKernelGGL((gemm_bf16_kernel<EPI, MOE_SCHED_STATIC>), dim3(grid),
                               dim3(kThreads), 0, s, MOE_BF16_ARGS);
            break;
        case MOE_SCHED_QUEUE:
            hipLaunchKernelGGL((gemm_bf16_kernel<EPI, MOE_SCHED_QUEUE>), dim3(grid),
                               dim3(kThreads), 0, s, MOE_BF16_ARGS);
            break;
        case MOE_SCHED_QUEUE_XCD:
            hipLaunchKernelGGL((gemm_bf16_kernel<EPI, MOE_SCHED_QUEUE_XCD>), dim3(grid),
                               dim3(kThreads), 0, s, MOE_BF16_ARGS);
            break;
        default:
            hipLaunchKernelGGL((gemm_bf16_kernel<EPI, MOE_SCHED_DISPATCH>), dim3(grid),
                               dim3(kThreads), 0, s, MOE_BF16_ARGS);
    }
#undef MOE_BF16_ARGS
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* a, int K, const uint16_t* w, int N,
                            const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                            int epilogue, void* out, hipStream_t s, const int32_t* sorted,
                            int kr, int sched, uint32_t* queue) {
    if (max_tasks <= 0) return hipSuccess;
    if (sched == MOE_SCHED_AUTO) sched = MOE_SCHED_DISPATCH;
    if ((sched == MOE_SCHED_QUEUE || sched == MOE_SCHED_QUEUE_XCD) && !queue)
        return hipErrorInvalidValue;
    const int4* t = reinterpret_cast<const int4*>(tasks);
    // one workgroup per tile in whole rounds of the 8 XCDs, or one per CU (one fits per CU)
    const unsigned grid = sched == MOE_SCHED_DISPATCH
                              ? (unsigned)((max_tasks + 7) / 8 * 8)
                              : (unsigned)(max(1, device_info().cu_count / 8) * 8);
    // tile groups of ~32 (one XCD's CUs): up to 4 panels x 32/4 chunks (8 x 4 and 12 x 2 were
    // 1-4 % slower with three weight stages)
    const int pw = min(4, N / kBN);
    const int gch = 32 / pw;
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            return launch_epi<MOE_EPI_STORE_BF16>(sched, grid, a, w, t, ntasks, out, K, N, pw,
                                                  gch, sorted, kr, queue, s);
        case MOE_EPI_SWIGLU_BF16:
            return launch_epi<MOE_EPI_SWIGLU_BF16>(sched, grid, a, w, t, ntasks, out, K, N, pw,
                                                   gch, sorted, kr, queue, s);
        default:
            return launch_epi<MOE_EPI_STORE_F32>(sched, grid, a, w, t, ntasks, out, K, N, pw,
                                                 gch, sorted, kr, queue, s);
    }
}

}  // namespace moe
