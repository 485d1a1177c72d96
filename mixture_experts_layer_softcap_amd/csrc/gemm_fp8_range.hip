// gemm_fp8_range.hip -- grouped FP8 GEMM for tasks of at most 16 routed rows and K = 512, 1024
// or 2048: the
// small-batch regime of the pages ([FMF8] problem table, about 4 rows per expert; Baseline
// item 6 with per-K-block scaling; [WEAVE] sections 2.2 and 4.2 for the persistent walk over a
// task list).
//
// Work split.  A task is (expert e, sorted rows [rb, rb+rc), 128-column panel nb), and all
// n_blocks panels of one chunk are consecutive in the list.  A subtask is one 16-column slice
// of a task's panel: 16 weight rows x K bytes, the A operand of one wave.  The subtasks are
// cut into one contiguous range per workgroup (equal counts are equal bytes, and a range of a
// few tasks touches one or two chunks of routed rows); inside the workgroup each wave pulls
// its next subtask from an LDS counter one subtask ahead, so a wave that streams faster does
// more of the range.
//
// Routed rows.  Each chunk's rows (16 x K bytes, the MFMA B operand, shared by all 8 waves)
// and their block scales go from global memory straight into LDS (global_load_lds), in MFMA
// fragment order, for every chunk of the range at once when they fit (4 at K = 2048, 16 at
// K = 512;
// otherwise in rounds).  Wave 0 scans the range and moves the tiles before its own weight
// loads; the barrier that publishes them leaves every wave's first weight burst in flight.
// There is no barrier per task.
//
// Weights.  A subtask is read as units of one k-block (16 rows x 128 bytes: two 16-byte loads
// per lane, lane (j, g) holding bytes [g*16, g*16+16) and [64+g*16, 80+g*16) of row j).  A ring
// of min(MOE_RANGE_RING, K/128) units lives in registers; each unit is refilled right after its MFMA has
// consumed it, with the same k-block of the next pass or of the next subtask, so a wave keeps
// the ring's loads in flight through subtask boundaries.  Weights carry the non-temporal hint.
// Measured on MI355X with this grid: the weight stream alone runs at 6.1 TB/s in this order
// (a fragment-major weight layout is slower), the MFMA consumption and the per-subtask stores
// of the fp32 rows cost 1-2 us each on top, and the compiler's own barriers or a conditional
// load anywhere in a wave's sequence make it drain the ring.
//
// Numerics.  One MFMA (v_mfma_f32_16x16x128_f8f6f4, unscaled) per k-block gives the exact
// dot product of 128 E4M3 pairs up to the unit's internal rounding; it is scaled by
// a_scale[row][kb] * w_scale[panel][kb] and accumulated in fp32, k-block by k-block.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// k-block units in a wave's register ring (8 measured fastest; 4 and 16 are within 1%)
#ifndef MOE_RANGE_RING
#define MOE_RANGE_RING 8
#endif

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRingMax = MOE_RANGE_RING;        // k-block units per wave in registers
constexpr int kTileBudget = 136 * 1024;         // LDS bytes for routed-row tiles

struct TaskD {
    int e, rb, rc, nb;
};

__device__ __forceinline__ TaskD load_task(const int4* __restrict__ tasks, int idx) {
    idx = __builtin_amdgcn_readfirstlane(idx);
    const int4 t = tasks[idx];
    return {t.x, t.y, t.z, t.w};
}

// position of the n-th (0-based) set bit of m; m has more than n set bits
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
    for (int i = 0; i < n; ++i) m &= m - 1;
    return __builtin_ctzll(m);
}

typedef __attribute__((address_space(3))) void lds_void;

template <int KB>
struct TileLds {
    static constexpr int kBytes = KB * 2 * 1024 + KB * 16 * 4;
    static constexpr int kMax = kTileBudget / kBytes;
    uint4 frag[kMax][KB * 2 * 64];              // fragment f = (k-block f/2, half f%2)
    float sa[kMax][KB * 16];                    // [k-block][row]
};

// Routed rows [rb, rb+rc) of a chunk into one LDS tile, moved by one wave.  Fragment f holds,
// for lane (j, g), the 16 bytes at [kb*128 + half*64 + g*16] of routed row j, so a
// wave-wide 16-byte LDS-direct load fills it (lane l lands at base + 16*l) and an MFMA
// operand read is 1 KiB contiguous.  Rows past rc repeat row rb (their output column is never
// stored).  The KB*16 scales ([k-block][row]) follow, one dword per lane.
template <int KB>
__device__ __forceinline__ void tile_dma(const uint8_t* __restrict__ a,
                                         const float* __restrict__ a_scales, int rows, int rb,
                                         int rc, uint4* frag, float* sa, int lane) {
    constexpr int K = KB * 128;
    const int j = lane & 15, g = lane >> 4;
    const int row = rb + (j < rc ? j : 0);
    const uint8_t* src = a + (size_t)row * K + g * 16;
#pragma unroll 2
    for (int f = 0; f < KB * 2; ++f)
        __builtin_amdgcn_global_load_lds(src + (f >> 1) * 128 + (f & 1) * 64,
                                         (lds_void*)(frag + f * 64), 16, 0, 0);
#pragma unroll 1
    for (int i = 0; i < KB / 4; ++i) {
        const int t = i * 64 + lane;
        const int kb = t >> 4, r = t & 15;
        const int srow = rb + (r < rc ? r : 0);
        __builtin_amdgcn_global_load_lds(a_scales + (size_t)kb * rows + srow,
                                         (lds_void*)(sa + i * 64), 4, 0, 0);
    }
}


// NT: weights are read with the non-temporal hint (streamed once, kept out of the caches).
template <int KB, int EPI, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_range_kernel(const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
                           const uint8_t* w, const float* __restrict__ w_scales,
                           const int4* __restrict__ tasks, const int32_t* __restrict__ ntasks,
                           const int32_t* __restrict__ sorted_ids, void* __restrict__ out,
                           int rows, int N) {
    constexpr int K = KB * 128;
    constexpr int kRing = KB < kRingMax ? KB : kRingMax;
    constexpr int P = KB / kRing;               // passes of the ring per subtask
    static_assert(KB % kRing == 0 && KB % 4 == 0, "K: a multiple of 512 and of the ring");
    constexpr int MAXT = TileLds<KB>::kMax;
    static_assert(MAXT >= 1, "one tile must fit");
    __shared__ TileLds<KB> L;
    __shared__ unsigned s_next;                 // next subtask of the range to hand out

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int nt = *ntasks;
    const int G = gridDim.x;
    // subtask s = (task s/8, 16-row group s%8 of its panel); this workgroup's share
    const long long ns = (long long)nt * kWaves;
    const int lo = (int)(ns * blockIdx.x / G);
    const int hi = (int)(ns * (blockIdx.x + 1) / G);
    if (lo >= hi) return;                       // whole workgroup: no barrier is left waiting
    const int Nb = N >> 7;
    const int t_lo = lo / kWaves, t_hi = (hi - 1) / kWaves + 1;   // tasks touched

    u32x4 wr0[kRing], wr1[kRing];
    // this lane's weight row of subtask s (task descriptor p), at byte g*16 of k-block 0
    auto wrow = [&](const TaskD& p, int s) -> const uint8_t* {
        return w + ((size_t)p.e * N + p.nb * 128 + (s % kWaves) * 16 + j) * K + g * 16;
    };
    auto ld = [&](const uint8_t* q) -> u32x4 {
        if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
        return *reinterpret_cast<const u32x4*>(q);
    };
    auto load_unit = [&](const uint8_t* wp, int kb, int u) {
        wr0[u] = ld(wp + kb * 128);
        wr1[u] = ld(wp + kb * 128 + 64);
    };
    auto pull = [&]() -> int {                  // next subtask index for this wave
        unsigned v = 0;
        if (lane == 0)
            v = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(v);
    };

    // Window of up to 64 tasks (one per lane): a tile starts at the window's first task and
    // wherever (rb, rc) changes.  Rounds take up to MAXT tiles each.  Wave 0 alone scans the
    // windows and moves the tiles; the other waves learn the round from LDS after the barrier
    // that publishes it, so their own weight loads never queue behind a descriptor load.
    __shared__ unsigned long long s_starts;
    __shared__ int s_wb, s_first, s_tend;
    uint64_t starts = 0;                        // window state: wave 0's working copy, and
    int wb = t_lo, wn = 0, ntile = 0, last = 0; // every wave's copy of the current round
    int first = 0, t_end = t_lo;
    auto scan_window = [&](int base) {
        wb = base;
        wn = min(64, t_hi - base);
        int rb = -1, rc = -1;
        if (lane < wn) {
            const int4 t = tasks[base + lane];
            rb = t.y;
            rc = t.z;
        }
        const int prb = __shfl_up(rb, 1), prc = __shfl_up(rc, 1);
        starts = __ballot(lane < wn && (lane == 0 || rb != prb || rc != prc));
        ntile = __popcll(starts);
    };
    // wave 0: choose the round after the current one, move its tiles, publish it
    auto plan_round = [&]() {
        if (t_end >= wb + wn) {
            scan_window(t_end);
            first = 0;
        } else {
            first = last;
        }
        last = min(ntile, first + MAXT);
        t_end = last < ntile ? wb + nth_set_bit(starts, last) : wb + wn;
        for (int s = 0; s < last - first; ++s) {
            const TaskD d = load_task(tasks, wb + nth_set_bit(starts, first + s));
            tile_dma<KB>(a, a_scales, rows, d.rb, d.rc, L.frag[s], L.sa[s], lane);
        }
        if (lane == 0) {
            s_starts = starts;
            s_wb = wb;
            s_first = first;
            s_tend = t_end;
        }
    };
    auto read_round = [&]() {
        starts = s_starts;
        wb = s_wb;
        first = s_first;
        t_end = s_tend;
    };
    auto tile_of = [&](int t) -> int {          // tile number of task t within the window
        const int i = t - wb;
        const uint64_t upto = i >= 63 ? ~0ull : ((2ull << i) - 1);
        return __popcll(starts & upto) - 1;
    };

    // the first subtask of every wave; wave 0 plans the first round before its weights
    int sc = lo + wave;
    if (wave == 0) plan_round();
    // (a wave without a first subtask, in a range of fewer than 8, loads the last one's
    // weights and never uses them: every wave issues the same loads, so the compiler's
    // accounting of outstanding loads stays exact and no barrier drains them)
    TaskD cur = load_task(tasks, min(sc, hi - 1) / kWaves);
    const uint8_t* wcur = wrow(cur, min(sc, hi - 1));
#pragma unroll
    for (int u = 0; u < kRing; ++u) load_unit(wcur, u, u);
    float sbc[KB];
    {
        const float* sbp = w_scales + ((size_t)cur.e * Nb + cur.nb) * KB;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sbc[kb] = sbp[kb];
    }
    if (threadIdx.x == 0) s_next = (unsigned)(lo + kWaves);
    int sn = hi;                                // next subtask (pulled after the first round)

    // one subtask; HN: a next subtask sn exists and its weights are loaded as units free up
    auto run_sub = [&](auto hn_tag, int tile_base) {
        constexpr bool HN = decltype(hn_tag)::value;
        const int t = sc / kWaves;
        const int slot = tile_of(t) - tile_base;
        const uint4* tb = L.frag[slot];
        const float* ts = L.sa[slot];
        TaskD nxt = cur;
        float sbn[KB];
        int sn2 = hi;
        if (HN) {
            sn2 = pull();                       // the one after next, used a subtask later
            nxt = load_task(tasks, sn / kWaves);
            const float* sbp = w_scales + ((size_t)nxt.e * Nb + nxt.nb) * KB;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sbn[kb] = sbp[kb];
        }
        const uint8_t* wnxt = wrow(nxt, sn);
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < P; ++p) {
            uint4 fb[3][2];                     // B fragments, read two units ahead
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                fb[u][0] = tb[((p * kRing + u) * 2 + 0) * 64 + lane];
                fb[u][1] = tb[((p * kRing + u) * 2 + 1) * 64 + lane];
            }
#pragma unroll
            for (int u = 0; u < kRing; ++u) {
                const int kb = p * kRing + u;
                if (u + 2 < kRing) {
                    fb[(u + 2) % 3][0] = tb[((kb + 2) * 2 + 0) * 64 + lane];
                    fb[(u + 2) % 3][1] = tb[((kb + 2) * 2 + 1) * 64 + lane];
                }
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f h = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    pack8v(wr0[u], wr1[u]), pack8(fb[u % 3][0], fb[u % 3][1]), zero, 0, 0, 0,
                    0, 0, 0);
                // the unit's registers are free again: refill with the same k-block of the
                // next pass, or of the next subtask
                if (p + 1 < P)
                    load_unit(wcur, kb + kRing, u);
                else if (HN)
                    load_unit(wnxt, u, u);
                __builtin_amdgcn_sched_barrier(0);
                acc += (ts[kb * 16 + j] * sbc[kb]) * h;
            }
        }
        // C layout of the 16x16 MFMA: lane (j, g) holds output rows 4g..4g+3 (weight
        // columns) of column j (routed row j)
        if (j < cur.rc) {
            const int n0 = cur.nb * 128 + (sc % kWaves) * 16 + g * 4;
            const size_t row = EPI == MOE_EPI_ROUTE_F32 ? (size_t)sorted_ids[cur.rb + j]
                                                        : (size_t)(cur.rb + j);
            if (EPI == MOE_EPI_STORE_BF16) {
                uint2 v;
                v.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
                v.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * N + n0) = v;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(out) + row * N + n0) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
        sc = sn;
        sn = sn2;
        if (HN) {
            cur = nxt;
            wcur = wnxt;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sbc[kb] = sbn[kb];
        }
    };

    // Every wave passes the same rounds; inside one it works through the subtasks it pulls
    // until its current one belongs to a later round.  The first barrier leaves every wave's
    // first weight burst in flight (wave 0's tiles went out before its burst).
    barrier_keep_vm<kRing * 2>();
    read_round();
    sn = pull();
    for (;;) {
        while (sc < hi && sc / kWaves < t_end) {
            if (sn < hi)
                run_sub(std::integral_constant<bool, true>{}, first);
            else
                run_sub(std::integral_constant<bool, false>{}, first);
        }
        if (t_end >= t_hi) break;
        __syncthreads();                        // every wave is done with the old tiles
        if (wave == 0) plan_round();
        __syncthreads();                        // the new tiles landed (vmcnt 0) and are visible
        read_round();
    }
}

template <int KB, bool NT>
hipError_t launch_kb(const uint8_t* a, const float* a_scales, int rows, const uint8_t* w,
                     const float* w_scales, int N, const moe_task* tasks,
                     const int32_t* ntasks, int epilogue, const int32_t* sorted, void* out,
                     int grid, hipStream_t s) {
    const int4* t = reinterpret_cast<const int4*>(tasks);
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            hipLaunchKernelGGL((gemm_fp8_range_kernel<KB, MOE_EPI_STORE_BF16, NT>), dim3(grid),
                               dim3(kThreads), 0, s, a, a_scales, w, w_scales, t, ntasks, sorted,
                               out, rows, N);
            break;
        case MOE_EPI_ROUTE_F32:
            hipLaunchKernelGGL((gemm_fp8_range_kernel<KB, MOE_EPI_ROUTE_F32, NT>), dim3(grid),
                               dim3(kThreads), 0, s, a, a_scales, w, w_scales, t, ntasks, sorted,
                               out, rows, N);
            break;
        default:
            hipLaunchKernelGGL((gemm_fp8_range_kernel<KB, MOE_EPI_STORE_F32, NT>), dim3(grid),
                               dim3(kThreads), 0, s, a, a_scales, w, w_scales, t, ntasks, sorted,
                               out, rows, N);
    }
    return hipGetLastError();
}

#ifndef MOE_RANGE_NT
#define MOE_RANGE_NT 1
#endif

}  // namespace

bool gemm_fp8_range_applies(int K, int chunk_rows) {
    // K = 4096 needs more registers than two waves per SIMD leave (it spills)
    return chunk_rows <= 16 && (K == 512 || K == 1024 || K == 2048);
}

hipError_t launch_gemm_fp8_range(const uint8_t* a, const float* a_scales, int rows, int K,
                                 const uint8_t* w, const float* w_scales, int N,
                                 const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                                 int epilogue, const int32_t* sorted, void* out,
                                 hipStream_t s) {
    int grid = device_info().cu_count;          // one 8-wave workgroup per CU
    if (grid > max_tasks) grid = max_tasks;
    if (grid <= 0) return hipSuccess;
    constexpr bool nt = MOE_RANGE_NT != 0;
    if (K == 512)
        return launch_kb<4, nt>(a, a_scales, rows, w, w_scales, N, tasks, ntasks, epilogue,
                                sorted, out, grid, s);
    if (K == 1024)
        return launch_kb<8, nt>(a, a_scales, rows, w, w_scales, N, tasks, ntasks, epilogue,
                                sorted, out, grid, s);
    return launch_kb<16, nt>(a, a_scales, rows, w, w_scales, N, tasks, ntasks, epilogue,
                             sorted, out, grid, s);
}

}  // namespace moe
