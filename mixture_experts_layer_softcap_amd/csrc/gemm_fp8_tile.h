// gemm_fp8_tile.h -- grouped FP8 GEMM against 128x128 block-scaled expert weights for larger
// routed-row counts: up to BM (128 or 256) routed rows of one expert against two adjacent
// 128-column weight panels, both operands staged in LDS ([FMF8] "Baseline: 7 kernels" item 6 and its
// listing: per-K-block scaling with a second accumulator, empty experts skipped; [WEAVE]
// sections 2.2 and 4.3: (expert, token_begin, token_num) tasks over a skewed load).
//
// Why a tiled form.  With tens to thousands of routed rows per expert (the pages' Zipf-skewed
// M=1024/4096 workloads) a weight panel streamed through registers against 16 rows at a time
// is re-read once per 16-64 rows.  Here a workgroup reads a 256 x K weight slab (two task
// panels of one chunk) once against up to BM rows, and the rows' FP8 codes once per slab.
// What bounds it on MI355X is the bytes each CU can have in flight to L2 (a few KB), so the
// design moves as few bytes per CU as it can: no padding rows, rows shared by two panels, and
// the chunks of one expert spread over the XCDs with their slabs back to back on one XCD.
//
// Stage = one 128-wide k-block (one scale block): the chunk's A rows [BM][128 B], the weight
// rows [256][128 B] and the row scales of that k-block go into LDS with global_load_lds;
// stages rotate (three at BM = 128, two at BM = 256), the DMA running one or two k-blocks
// ahead of the MFMAs.  An 8-row A group past the chunk moves the same 16 bytes of the chunk's
// last row into every lane instead of eight rows: every wave issues the same DMA instructions
// per stage (so the compiler's wait tracking stays exact), but padding costs one cache line.  The 16-byte chunk c of
// row r sits at position c ^ ((r/2) % 8) of its 128-byte LDS row: the LDS serves a 16-byte
// read for 16 lanes per clock over 64 banks (two rows side by side), and the rows of equal
// parity that an MFMA fragment read touches land on 8 distinct positions, so reads are
// conflict-free.  Every stage is a __shared__ object of its own and the k loop is unrolled by
// the stage count: the compiler then tells a DMA into one stage from reads of another and
// waits for exactly the stage a read needs, while the reads stay ordinary loads.
//
// MFMA.  V_MFMA_F32_16X16X128_F8F6F4, weights as the 16-row A side (output columns n), 16
// routed rows as the B side; one instruction spans exactly one scale block, so
//   acc[n][r] += (sa[r][b] * sw[n/128][b]) * mfma(w_block, a_block, 0).
// Each lane feeds bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the block's 128 for its row
// (g = lane/16), on both sides, so the dot product does not depend on the order the matrix
// core uses inside the instruction.  Eight waves; wave w owns weight rows [32w, 32w+32) of the
// slab (two 16-row blocks) against every routed row; 16-row groups past the chunk are skipped
// (LDS rows past the chunk hold stale or padding data, which only reaches output columns that
// are not stored).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 256;                      // weight rows (output columns) per workgroup
constexpr int kMaxKB = 64;                    // K <= 8192

typedef __attribute__((address_space(3))) void lds_void;

// Epilogue of the pages' scatter-add form (internal; gathering launches only): every routed
// row h of route r (token r / kr) is added as w[r] * h into the fp32 accumulator rows `out`
// [M][N] with float atomics.
constexpr int kEpiAtomicAdd = 100;

template <int BM>
struct TileCfg {
    static constexpr int kStages = BM == 128 ? 3 : 2;
    static constexpr int kGroups = BM / 16;           // 16-row MFMA groups
    static constexpr int kADma = BM / 64;             // A DMA instructions per wave
    static constexpr int kDma = 4 + kADma + 1;        // weight + A + row-scale DMAs per wave
};

// One stage: [row][16-byte position] of the A rows and of the weight rows, and the row scales
// of the stage's k-block (room for one 64-row block per wave; rows past the chunk repeat).
template <int BM>
struct TileStage {
    uint4 a[BM * 8];
    uint4 w[kBN * 8];
    float sa[kWaves * 64];
};

// Item enumeration shared by the schedules.  The task list holds Nb consecutive tasks per chunk
// (one per 128-column panel); an item is one chunk against a panel pair (a 256-row weight
// slab).  XCD-local order: XCD x owns chunks x, x+8, x+16, ... (the list is largest first,
// so every XCD gets some of the largest), item q of XCD x is chunk x + 8 (q / pairs) against
// pair q % pairs.  Global order (one shared queue): item g is chunk g / pairs, pair g % pairs.
struct Items {
    int Nb, pairs, nchunks;
    __device__ int xcd_items(int x) const {
        const int ncx = (nchunks - x + 7) >> 3;
        return ncx > 0 ? ncx * pairs : 0;
    }
    // task index and panels of XCD x's item q
    __device__ void of_xcd(int x, int q, int& task, int& nb0, int& np) const {
        nb0 = 2 * (q % pairs);
        np = min(2, Nb - nb0);
        task = (x + 8 * (q / pairs)) * Nb + nb0;
    }
    __device__ void of_global(int g, int& task, int& nb0, int& np) const {
        nb0 = 2 * (g % pairs);
        np = min(2, Nb - nb0);
        task = (g / pairs) * Nb + nb0;
    }
};

// GATHER: sorted row r is token sorted_route_ids[r] / kr of the token-major codes `a` [M][K]
// and scales [K/128][M] (rows = M), instead of row r of a sorted copy.
// KBC: the number of k-blocks when known at compile time (0: K / 128 at run time).  With it the
// k loop is fully unrolled and no DMA sits behind a run-time branch: the compiler's wait
// tracking, which turns conservative where paths with different DMAs in flight meet, then
// waits for exactly the stage each read needs.
// SCHED: MOE_SCHED_DISPATCH -- one workgroup per item, the hardware dispatcher hands them out
// (per XCD, in order, as CUs free up); an XCD whose last round of slabs would be at most half
// full runs those as single panels.  MOE_SCHED_STATIC -- one workgroup per CU, each walking a
// fixed share of its XCD's items (the static big kernel of [WEAVE] sections 1.2 and 3.1).  MOE_SCHED_QUEUE /
// MOE_SCHED_QUEUE_XCD -- one workgroup per CU pulling items from atomic counters ([WEAVE]
// sections 2.2 and 4.2), queue[0..7] tickets, queue[8] the exit count (the last workgroup out
// resets queue[0..8]), queue[9] set to 1 if a workgroup ever hit its iteration cap.
template <int BM, int EPI, int KBC, bool GATHER, int SCHED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_tile_kernel(const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
                          const uint8_t* __restrict__ w, const float* __restrict__ w_scales,
                          const int4* __restrict__ tasks, const int32_t* __restrict__ ntasks,
                          const int32_t* __restrict__ sorted_route_ids, void* __restrict__ out,
                          int rows, int K, int N, int pairs, int cus_x, int kr,
                          uint32_t* __restrict__ queue, const float* __restrict__ topk_weights) {
    using Cfg = TileCfg<BM>;
    constexpr int S = Cfg::kStages;
    constexpr bool PERSIST = SCHED != MOE_SCHED_DISPATCH;
    __shared__ TileStage<BM> st0, st1, st2;     // st2 is used only with three stages
    __shared__ float s_sw[kWaves][kMaxKB];    // rows 0, 1: scales of the two weight panels
    __shared__ int s_ids[kWaves * 64];        // GATHER: sorted route ids of the chunk rows
    __shared__ int s_item[2];                 // tickets published to the workgroup
    auto stage = [&](auto bt) __attribute__((always_inline)) -> TileStage<BM>& {
        constexpr int Bi = decltype(bt)::value;
        if constexpr (Bi == 0) return st0;
        else if constexpr (Bi == 1) return st1;
        else return st2;
    };
    const int Nb = N >> 7;
    const int xcd = (int)(blockIdx.x & 7);
    const int slot = (int)(blockIdx.x >> 3);
    const int nt = *ntasks;
    const Items items{Nb, pairs, (nt + Nb - 1) / Nb};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int KB = KBC ? KBC : K >> 7;
    const int dl = lane >> 3;

    // one item: expert chunk task `task` against panels nb0 .. nb0+np-1
    auto run_tile = [&](int task, int nb0, int np) __attribute__((always_inline)) {
        const int4 td = tasks[task];
        const int e = td.x, rb = td.y, rc = td.z;     // td.w == nb0

        // Start-up order.  A CU serves its memory requests in order and a wait covers every
        // older request, so nothing waits before the first stages' weight DMAs, which need
        // only the task: the weight-panel scales and the gathered rows' sorted route ids go
        // straight into LDS (the oldest requests), then the weights of stages 0 and 1 go out,
        // and the row DMAs follow once the ids are in.  Everything in flight is LDS DMA: with
        // plain loads into registers pending beside LDS DMAs the compiler can no longer count
        // which has landed and waits for all of them.
        //
        // DMA sources.  Weight rows: wave w moves slab rows [32w, 32w+32) (4 instructions of
        // 8 rows; a slab with one panel repeats it).  A rows: 8-row group w + 8i (i < BM/64)
        // holds chunk rows when it is below ngroups (rows past the chunk in that group repeat
        // its last row); otherwise every lane moves the same 16 bytes of the last row.  Row
        // scales: wave w moves those of rows [64w, 64w+64), clamped to the chunk.
        const int ngroups = (rc + 7) >> 3;
        // weight-panel scales of every k-block: wave w moves panel min(w, np-1)'s into row w of
        // s_sw (rows 0 and 1 are read; every wave issues the same DMA)
        __builtin_amdgcn_global_load_lds(
            w_scales + ((size_t)e * Nb + nb0 + min(wave, np - 1)) * KB + min(lane, KB - 1),
            (lds_void*)&s_sw[wave][0], 4, 0, 0);
        // GATHER: wave w moves the sorted route ids of chunk rows [64w, 64w+64) (clamped to the
        // chunk) into s_ids, read after the barrier below
        if constexpr (GATHER)
            __builtin_amdgcn_global_load_lds(sorted_route_ids + rb + min(wave * 64 + lane, rc - 1),
                                             (lds_void*)&s_ids[wave * 64], 4, 0, 0);
        __builtin_amdgcn_sched_barrier(0);

        const uint8_t* srcW[4];
        const uint8_t* srcA[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 32 + i * 8 + dl;
            const int dc = (lane & 7) ^ ((r >> 1) & 7);
            const int wr = nb0 * 128 + (r < np * 128 ? r : r - 128);
            srcW[i] = w + ((size_t)e * N + wr) * K + dc * 16;
        }
        auto issue_w = [&](auto bt, int kb) __attribute__((always_inline)) {
            TileStage<BM>& T = stage(bt);
            const int k0 = kb * 128;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds(srcW[i] + k0,
                                                 (lds_void*)&T.w[(wave * 32 + i * 8) * 8], 16,
                                                 0, 0);
        };
        issue_w(std::integral_constant<int, 0>{}, 0);
        if (S == 3 && KB > 1) issue_w(std::integral_constant<int, 1>{}, 1);
        __builtin_amdgcn_sched_barrier(0);
        // source row of chunk row i (i < rc)
        auto src_row = [&](int i) __attribute__((always_inline)) -> size_t {
            if (GATHER) return (size_t)(s_ids[i] / kr);
            return (size_t)(rb + i);
        };
        if constexpr (GATHER) {
            // every wave's ids have landed (only the weight DMAs may still be in flight)
            if (S == 3 && KB > 1)
                barrier_keep_vm<8>();
            else
                barrier_keep_vm<4>();
        }

#pragma unroll
        for (int i = 0; i < Cfg::kADma; ++i) {
            const int r = (wave + 8 * i) * 8 + dl;
            const int dc = (lane & 7) ^ ((r >> 1) & 7);
            srcA[i] = a + src_row(min(r, rc - 1)) * K + dc * 16;
        }
        const uint8_t* srcPad = a + src_row(rc - 1) * K;
        const float* srcS = a_scales + src_row(min(wave * 64 + lane, rc - 1));

        // the row DMAs (and row scales) of k-block kb into stage bt
        auto issue_a = [&](auto bt, int kb) __attribute__((always_inline)) {
            TileStage<BM>& T = stage(bt);
            const int k0 = kb * 128;
#pragma unroll
            for (int i = 0; i < Cfg::kADma; ++i) {
                lds_void* dst = (lds_void*)&T.a[(wave + 8 * i) * 64];
                // (a select, not a branch: DMAs behind a branch make the wait tracking drain)
                const uint8_t* src = wave + 8 * i < ngroups ? srcA[i] : srcPad;
                __builtin_amdgcn_global_load_lds(src + k0, dst, 16, 0, 0);
            }
            __builtin_amdgcn_global_load_lds(srcS + (size_t)kb * rows,
                                             (lds_void*)&T.sa[wave * 64], 4, 0, 0);
        };
        auto issue = [&](auto bt, int kb) __attribute__((always_inline)) {
            issue_w(bt, kb);
            issue_a(bt, kb);
        };
        issue_a(std::integral_constant<int, 0>{}, 0);
        if (S == 3 && KB > 1) issue_a(std::integral_constant<int, 1>{}, 1);

        v4f acc[2][Cfg::kGroups];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < Cfg::kGroups; ++r) acc[b][r] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const int nrg = (rc + 15) >> 4;           // 16-row groups holding chunk rows
        // fragment positions of lane (j, g) inside a row, in bytes: chunks g and 4 + g at their
        // swizzled positions (every row a lane reads has (row/2)%8 = (j/2)%8)
        const int p0 = (g ^ ((j >> 1) & 7)) * 16;
        const int p1 = ((4 + g) ^ ((j >> 1) & 7)) * 16;

        // the MFMAs of k-block kb on stage bt
        auto compute = [&](auto bt, int kb) __attribute__((always_inline)) {
            const TileStage<BM>& T = stage(bt);
            const float sw = s_sw[wave >> 2][kb];
            // (plain element indexing of the stage arrays keeps the alias information the
            // compiler's wait tracking needs; byte-pointer arithmetic on them loses it)
            const int wrow = (wave * 32 + j) * 8, arow = j * 8, i0 = p0 >> 4, i1 = p1 >> 4;
            v8i wf[2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
                wf[b] = pack8(T.w[wrow + b * 128 + i0], T.w[wrow + b * 128 + i1]);
            // row groups: group r+1's fragment is read before group r's MFMAs
            uint4 c0 = T.a[arow + i0];
            uint4 c1 = T.a[arow + i1];
            float cs = T.sa[j];
#pragma unroll
            for (int r = 0; r < Cfg::kGroups; ++r) {
                if (r >= nrg) break;
                uint4 n0 = c0, n1 = c1;
                float ns = cs;
                if (r + 1 < Cfg::kGroups && r + 1 < nrg) {
                    n0 = T.a[arow + (r + 1) * 128 + i0];
                    n1 = T.a[arow + (r + 1) * 128 + i1];
                    ns = T.sa[(r + 1) * 16 + j];
                }
                const v8i af = pack8(c0, c1);
                const float f = cs * sw;
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const v4f h = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf[b], af, zero, 0, 0, 0, 0, 0, 0);
                    acc[b][r] += f * h;
                }
                c0 = n0;
                c1 = n1;
                cs = ns;
            }
        };

        // one k-block on stage Bi: wait for it, publish it, refill the stage the barrier freed
        auto step = [&](auto bt, int kb) __attribute__((always_inline)) {
            constexpr int Bi = decltype(bt)::value;
            if constexpr (S == 3) {
                // this wave's DMA of stage kb has landed (stage kb+1's may still be in flight);
                // the barrier publishes every wave's and frees the stage read one k-block ago.
                // The first two stages went out weights first (W0 W1 A0 S0 A1 S1, after the
                // panel scales), so at kb = 0 only stage 1's row and scale DMAs may stay in
                // flight.
                if (kb + 1 < KB) {
                    if (kb == 0)
                        barrier_keep_vm<Cfg::kADma + 1>();
                    else
                        barrier_keep_vm<Cfg::kDma>();
                } else {
                    barrier_keep_vm<0>();
                }
                if (kb + 2 < KB) issue(std::integral_constant<int, (Bi + 2) % 3>{}, kb + 2);
            } else {
                // two stages: stage kb has landed everywhere and the other one is no longer read
                barrier_keep_vm<0>();
                if (kb + 1 < KB) issue(std::integral_constant<int, Bi ^ 1>{}, kb + 1);
            }
            compute(bt, kb);
        };

#pragma unroll
        for (int kb = 0; kb < KB; kb += S) {
            step(std::integral_constant<int, 0>{}, kb);
            if (kb + 1 < KB) step(std::integral_constant<int, 1>{}, kb + 1);
            if constexpr (S == 3)
                if (kb + 2 < KB) step(std::integral_constant<int, 2>{}, kb + 2);
        }

        // C layout of the 16x16 MFMA: lane (j, g) holds rows 4g..4g+3 (weight rows, i.e. output
        // columns) of column j (routed row r*16 + j); waves of a missing second panel store
        // nothing
        if ((wave >> 2) < np) {
#pragma unroll
            for (int r = 0; r < Cfg::kGroups; ++r) {
                const int m = r * 16 + j;
                if (r >= nrg || m >= rc) continue;
                size_t row = (size_t)(rb + m);
                if (EPI == MOE_EPI_ROUTE_F32 || EPI == kEpiAtomicAdd)   // (GATHER: from LDS)
                    row = (size_t)(GATHER ? s_ids[m] : sorted_route_ids[rb + m]);
                float wv = 0.0f;
                if constexpr (EPI == kEpiAtomicAdd) wv = topk_weights[row];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int n = nb0 * 128 + wave * 32 + b * 16 + g * 4;
                    const v4f c = acc[b][r];
                    if constexpr (EPI == kEpiAtomicAdd) {
                        float* dst = static_cast<float*>(out) + (row / kr) * N + n;
#pragma unroll
                        for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + i, wv * c[i]);
                    } else if (EPI == MOE_EPI_STORE_BF16) {
                        uint2 v;
                        v.x = f32_to_bf16(c[0]) | (f32_to_bf16(c[1]) << 16);
                        v.y = f32_to_bf16(c[2]) | (f32_to_bf16(c[3]) << 16);
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * N + n) = v;
                    } else {
                        *reinterpret_cast<float4*>(static_cast<float*>(out) + row * N + n) =
                            make_float4(c[0], c[1], c[2], c[3]);
                    }
                }
            }
        }
    };

    if constexpr (!PERSIST) {
        // The XCD runs its P panel-pair items on cus_x CUs; when its last round would hold r <=
        // cus_x/2 items, those r items run as 2r single panels instead (a round of pairs then
        // ends in a shorter round of singles).
        const int P = items.xcd_items(xcd);
        const int r = P % cus_x;
        const int R = 2 * r <= cus_x ? r : 0;
        int task, nb0, np;
        if (slot < P - R) {
            items.of_xcd(xcd, slot, task, nb0, np);
        } else {
            const int i = slot - (P - R);
            if (i >= 2 * R) return;
            items.of_xcd(xcd, P - R + (i >> 1), task, nb0, np);
            nb0 += i & 1;
            np = 1;
            if (nb0 >= Nb) return;                // odd Nb: the last pair has one panel
            task += i & 1;
        }
        if (task >= nt) return;
        run_tile(task, nb0, np);
    } else {
        // persistent: the workgroup walks its items; between two items one barrier keeps the
        // stage buffers and s_sw from being rewritten while another wave still reads them
        const int cap = items.nchunks * pairs + 1;    // no walk is longer than the item count
        int victim = 0;                                // QUEUE_XCD: the XCD being drained
        auto next_ticket = [&]() -> int {             // thread 0 only
            if (SCHED == MOE_SCHED_QUEUE) {
                const int gi = (int)atomicAdd(&queue[0], 1u);
                return gi < items.nchunks * pairs ? gi : -1;
            }
            for (; victim < 8; ++victim) {
                const int x = (xcd + victim) & 7;
                const int n = items.xcd_items(x);
                if (n <= 0) continue;
                const int t = (int)atomicAdd(&queue[x], 1u);
                if (t < n) return (x << 24) | t;
            }
            return -1;
        };
        int cur;
        if (SCHED == MOE_SCHED_STATIC) {
            cur = slot < items.xcd_items(xcd) ? (xcd << 24) | slot : -1;
        } else {
            if (tid == 0) s_item[0] = next_ticket();
            __syncthreads();
            cur = s_item[0];
        }
        int iter = 0;
        while (cur >= 0) {
            int task, nb0, np;
            if (SCHED == MOE_SCHED_QUEUE)
                items.of_global(cur, task, nb0, np);
            else
                items.of_xcd(cur >> 24, cur & 0xFFFFFF, task, nb0, np);
            run_tile(task, nb0, np);
            ++iter;
            if (SCHED == MOE_SCHED_STATIC) {
                const int q = slot + iter * cus_x;
                cur = q < items.xcd_items(xcd) ? (xcd << 24) | q : -1;
                __syncthreads();
            } else {
                if (tid == 0) s_item[iter & 1] = next_ticket();
                __syncthreads();
                cur = s_item[iter & 1];
            }
            if (iter >= cap && cur >= 0) {            // cannot happen with a sound counter
                if (SCHED != MOE_SCHED_STATIC && tid == 0) atomicOr(&queue[9], 1u);
                break;
            }
        }
        if (SCHED != MOE_SCHED_STATIC && tid == 0) {
            if (atomicAdd(&queue[8], 1u) == gridDim.x - 1u) {
#pragma unroll
                for (int i = 0; i < 9; ++i) atomicExch(&queue[i], 0u);
            }
        }
    }
}

// Grid of a launch: one workgroup per item (plus the single-panel split of a short last round)
// for MOE_SCHED_DISPATCH, one per CU otherwise.
inline unsigned tile_grid(int sched, int N, int max_tasks) {
    const int Nb = N / 128;
    const int pairs = (Nb + 1) / 2;
    const int max_chunks = (max_tasks + Nb - 1) / Nb;
    const int cpx = (max_chunks + 7) / 8;
    const int cus_x = max(2, device_info().cu_count / 8);   // CUs per XCD
    if (sched != MOE_SCHED_DISPATCH) return (unsigned)(8 * cus_x);
    return (unsigned)(8 * (cpx * pairs + cus_x / 2));
}

template <int BM, int EPI, int KBC, bool GATHER, int SCHED>
hipError_t launch_tile(const uint8_t* a, const float* a_scales, int rows, int K,
                       const uint8_t* w, const float* w_scales, int N, const moe_task* tasks,
                       const int32_t* ntasks, int max_tasks, const int32_t* sorted, void* out,
                       int kr, uint32_t* queue, hipStream_t s,
                       const float* topk_weights = nullptr) {
    const int Nb = N / 128;
    const int pairs = (Nb + 1) / 2;
    const int cus_x = max(2, device_info().cu_count / 8);
    hipLaunchKernelGGL((gemm_fp8_tile_kernel<BM, EPI, KBC, GATHER, SCHED>),
                       dim3(tile_grid(SCHED, N, max_tasks)), dim3(kThreads), 0, s, a, a_scales, w,
                       w_scales, reinterpret_cast<const int4*>(tasks), ntasks, sorted, out, rows,
                       K, N, pairs, cus_x, kr, queue, topk_weights);
    return hipGetLastError();
}

}  // namespace
}  // namespace moe
