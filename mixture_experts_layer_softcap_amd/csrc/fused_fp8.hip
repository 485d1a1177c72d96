// fused_fp8.hip -- small-batch grouped FP8 GEMM straight from the routed ids: the layout,
// sort/gather and quantisation stages ([FMF8] "Baseline: 7 kernels" items 2-5, Fusion 2 and 3)
// folded into the grouped GEMM (item 6, per-K-block scaling) for at most 2048 routed rows and
// K = 256, 512, 1024 or 2048 -- the decode-sized regime of the pages' problem table (a few rows
// per expert).
//
// Work split.  The weights, not the routed rows, are divided among the workgroups: the E*N/16
// slices of 16 weight rows x K bytes, in expert-major order, are cut into one contiguous range
// per workgroup (one workgroup per CU).  Every workgroup streams the same number of bytes
// whatever the routing, the split needs no layout stage, and each slice is read once, against
// all routed rows of its expert.  A range covers one expert's slices, or a few experts' (at
// most kMaxLocal); a slice of an expert nobody chose is not read.
//
// Routed rows.  Each workgroup finds its experts' routes in the ids (ballot scans, so an
// expert's rows stay in ascending route id), cuts them into tiles of 16 rows and quantises the
// rows of x (bf16) per 128-value block with the rule of the QSG stage (amax / 448, E4M3 RNE)
// straight into LDS, in MFMA fragment order.  Up to kTiles tiles are resident; an expert with
// more routed rows than fit goes round by round, its slices streamed once per round.
//
// Weights.  Each wave walks every 8th slice of the round (and, for an expert with several
// resident tiles, each slice once per tile) with a ring of kRing = K/128 k-block units in
// registers -- a whole slice, two 16-byte loads per lane per unit -- refilling each unit right
// after its MFMA with the same k-block of the wave's next item, so the stream does not pause
// between items.
//
// Start-up order (measured on MI355X with one workgroup per CU).  Once every CU streams its
// weights, any request, an L2 hit included, waits several us behind the chip-wide burst, and
// a CU serves its own requests in order.  So: the ids, then a small early burst (kPre units,
// which drains while the route list is built), the x rows of the tiles, and only when every
// wave of the CU holds its x rows the rest of the burst; the rows are quantised while the
// burst is in flight, and the barrier that publishes the tiles leaves it in flight.
//
// Output.  fp32 rows at their route ids (rows[t*k + j] = x[t] . W[e_tj]^T with both operands
// dequantised per block), which the combine reads without a slot table.
//
// Routing inside (the ROUTE form; [FMF8] "Baseline: 7 kernels" item 1 folded in as well).
// Token t is routed by wave t / G of workgroup t % G (G workgroups) before that wave waits for
// anything; its logits loads go out ahead of the CU's weight burst (a workgroup barrier right
// after they are issued), since the CU serves its requests in order.  The wave writes the
// token's ids and weights for the combine, and each route once more into the handoff words as
// tag | expert with an agent-scope store: a word carries its own validity, so no flag, fence
// or ordering between stores is needed.  Every thread of every workgroup polls its four route
// words (agent-scope loads, which also fetch the ids it needs) until they carry this call's
// tag, at most max_polls rounds; a wave whose words are still missing then routes those
// tokens itself (the same selection, so the same experts) and sets *status, so no wait can
// fail and no wait depends on a workgroup that has not been dispatched.  A word is
// 0x7FA00000 | epoch << 8 | expert (a 12-bit epoch that changes with every call, an 8-bit
// expert): as a float every such word is a signalling NaN (computed NaNs are the quiet
// default, +-inf is 0x7F800000 / 0xFF800000), and its top byte 0x7F is a code the library's
// E4M3 encoder never writes, so old bytes do not pass for a route, and a word left by an
// earlier call carries an older epoch (the forward's combine also clears them).
#include "moe_device.h"
#include "moe_internal.h"

#include <atomic>
#include <type_traits>

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxRoutes = 2048;              // M * k
constexpr int kMaxLocal = 4;                  // experts touched by one workgroup's range
constexpr int kTiles = 4;                     // resident 16-row tiles
constexpr int kRouteVPL = 4;                  // ROUTE form: logits per lane, E <= 256

// KB = K / 128 k-blocks per row: 2, 4, 8 or 16 (K = 256 .. 2048)
template <int KB>
struct FusedLds {
    uint4 frag[kTiles][KB * 2 * 64];          // fragment f = (k-block f/2, half f%2)
    float sa[kTiles][KB * 16];                // [k-block][row]
    int list[kMaxRoutes];                     // (token << 12) | route, expert-major
    int cnt[kMaxLocal];                       // routes per local expert
    int first[kMaxLocal];                     // list position of its first route
    int tp[kMaxLocal + 1];                    // tile prefix over the local experts
    int trc[kTiles];                          // rows of each resident tile
    int tlb[kTiles];                          // list position of its row 0
    int wsum[2][kWaves];
};

// Arguments of the ROUTE form (unused otherwise).
struct FusedRoute {
    const float* logits;                      // f32 [M][E]
    int32_t* ids;                             // out: topk_ids [M][k]
    float* weights;                           // out: topk_weights [M][k]
    uint32_t* handoff;                        // [M*k] route words, without this call's tag
    uint32_t* status;                         // set to 1 when a wave routed tokens itself
    uint32_t tag;                             // 0x7FA00000 | epoch << 8
    int max_polls;                            // poll rounds before a wave routes for itself
    int M, E;
    float softcap;
};

// ACT form (the FP8 MLP's down projection): the A rows are act = silu(g) * u of the fp32
// gate+up rows h [R][2K] at route ids, requantised per 128 columns as by moe_swiglu_quant;
// the codes [R][K] and scales [K/128][R] also go to a_q / a_s when those are set.
struct FusedAct {
    uint8_t* a_q;
    float* a_s;
};

// Workgroup barrier for LDS data only: vector-memory operations stay in flight.
__device__ __forceinline__ void barrier_lds() { barrier_keep_vm<63>(); }

// Exclusive scan over the 512-thread workgroup of a count c in [0, 7] per thread, from three
// wave ballots of its bits (no shuffles); one barrier; s_w must not be written again before
// every wave has passed the next barrier.
__device__ __forceinline__ int scan512_small(int c, int* s_w, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t m0 = __ballot(c & 1), m1 = __ballot(c & 2), m2 = __ballot(c & 4);
    const uint64_t lt = (1ull << lane) - 1ull;
    const int below = __popcll(m0 & lt) + 2 * __popcll(m1 & lt) + 4 * __popcll(m2 & lt);
    if (lane == 0) s_w[wave] = __popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2);
    barrier_lds();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = s_w[i];
        base += i < wave ? t : 0;
        tot += t;
    }
    total = tot;
    return base + below;
}

template <int KB, bool NT, bool ROUTE, bool ACT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_fused_kernel(const void* xin, const int32_t* __restrict__ ids, int R, int k,
                           const uint8_t* w, const float* __restrict__ w_scales, int N,
                           int slices, float* __restrict__ rows_out, FusedRoute rt,
                           FusedAct act) {
    static_assert(!(ROUTE && ACT), "the ACT form reads routed ids");
    const uint16_t* x = static_cast<const uint16_t*>(xin);      // bf16 [M][K]
    const float* hin = static_cast<const float*>(xin);          // ACT: fp32 [R][2K]
    constexpr int kKB = KB;                     // k-blocks per row
    constexpr int kK = KB * 128;
    constexpr int kRing = KB < 16 ? KB : 16;    // k-block units per wave in registers
    constexpr int kPasses = kKB / kRing;
    constexpr int kXSteps = KB / 2;             // x loads per lane for one tile (16 * KB blocks)
    __shared__ FusedLds<KB> L;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int NS = N >> 4;                      // slices per expert
    const int Nb = N >> 7;                      // 128-row weight-scale blocks per expert
    const int lo = (int)((long long)slices * blockIdx.x / gridDim.x);
    const int hi = (int)((long long)slices * (blockIdx.x + 1) / gridDim.x);
    if constexpr (ROUTE) {
        const int t = blockIdx.x + gridDim.x * wave;
        float val[kRouteVPL];
        if (t < rt.M) route_load_row<kRouteVPL>(rt.logits + (size_t)t * rt.E, rt.E, lane, val);
        if (blockIdx.x < rt.M) barrier_lds();   // the logits go out ahead of the weight burst
        if (t < rt.M) {                         // wave-uniform: this wave routes token t
            int my_e;
            float my_w;
            route_select<kRouteVPL>(val, rt.E, k, rt.softcap, lane, my_e, my_w);
            if (lane < k) {
                const size_t r = (size_t)t * k + lane;
                __hip_atomic_store(rt.handoff + r, rt.tag | (uint32_t)my_e,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                rt.ids[r] = my_e;
                rt.weights[r] = my_w;
            }
        }
    }
    if (lo >= hi) return;                       // whole workgroup
    const int e0 = lo / NS;
    const int ne = (hi - 1) / NS - e0 + 1;      // local experts e0 .. e0+ne-1 (<= kMaxLocal)

    // ---- weights ----
    u32x4 wr0[kRing], wr1[kRing];
    auto ld = [&](const uint8_t* q) __attribute__((always_inline)) -> u32x4 {
        if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
        return *reinterpret_cast<const u32x4*>(q);
    };
    auto load_unit = [&](const uint8_t* wp, int kb, int u) __attribute__((always_inline)) {
        wr0[u] = ld(wp + kb * 128);
        wr1[u] = ld(wp + kb * 128 + 64);
    };
    // this lane's weight row of slice s, at byte g*16 of k-block 0
    auto slice_ptr = [&](int s) __attribute__((always_inline)) -> const uint8_t* {
        const int e = s / NS, cs = s - e * NS;
        return w + ((size_t)e * N + cs * 16 + j) * kK + g * 16;
    };
    auto slice_scales = [&](int s, float* dst) __attribute__((always_inline)) {
        const int e = s / NS, cs = s - e * NS;
        const float* p = w_scales + ((size_t)e * Nb + (cs >> 3)) * kKB;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) dst[kb] = p[kb];
    };

    // ---- the routes of the local experts, each expert's in ascending route id ----
    // Thread tid looks at routes 4*tid .. 4*tid+3 (unconditional, clamped loads).  Behind the
    // ids goes a small first burst: the first kPre units of the wave's first slice of the
    // range (unless routing moves the wave's start, the slice it will stream first).  It keeps
    // the memory busy while the tiles are built, yet drains before the x rows are requested.
    constexpr int kPre = (ROUTE ? 6 : 4) < kRing ? (ROUTE ? 6 : 4) : kRing;
    const int s_pre = min(lo + wave, hi - 1);
    int v[4];
    if constexpr (!ROUTE) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = ids[min(tid * 4 + u, R - 1)];
        __builtin_amdgcn_sched_barrier(0);      // the ids go out first
        {
            const uint8_t* wp = slice_ptr(s_pre);
#pragma unroll
            for (int u = 0; u < kPre; ++u) load_unit(wp, u, u);
        }
        MOE_WAIT_VMCNT(2 * kPre);               // the ids
    } else {
        // the early burst goes out while the routing waves finish; then every thread waits
        // for its four route words, which bring the ids
        {
            const uint8_t* wp = slice_ptr(s_pre);
#pragma unroll
            for (int u = 0; u < kPre; ++u) load_unit(wp, u, u);
        }
        __builtin_amdgcn_sched_barrier(0);
        unsigned have = 0;                      // bit u: v[u] arrived
        for (int it = 0; it < rt.max_polls; ++it) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!(have >> u & 1u)) {
                    const uint32_t wd = __hip_atomic_load(rt.handoff + min(tid * 4 + u, R - 1),
                                                          __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                    if ((wd & 0xFFFFFF00u) == rt.tag) {
                        v[u] = (int)(wd & 0xFFu);
                        have |= 1u << u;
                    }
                }
            }
            if (__ballot(have != 15u) == 0) break;
            __builtin_amdgcn_s_sleep(2);
        }
        // Words still missing (their routing wave is late): the wave routes those tokens
        // itself, one token per round, the lowest lane's first missing word first, and every
        // lane takes the experts of its words on that token.  Each round fills at least one
        // word, so at most 256 rounds.
        uint64_t need = __ballot(have != 15u);
        if (need != 0) {
            if (lane == 0)
                __hip_atomic_store(rt.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            do {
                const int src = __ffsll((unsigned long long)need) - 1;
                const unsigned hs = __shfl(have, src);
                const int rs = min((wave * 64 + src) * 4 + __ffs(~hs & 15u) - 1, R - 1);
                const int ts = rs / k;
                float val[kRouteVPL];
                route_load_row<kRouteVPL>(rt.logits + (size_t)ts * rt.E, rt.E, lane, val);
                int my_e;
                float my_w;
                route_select<kRouteVPL>(val, rt.E, k, rt.softcap, lane, my_e, my_w);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = min(tid * 4 + u, R - 1) - ts * k;   // word's place in token ts
                    const int e_j = __shfl(my_e, j & 63);
                    if (!(have >> u & 1u) && j >= 0 && j < k) {
                        v[u] = e_j;
                        have |= 1u << u;
                    }
                }
                need = __ballot(have != 15u);
            } while (need != 0);
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)                 // local expert index; invalid ids match none
        v[u] = tid * 4 + u < R ? v[u] - e0 : -1;
    int base = 0;
    int i = 0;
    do {                                        // (ne >= 1: the ids' uses stay unconditional)
        const int c = (v[0] == i) + (v[1] == i) + (v[2] == i) + (v[3] == i);
        int tot;
        int p = base + scan512_small(c, L.wsum[i & 1], tot);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (v[u] == i) {
                const int r = tid * 4 + u;
                L.list[p++] = ((r / k) << 12) | r;
            }
        }
        if (tid == 0) {
            L.cnt[i] = tot;
            L.first[i] = base;
        }
        base += tot;
    } while (++i < ne);
    if (tid == 0) {
        int t = 0;
        for (int i = 0; i < ne; ++i) {
            L.tp[i] = t;
            t += (L.cnt[i] + 15) >> 4;
        }
        L.tp[ne] = t;
    }
    barrier_lds();

    auto tp_at = [&](int i) __attribute__((always_inline)) -> int { return __builtin_amdgcn_readfirstlane(L.tp[i]); };
    const int T = tp_at(ne);                    // tiles of the range

    float sbc[kKB];

    for (int qa = 0; qa < T; qa += kTiles) {
        const int qb = min(T, qa + kTiles);    // tiles [qa, qb) are resident this round
        int ia = 0;
        while (tp_at(ia + 1) <= qa) ++ia;
        int ib = ia;
        while (tp_at(ib + 1) < qb) ++ib;
        // slices of the round's experts within the range
        const int a = max(lo, (e0 + ia) * NS);
        const int b = min(hi, (e0 + ib + 1) * NS);
        auto ntiles_of = [&](int i) __attribute__((always_inline)) -> int { return min(tp_at(i + 1), qb) - max(tp_at(i), qa); };
        auto next_valid = [&](int s) __attribute__((always_inline)) -> int {   // this wave's next slice with resident tiles
            while (s < b && ntiles_of(s / NS - e0) <= 0) s += kWaves;
            return s;
        };
        int sc = next_valid(a + wave);
        // a wave without a slice loads the round's last one and never uses it: every wave
        // issues the same loads, so no barrier has to drain them
        const int s_first = sc < b ? sc : b - 1;
        const uint8_t* wcur = slice_ptr(s_first);
        slice_scales(s_first, sbc);
        // units [u0, kRing) of the burst are still to load (the first round keeps the early
        // units when the wave starts where it was expected to)
        const int u0 = qa == 0 && s_first == s_pre ? kPre : 0;

        // ---- tiles: x rows -> E4M3 fragments and block scales in LDS ----
        auto build_tile = [&](int t, auto burst_tag) __attribute__((always_inline)) {
            constexpr bool BURST = decltype(burst_tag)::value;
            const int q = qa + t;
            int i = ia;
            while (tp_at(i + 1) <= q) ++i;
            const int ci = q - tp_at(i);
            const int lb = __builtin_amdgcn_readfirstlane(L.first[i]) + ci * 16;
            const int rc = min(16, __builtin_amdgcn_readfirstlane(L.cnt[i]) - ci * 16);
            if (tid == 0) {
                L.trc[t] = rc;
                L.tlb[t] = lb;
            }
            // step st covers blocks 4*st .. 4*st+3 (row b/KB, k-block b%KB), one per 16 lanes;
            // rows past rc are not quantised (their columns are not stored); their lanes still
            // load, unconditionally, but all from the first 256 bytes of x, which stay in the
            // CU's L1 and take no place among its requests to L2 (at a few routes per expert
            // most of a tile is padding)
            uint4 xr[kXSteps];
            float4 hg0[ACT ? kXSteps : 1], hg1[ACT ? kXSteps : 1];
            float4 hu0[ACT ? kXSteps : 1], hu1[ACT ? kXSteps : 1];
#pragma unroll
            for (int i8 = 0; i8 < kXSteps; ++i8) {
                const int bq = (wave + i8 * kWaves) * 4 + g;
                const int jj = bq / kKB, kb = bq % kKB;
                const int ent = L.list[lb + (jj < rc ? jj : 0)];
                if constexpr (ACT) {
                    // gate and up values of columns kb*128 + 8j .. +8 of the route's row (rows
                    // past rc read route 0's row)
                    const float* hr = hin + (jj < rc ? (size_t)(ent & 0xFFF) * 2 * kK : 0) +
                                      kb * 128 + j * 8;
                    hg0[i8] = *reinterpret_cast<const float4*>(hr);
                    hg1[i8] = *reinterpret_cast<const float4*>(hr + 4);
                    hu0[i8] = *reinterpret_cast<const float4*>(hr + kK);
                    hu1[i8] = *reinterpret_cast<const float4*>(hr + kK + 4);
                } else {
                    const size_t off = jj < rc ? (size_t)(ent >> 12) * kK + kb * 128 : 0;
                    xr[i8] = *reinterpret_cast<const uint4*>(x + off + j * 8);
                }
            }
            MOE_WAIT_VMCNT(0);
            if (BURST) {
                // The weights follow the round's last x rows once every wave of the CU has
                // them (its memory pipeline serves requests in order), and before the rows are
                // quantised: while the burst is issued the wave may stall on a full memory
                // queue, and the tiles are not needed before the weights land anyway.
                barrier_keep_vm<0>();
                if (u0 == 0) {
#pragma unroll
                    for (int u = 0; u < kPre; ++u) load_unit(wcur, u, u);
                }
#pragma unroll
                for (int u = kPre; u < kRing; ++u) load_unit(wcur, u, u);
            }
#pragma unroll
            for (int i8 = 0; i8 < kXSteps; ++i8) {
                const int bq = (wave + i8 * kWaves) * 4 + g;
                const int jj = bq / kKB, kb = bq % kKB;
                if (jj < rc) {                  // whole 16-lane groups
                    Quant8 qv;
                    if constexpr (ACT) {
                        float v[8];
                        silu_mul8(hg0[i8], hg1[i8], hu0[i8], hu1[i8], v);
                        qv = quantise8_f32(v, true);
                        if (act.a_q) {          // the codes in route order, as moe_swiglu_quant
                            const int route = L.list[lb + jj] & 0xFFF;
                            *reinterpret_cast<uint2*>(act.a_q + (size_t)route * kK + kb * 128 +
                                                      j * 8) = qv.codes;
                            if (j == 0) act.a_s[(size_t)kb * R + route] = qv.scale;
                        }
                    } else {
                        qv = quantise8(xr[i8], true);
                    }
                    const int el = j * 8;       // element offset inside the 128-value block
                    const int f = kb * 2 + (el >> 6);
                    uint8_t* dst = reinterpret_cast<uint8_t*>(
                        &L.frag[t][f * 64 + ((el & 63) >> 4) * 16 + jj]);
                    *reinterpret_cast<uint2*>(dst + (el & 15)) = qv.codes;
                    if (j == 0) L.sa[t][kb * 16 + jj] = qv.scale;
                }
            }
        };
        // Under a chip-wide burst every request, L2 hits included, waits several us: the x rows
        // are all in before the weights go out.
        const int n = qb - qa;
        for (int t = 0; t + 1 < n; ++t) build_tile(t, std::false_type{});
        build_tile(n - 1, std::true_type{});
        barrier_keep_vm<2 * kRing>();           // tiles visible; the burst stays in flight

        // ---- this wave's work: (slice, tile) items, the tiles of one slice back to back ----
        auto first_tile = [&](int s) __attribute__((always_inline)) -> int {
            return max(tp_at(s / NS - e0), qa) - qa;
        };
        auto last_tile = [&](int s) __attribute__((always_inline)) -> int {
            return min(tp_at(s / NS - e0 + 1), qb) - qa - 1;
        };
        auto advance = [&](int& s, int& t) __attribute__((always_inline)) {
            if (t < last_tile(s)) {
                ++t;                            // the same slice again, against its next tile
            } else {
                s = next_valid(s + kWaves);
                t = s < b ? first_tile(s) : 0;
            }
        };
        int tc = sc < b ? first_tile(sc) : 0;
        int sn = sc, tn = tc;
        if (sc < b)
            advance(sn, tn);
        else
            sn = b;
        // one item; HN: item (sn, tn) follows and its weights are loaded as the ring frees up
        auto run = [&](auto hn_tag) __attribute__((always_inline)) {
            constexpr bool HN = decltype(hn_tag)::value;
            const int cs = sc - (sc / NS) * NS;
            const uint4* tb = L.frag[tc];
            const float* ts = L.sa[tc];
            float sbn[kKB];
            const uint8_t* wnxt = wcur;
            if (HN) {
                wnxt = slice_ptr(sn);
                slice_scales(sn, sbn);
            }
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
            v4f hprev = acc;
            float sprev = 0.0f;
            uint4 fb[2][2];                     // B fragments, read one k-block ahead
            fb[0][0] = tb[0 * 64 + lane];
            fb[0][1] = tb[1 * 64 + lane];
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
#pragma unroll
                for (int u = 0; u < kRing; ++u) {
                    const int kb = p * kRing + u;
                    if (kb + 1 < kKB) {
                        fb[(kb + 1) & 1][0] = tb[((kb + 1) * 2 + 0) * 64 + lane];
                        fb[(kb + 1) & 1][1] = tb[((kb + 1) * 2 + 1) * 64 + lane];
                    }
                    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f h = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        pack8v(wr0[u], wr1[u]), pack8(fb[kb & 1][0], fb[kb & 1][1]), zero, 0,
                        0, 0, 0, 0, 0);
                    // the unit's registers are free again: refill with the same k-block of the
                    // next pass, or of the next item (kept after the MFMA, so the loads land
                    // in the registers it has just read and the ring is never renamed)
                    __builtin_amdgcn_sched_barrier(0);
                    if (p + 1 < kPasses)
                        load_unit(wcur, kb + kRing, u);
                    else if (HN)
                        load_unit(wnxt, u, u);
                    __builtin_amdgcn_sched_barrier(0);
                    // the previous unit's product joins the sum now (its MFMA is long done),
                    // pinned here so that at most two products are ever live
                    if (kb > 0) {
                        acc += sprev * hprev;
                        asm volatile("" : "+v"(acc));
                    }
                    hprev = h;
                    sprev = ts[kb * 16 + j] * sbc[kb];
                }
            }
            acc += sprev * hprev;
            // C layout of the 16x16 MFMA: lane (j, g) holds output rows 4g..4g+3 (weight rows
            // of the slice) of column j (routed row j of the tile)
            if (j < L.trc[tc]) {
                const int route = L.list[L.tlb[tc] + j] & 0xFFF;
                *reinterpret_cast<float4*>(rows_out + (size_t)route * N + cs * 16 + g * 4) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
            sc = sn;
            tc = tn;
            if (HN) {
                advance(sn, tn);
                wcur = wnxt;
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb) sbc[kb] = sbn[kb];
            }
        };
        if (sc < b) {
            while (sn < b) run(std::true_type{});
            run(std::false_type{});             // the last item issues no loads
        }
        // every wave is done with the tiles before the next round rewrites them (LDS only:
        // the row stores may stay in flight)
        barrier_keep_vm<63>();
    }
}

}  // namespace

int fused_max_local_experts(int E, int N, int grid) {
    const long long slices = (long long)E * (N / 16);
    const long long span = (slices + grid - 1) / grid;
    return (int)((span + N / 16 - 1) / (N / 16)) + 1;
}

bool forward_fused_applies(int M, int k, int E, int K, int N, int chunk_rows) {
    return (K == 256 || K == 512 || K == 1024 || K == 2048) && chunk_rows == 16 && (long long)M * k <= kMaxRoutes && N % 128 == 0 &&
           fused_max_local_experts(E, N, device_info().cu_count) <= kMaxLocal;
}

bool fused_route_applies(int M, int k, int E) {
    return E <= 64 * kRouteVPL && (long long)M <= (long long)kWaves * device_info().cu_count &&
           k <= 64;
}

namespace {

// one launch of the kernel for K = 128 * KB
template <bool ROUTE, bool ACT>
hipError_t launch_fused_k(int K, const void* x, const int32_t* ids, int R, int k,
                          const uint8_t* w, const float* w_scales, int N, int slices,
                          float* rows_out, const FusedRoute& rt, const FusedAct& act,
                          hipStream_t s) {
    const int grid = device_info().cu_count;    // one 8-wave workgroup per CU
#define MOE_FUSED_LAUNCH(KB_)                                                                     \
    hipLaunchKernelGGL((gemm_fp8_fused_kernel<KB_, true, ROUTE, ACT>), dim3(grid),               \
                       dim3(kThreads), 0, s, x, ids, R, k, w, w_scales, N, slices, rows_out, rt, \
                       act)
    switch (K) {
        case 256: MOE_FUSED_LAUNCH(2); break;
        case 512: MOE_FUSED_LAUNCH(4); break;
        case 1024: MOE_FUSED_LAUNCH(8); break;
        case 2048: MOE_FUSED_LAUNCH(16); break;
        default: return hipErrorInvalidValue;
    }
#undef MOE_FUSED_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_fused(const uint16_t* x, const int32_t* ids, int M, int k, int E,
                                 int K, const uint8_t* w, const float* w_scales, int N,
                                 float* rows_out, hipStream_t s) {
    const FusedRoute none{};
    const FusedAct no_act{};
    return launch_fused_k<false, false>(K, x, ids, M * k, k, w, w_scales, N, E * (N / 16),
                                        rows_out, none, no_act, s);
}

hipError_t launch_gemm_fp8_fused_act(const float* h, const int32_t* ids, int M, int k, int E,
                                     int K, const uint8_t* w, const float* w_scales, int N,
                                     float* rows_out, uint8_t* a_q, float* a_s, hipStream_t s) {
    const FusedRoute none{};
    const FusedAct act{a_q, a_s};
    return launch_fused_k<false, true>(K, h, ids, M * k, k, w, w_scales, N, E * (N / 16),
                                       rows_out, none, act, s);
}

hipError_t launch_gemm_fp8_fused_route(const float* logits, const uint16_t* x, int M, int k,
                                       int E, int K, float softcap, const uint8_t* w,
                                       const float* w_scales, int N, int32_t* ids,
                                       float* weights, uint32_t* handoff, uint32_t* status,
                                       float* rows_out, bool self_route, hipStream_t s) {
    static std::atomic<uint32_t> epoch{0};
    const uint32_t tag = 0x7FA00000u | ((epoch.fetch_add(1) & 0xFFFu) << 8);
    // a routing wave normally publishes within a few microseconds; 4096 rounds of polls
    // (milliseconds) only run out when its workgroup waits for a CU another kernel holds
    const int max_polls = self_route ? 0 : 4096;
    // (one workgroup per CU: every token's routing wave is in the grid)
    const FusedRoute rt{logits, ids, weights, handoff, status, tag, max_polls, M, E, softcap};
    const FusedAct no_act{};
    return launch_fused_k<true, false>(K, x, nullptr, M * k, k, w, w_scales, N, E * (N / 16),
                                       rows_out, rt, no_act, s);
}

}  // namespace moe
