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
// step's fragments are read during the previous step's MFMAs.  The operand reads are inline
// ds_read_b128 with explicit lgkmcnt waits tied to the fragment registers: the compiler
// cannot tell a DMA into one stage from reads of the other and would otherwise drain the DMA
// before every read.
// Rows past rc repeat row rb + rc - 1 (never stored).  With a sorted route list the A rows
// are gathered on load: sorted row s is token row sorted[s] / k of the layer input, so no
// expert-sorted copy of the input is written first.
//
// Order.  Workgroups go round-robin over the 8 XCDs; each XCD takes one contiguous run of the
// chunk-major task list, regrouped so that the tiles it runs together cover a few chunks x a
// few panels (fewer distinct operand slices per k step in its L2).
//
// Epilogues.  STORE_F32 / STORE_BF16 write h; SWIGLU_BF16 computes a 128-column block of
// act = bf16(silu(g) * u) from the gate columns [nb*128, nb*128+128) and the up columns
// [N/2 + nb*128, ...) of the same task (each wave holds 64 gate columns and their up columns).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
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

// one 16-byte LDS read at byte address addr + OFF (issued now, waited for by lds_wait)
template <int OFF>
__device__ __forceinline__ i32x4 lds_read16(uint32_t addr) {
    i32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// The LDS reads issued before the last N (of this wave) have landed in the eight fragment
// registers.  The registers are in-out operands of the wait, so the compiler cannot use or
// move their values before it; reads stay in one asm statement each and nothing else touches
// a fragment register between its read and its wait.
template <int N>
__device__ __forceinline__ void lds_wait(i32x4& a0, i32x4& a1, i32x4& a2, i32x4& a3,
                                         i32x4& b0, i32x4& b1, i32x4& b2, i32x4& b3) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b0), "+v"(b1), "+v"(b2),
                   "+v"(b3)
                 : "i"(N));
}

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
                      const int4* __restrict__ tasks, const int32_t* __restrict__ ntasks,
                      void* __restrict__ out, int K, int N, int pw, int gch,
                      const int32_t* __restrict__ sorted, int kr) {
    __shared__ uint4 sA[2][kBM * 8];             // routed rows: 2 stages x 256 x 128 bytes
    __shared__ uint4 sW[3][kBN * 8];             // weights: three stages
    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs, so workgroup b
    // runs on XCD b%8; each XCD takes one contiguous run of the (chunk-major) task list, so
    // the tiles running together on an XCD share routed-row chunks and weight panels, and
    // walk K in near lockstep, out of that XCD's L2.
    const int nt = *ntasks;
    const int per_xcd = (nt + 7) >> 3;
    const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per_xcd || t >= nt) return;
    // Inside a run, gch consecutive chunks (same expert where possible) are taken pw panels
    // at a time: the ~32 tiles an XCD runs together then cover gch chunks x pw panels, so
    // each k step asks its L2 for gch + pw distinct slices instead of ~3 + N/256.
    const int nbk = N / kBN;                    // tasks per chunk (both epilogue layouts)
    const int grp = t / (gch * nbk);
    const int gc = min(gch, nt / nbk - grp * gch);
    int i = t - grp * gch * nbk;
    const int pb = i / (gc * pw);
    const int pwb = min(pw, nbk - pb * pw);
    i -= pb * gc * pw;
    const int task = (grp * gch + i / pwb) * nbk + pb * pw + i % pwb;
    const int4 td = tasks[task];
    const int e = td.x, rb = td.y, rc = td.z, nb = td.w;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int j = lane & 31, h = lane >> 5;
    const int nk = K / kBK;

    // Operand tiles in LDS, per stage: [256 rows][128 bytes] for A and for W (the stage's 64
    // k values of each row), the 16-byte chunk c of row r stored at position c ^ ((r/2) % 8).
    // A DMA instruction moves 8 whole 128-byte row segments (lane l: row l/8, position l%8);
    // every line it touches is read in full.  The LDS serves a 16-byte read for 16 lanes per
    // clock over 64 four-byte banks, i.e. two 128-byte rows side by side: an MFMA fragment read
    // (lanes j..j+15 of one half h: rows g*32 + j, one chunk 2s + h) then has rows of equal
    // parity at 8 distinct positions, so it is free of bank conflicts.
    const int dl = lane >> 3;                   // row within a DMA instruction
    const uint16_t* srcA[8];
    const uint16_t* srcW[8];
    // A row of tile row r: sorted row rb + r, or with a sorted route list the token row it was
    // routed from (the eight lookups issued together)
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

    // Fragment read addresses, per 16-wide k step s: row j of a 32-row group, chunk 2s + h at
    // its swizzled position; A groups 4wm.., W groups of this wave ((4wn..) or, for SwiGLU,
    // gate groups 2wn, 2wn+1 and up groups 4+2wn, 5+2wn)
    const int wg0 = EPI == MOE_EPI_SWIGLU_BF16 ? 2 * wn : 4 * wn;
    const int wg2 = EPI == MOE_EPI_SWIGLU_BF16 ? 4 + 2 * wn : 4 * wn + 2;
    const uint32_t baseA = (uint32_t)(uintptr_t)(lds_void*)&sA[0][0];
    const uint32_t baseW = (uint32_t)(uintptr_t)(lds_void*)&sW[0][0];
    uint32_t pa[4], pw0[4], pw2[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const uint32_t in_row = (uint32_t)(j * 128 + (((2 * st + h) ^ ((j >> 1) & 7)) << 4));
        pa[st] = baseA + (uint32_t)(4 * wm) * 4096u + in_row;
        pw0[st] = baseW + (uint32_t)wg0 * 4096u + in_row;
        pw2[st] = baseW + (uint32_t)wg2 * 4096u + in_row;
    }
    constexpr uint32_t kStage = 256 * 128;      // bytes per stage buffer

    // One k step from buffer boff.  With DMA, the next step's 16 DMA instructions are spread
    // over the step's 64 MFMAs (one after every fourth): a wave issues in order, and a burst
    // of DMA instructions stalls it on the memory pipeline long enough to hold back its
    // MFMAs, so the two would otherwise run one after the other.
    // Fragments of one 16-wide k step: 4 of A, 4 of W
    struct Frag {
        i32x4 a0, a1, a2, a3, w0, w1, w2, w3;
    };
    auto read_frags = [&](Frag& f, uint32_t boffA, uint32_t boffW, int st)
                          __attribute__((always_inline)) {
        const uint32_t qa = pa[st] + boffA, qw0 = pw0[st] + boffW, qw2 = pw2[st] + boffW;
        f.a0 = lds_read16<0 * 4096>(qa);
        f.a1 = lds_read16<1 * 4096>(qa);
        f.a2 = lds_read16<2 * 4096>(qa);
        f.a3 = lds_read16<3 * 4096>(qa);
        f.w0 = lds_read16<0>(qw0);
        f.w1 = lds_read16<4096>(qw0);
        f.w2 = lds_read16<0>(qw2);
        f.w3 = lds_read16<4096>(qw2);
    };

    // One k step from buffer boff: the fragments of 16-wide step st+1 are read while the
    // MFMAs of step st run.  With DMA, the next k step's 16 DMA instructions go out one after
    // every second MFMA of the step's first half, from the first on: a wave issues in order,
    // and a burst of DMA instructions stalls it on the memory pipeline long enough to hold
    // back its MFMAs, while DMA issued late in the step leaves its latency to the next
    // barrier (one per fourth MFMA over the whole step measured 3-7 % slower, one per third
    // 1-3 % slower).
    auto compute = [&](uint32_t boffA, uint32_t boffW, int nbufA, int nbufW, int nktA,
                       int nktW, auto dma_a, auto dma_w) {
        uint4* dA = sA[nbufA];
        uint4* dW = sW[nbufW];
        const int k0A = nktA * kBK, k0W = nktW * kBK;
        Frag f[2];
        read_frags(f[0], boffA, boffW, 0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            Frag& c = f[st & 1];
            if (st < 3) {
                read_frags(f[(st + 1) & 1], boffA, boffW, st + 1);
                lds_wait<8>(c.a0, c.a1, c.a2, c.a3, c.w0, c.w1, c.w2, c.w3);
            } else {
                lds_wait<0>(c.a0, c.a1, c.a2, c.a3, c.w0, c.w1, c.w2, c.w3);
            }
            const bf16x8 A[4] = {as_bf16x8(c.a0), as_bf16x8(c.a1), as_bf16x8(c.a2),
                                 as_bf16x8(c.a3)};
            const bf16x8 B[4] = {as_bf16x8(c.w0), as_bf16x8(c.w1), as_bf16x8(c.w2),
                                 as_bf16x8(c.w3)};
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B[ni], A[mi],
                                                                         acc[mi][ni], 0, 0, 0);
                    {
                        const int m = st * 16 + mi * 4 + ni;     // MFMA index in the step
                        if (m % 2 == 0 && m / 2 < 16) {
                            const int q = m / 2;                     // DMA slot 0..15
                            if (q < 8) {
                                if constexpr (decltype(dma_a)::value)
                                    __builtin_amdgcn_global_load_lds(
                                        srcA[q] + k0A, (lds_void*)(dA + (wave * 64 + q * 8) * 8),
                                        16, 0, 0);
                            } else {
                                if constexpr (decltype(dma_w)::value)
                                    __builtin_amdgcn_global_load_lds(
                                        srcW[q - 8] + k0W,
                                        (lds_void*)(dW + (wave * 64 + (q - 8) * 8) * 8), 16, 0,
                                        0);
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // Weights run two steps ahead (three stages), routed rows one (two stages).  Step kt
    // issues A(kt+1), then W(kt+2); its barrier waits for A(kt) and W(kt), leaving W(kt+1)
    // (the newest 8 DMA instructions) in flight.
    auto issueA = [&](int buf, int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(srcA[i] + k0,
                                             (lds_void*)(sA[buf] + (wave * 64 + i * 8) * 8), 16,
                                             0, 0);
    };
    auto issueW = [&](int buf, int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(srcW[i] + k0,
                                             (lds_void*)(sW[buf] + (wave * 64 + i * 8) * 8), 16,
                                             0, 0);
    };
    using T = std::integral_constant<bool, true>;
    issueA(0, 0);
    issueW(0, 0);
    issueW(1, min(1, nk - 1));
    int bw = 0;                                 // kt % 3
    for (int kt = 0; kt < nk; ++kt) {
        // A(kt) and W(kt) have landed; W(kt+1) (the newest 8) may still be in flight.  Past
        // the end the DMA repeats the last stage into a free buffer (never read).
        barrier_after_vmcnt<8>();
        const uint32_t bA = (kt & 1) ? kStage : 0u, bW = (uint32_t)bw * kStage;
        const int bw2 = bw == 0 ? 2 : bw - 1;   // (kt + 2) % 3
        compute(bA, bW, (kt + 1) & 1, bw2, min(kt + 1, nk - 1), min(kt + 2, nk - 1), T{}, T{});
        bw = bw == 2 ? 0 : bw + 1;
    }
    // no DMA may still write this workgroup's LDS when it exits
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
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* a, int K, const uint16_t* w, int N,
                            const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                            int epilogue, void* out, hipStream_t s, const int32_t* sorted,
                            int kr) {
    if (max_tasks <= 0) return hipSuccess;
    const int4* t = reinterpret_cast<const int4*>(tasks);
    const int grid = (max_tasks + 7) / 8 * 8;    // whole rounds of the 8 XCDs
    // tile groups of ~32 (one XCD's CUs): up to 4 panels x 32/4 chunks (8 x 4 and 12 x 2 were
    // 1-4 % slower with three weight stages)
    const int pw = min(4, N / kBN);
    const int gch = 32 / pw;
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            hipLaunchKernelGGL(gemm_bf16_kernel<MOE_EPI_STORE_BF16>, dim3(grid),
                               dim3(kThreads), 0, s, a, w, t, ntasks, out, K, N, pw, gch,
                               sorted, kr);
            break;
        case MOE_EPI_SWIGLU_BF16:
            hipLaunchKernelGGL(gemm_bf16_kernel<MOE_EPI_SWIGLU_BF16>, dim3(grid),
                               dim3(kThreads), 0, s, a, w, t, ntasks, out, K, N, pw, gch,
                               sorted, kr);
            break;
        default:
            hipLaunchKernelGGL(gemm_bf16_kernel<MOE_EPI_STORE_F32>, dim3(grid),
                               dim3(kThreads), 0, s, a, w, t, ntasks, out, K, N, pw, gch,
                               sorted, kr);
    }
    return hipGetLastError();
}

}  // namespace moe
