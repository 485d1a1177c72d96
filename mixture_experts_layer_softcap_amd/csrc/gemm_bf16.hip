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
// Operands.  Both tiles go from global memory straight into LDS with global_load_lds_dwordx4,
// in MFMA fragment order: fragment (32-row group g, 16-wide k step s) is 1 KiB, lane l's
// 16 bytes being row g*32 + l%32, k = s*16 + (l/32)*8 .. +8, so every operand read is one
// conflict-free ds_read_b128 and every DMA instruction reads 32-byte runs of 32 rows.  Two
// stages of 64 KiB alternate; one barrier per k step publishes a stage and frees the other.
// The operand reads are written as inline ds_read_b128 with explicit lgkmcnt waits tied to
// the fragment registers: the compiler cannot tell a DMA into one stage from reads of the
// other and would otherwise drain the DMA before every read.  Rows past rc repeat row rb
// (never stored).
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
constexpr int kGF = 8 * (kBK / 16);             // fragments per operand per stage (32)

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

// every LDS read issued so far has landed in the eight fragment registers
__device__ __forceinline__ void lds_wait(i32x4& a0, i32x4& a1, i32x4& a2, i32x4& a3,
                                         i32x4& b0, i32x4& b1, i32x4& b2, i32x4& b3) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b0), "+v"(b1), "+v"(b2),
                   "+v"(b3));
}

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
                      const int4* __restrict__ tasks, const int32_t* __restrict__ ntasks,
                      void* __restrict__ out, int K, int N) {
    __shared__ uint4 sA[2][kGF * 64];
    __shared__ uint4 sW[2][kGF * 64];
    const int task = blockIdx.x;
    if (task >= *ntasks) return;
    const int4 td = tasks[task];
    const int e = td.x, rb = td.y, rc = td.z, nb = td.w;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int j = lane & 31, h = lane >> 5;
    const int nk = K / kBK;

    // weight row of n-group g (32 rows) for this lane
    auto wrow = [&](int g) -> int {
        if (EPI == MOE_EPI_SWIGLU_BF16)
            return g < 4 ? nb * 128 + g * 32 + j : N / 2 + nb * 128 + (g - 4) * 32 + j;
        return nb * kBN + g * 32 + j;
    };
    // DMA sources: this wave moves row groups 2w and 2w+1 of both operands in every stage
    const uint16_t* srcA0 = a + (size_t)(rb + min(2 * wave * 32 + j, rc - 1)) * K + h * 8;
    const uint16_t* srcA1 = a + (size_t)(rb + min((2 * wave + 1) * 32 + j, rc - 1)) * K + h * 8;
    const uint16_t* srcW0 = w + ((size_t)e * N + wrow(2 * wave)) * K + h * 8;
    const uint16_t* srcW1 = w + ((size_t)e * N + wrow(2 * wave + 1)) * K + h * 8;

    auto issue = [&](int buf, int kt) {
        uint4* dA = sA[buf];
        uint4* dW = sW[buf];
        const int k0 = kt * kBK;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int f0 = (2 * wave) * 4 + s, f1 = (2 * wave + 1) * 4 + s;
            __builtin_amdgcn_global_load_lds(srcA0 + k0 + s * 16, (lds_void*)(dA + f0 * 64), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(srcA1 + k0 + s * 16, (lds_void*)(dA + f1 * 64), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(srcW0 + k0 + s * 16, (lds_void*)(dW + f0 * 64), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(srcW1 + k0 + s * 16, (lds_void*)(dW + f1 * 64), 16, 0, 0);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    // LDS byte addresses of this lane's fragments: A row groups 4wm.., W groups of this wave
    // ((4wn..) or, for SwiGLU, gate groups 2wn, 2wn+1 and up groups 4+2wn, 5+2wn)
    const uint32_t lA = (uint32_t)(uintptr_t)(lds_void*)&sA[0][(4 * wm) * 4 * 64 + lane];
    const int wg0 = EPI == MOE_EPI_SWIGLU_BF16 ? 2 * wn : 4 * wn;
    const int wg2 = EPI == MOE_EPI_SWIGLU_BF16 ? 4 + 2 * wn : 4 * wn + 2;
    const uint32_t lW0 = (uint32_t)(uintptr_t)(lds_void*)&sW[0][wg0 * 4 * 64 + lane];
    const uint32_t lW2 = (uint32_t)(uintptr_t)(lds_void*)&sW[0][wg2 * 4 * 64 + lane];
    constexpr uint32_t kStage = kGF * 64 * 16;  // bytes per stage buffer
    constexpr int kG = 4 * 1024;                // bytes between row groups (4 k steps)

    auto compute = [&](uint32_t boff) {
        const uint32_t pa = lA + boff, pw0 = lW0 + boff, pw2 = lW2 + boff;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            i32x4 fa0, fa1, fa2, fa3, fw0, fw1, fw2, fw3;
            switch (s) {
#define MOE_READS(S)                                                         \
    case S:                                                                  \
        fa0 = lds_read16<0 * kG + S * 1024>(pa);                             \
        fa1 = lds_read16<1 * kG + S * 1024>(pa);                             \
        fa2 = lds_read16<2 * kG + S * 1024>(pa);                             \
        fa3 = lds_read16<3 * kG + S * 1024>(pa);                             \
        fw0 = lds_read16<0 * kG + S * 1024>(pw0);                            \
        fw1 = lds_read16<1 * kG + S * 1024>(pw0);                            \
        fw2 = lds_read16<0 * kG + S * 1024>(pw2);                            \
        fw3 = lds_read16<1 * kG + S * 1024>(pw2);                            \
        break;
                MOE_READS(0) MOE_READS(1) MOE_READS(2) MOE_READS(3)
#undef MOE_READS
            }
            lds_wait(fa0, fa1, fa2, fa3, fw0, fw1, fw2, fw3);
            const bf16x8 A[4] = {as_bf16x8(fa0), as_bf16x8(fa1), as_bf16x8(fa2), as_bf16x8(fa3)};
            const bf16x8 B[4] = {as_bf16x8(fw0), as_bf16x8(fw1), as_bf16x8(fw2), as_bf16x8(fw3)};
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B[ni], A[mi],
                                                                         acc[mi][ni], 0, 0, 0);
        }
    };

    // k step kt on buffer kt%2: wait for it (the DMA of step kt+1 is not issued yet), publish
    // it and free the other buffer, start step kt+1 there, compute
    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        barrier_after_vmcnt<0>();
        if (kt + 1 < nk) issue((kt + 1) & 1, kt + 1);
        compute((kt & 1) ? kStage : 0u);
    }

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
                            int epilogue, void* out, hipStream_t s) {
    if (max_tasks <= 0) return hipSuccess;
    const int4* t = reinterpret_cast<const int4*>(tasks);
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            hipLaunchKernelGGL(gemm_bf16_kernel<MOE_EPI_STORE_BF16>, dim3(max_tasks),
                               dim3(kThreads), 0, s, a, w, t, ntasks, out, K, N);
            break;
        case MOE_EPI_SWIGLU_BF16:
            hipLaunchKernelGGL(gemm_bf16_kernel<MOE_EPI_SWIGLU_BF16>, dim3(max_tasks),
                               dim3(kThreads), 0, s, a, w, t, ntasks, out, K, N);
            break;
        default:
            hipLaunchKernelGGL(gemm_bf16_kernel<MOE_EPI_STORE_F32>, dim3(max_tasks),
                               dim3(kThreads), 0, s, a, w, t, ntasks, out, K, N);
    }
    return hipGetLastError();
}

}  // namespace moe
