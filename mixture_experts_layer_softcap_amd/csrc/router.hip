// router.hip -- the router projection ahead of the route ([WEAVE] section 3.1 counts the gate
// in the layer's forward): logits[t][e] = sum_h x[t][h] * w_gate[e][h], bf16 operands, fp32
// accumulate, fp32 logits.
//
// The operation is a skinny GEMM (E = 8..1024 columns) that is bound by reading x and w_gate,
// so it runs straight from global memory without LDS staging: per 64-wide k step a lane loads
// 2 x 16 bytes of one gate row and 2 x 16 bytes of one token row (each row's 128 bytes read
// by 4 lanes, whole cache lines), and feeds v_mfma_f32_16x16x32_bf16 with gate rows as the
// 16-row A side and tokens as the B side, so a lane ends with 4 consecutive logits of one
// token per 16 x 16 block.  A workgroup owns 16*TB tokens x 16*EB experts, every wave all of
// them, so a k step's TB + EB row loads feed TB * EB block products; its 4 waves split K in
// contiguous quarters and sum their fp32 partials through LDS in wave order, so the result
// does not depend on timing.  Token rows past M and gate rows past E repeat the last row and
// are not stored.
//
// A workgroup reads 2 * H * 16 * (TB + EB) bytes, which each CU fetches at the rate its few
// KB of reads in flight allow, so the launcher takes the largest tile that still gives every
// CU a workgroup.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int TB, int EB>
__global__ __launch_bounds__(kWaves * 64) void router_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wg,
                                                             int M, int H, int E,
                                                             float* __restrict__ logits) {
    constexpr int kRing = TB + EB <= 2 ? 4 : 2;   // 64-wide k steps in flight per wave
    __shared__ v4f s_part[kWaves - 1][TB * EB][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, g = lane >> 4;
    // workgroup i runs on XCD i % 8 (round-robin dispatch); when the expert blocks divide
    // evenly over the 8 XCDs, all token blocks of one expert block go to the same XCD, so its
    // gate rows come from HBM once and are re-read from that XCD's L2
    const int ntb = (M + 16 * TB - 1) / (16 * TB), neb = gridDim.x / ntb;
    int tb = blockIdx.x % ntb, eb = blockIdx.x / ntb;
    if ((neb & 7) == 0) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        tb = slot % ntb;
        eb = xcd + 8 * (slot / ntb);
    }
    const int t0 = tb * 16 * TB;
    const int e0 = eb * 16 * EB;
    const int nsteps = H >> 6;
    const int s0 = nsteps * wave / kWaves, s1 = nsteps * (wave + 1) / kWaves;

    // this lane's rows: tokens t0 + 16i + j (B side) and gate rows e0 + 16b + j (A side),
    // bytes [16g, 16g+16) and [64+16g, 64+16g+16) of every 128-byte k step
    const uint16_t* xr[TB];
    const uint16_t* wr[EB];
#pragma unroll
    for (int i = 0; i < TB; ++i) xr[i] = x + (size_t)min(t0 + 16 * i + j, M - 1) * H + g * 8;
#pragma unroll
    for (int b = 0; b < EB; ++b) wr[b] = wg + (size_t)min(e0 + 16 * b + j, E - 1) * H + g * 8;

    v4f acc[TB][EB];
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int b = 0; b < EB; ++b) acc[i][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    struct Unit {
        uint4 x0[TB], x1[TB], w0[EB], w1[EB];
    };
    Unit ring[kRing];
    auto load = [&](Unit& u, int s) __attribute__((always_inline)) {
        const int k = s * 64;
#pragma unroll
        for (int b = 0; b < EB; ++b) {
            u.w0[b] = *reinterpret_cast<const uint4*>(wr[b] + k);
            u.w1[b] = *reinterpret_cast<const uint4*>(wr[b] + k + 32);
        }
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            u.x0[i] = *reinterpret_cast<const uint4*>(xr[i] + k);
            u.x1[i] = *reinterpret_cast<const uint4*>(xr[i] + k + 32);
        }
    };
    // (loads past s1 repeat the last step so every lane issues the same loads; never used)
#pragma unroll
    for (int r = 0; r < kRing; ++r) load(ring[r], min(s0 + r, max(s1 - 1, s0)));
    for (int s = s0; s < s1; s += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            if (s + r < s1) {
                const Unit u = ring[r];
#pragma unroll
                for (int i = 0; i < TB; ++i)
#pragma unroll
                    for (int b = 0; b < EB; ++b) {
                        acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(u.w0[b]), as_bf16x8(u.x0[i]), acc[i][b], 0, 0, 0);
                        acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(u.w1[b]), as_bf16x8(u.x1[i]), acc[i][b], 0, 0, 0);
                    }
                load(ring[r], min(s + r + kRing, s1 - 1));
            }
        }
    }

    // partials of waves 1..3 to LDS; wave 0 adds them in wave order and stores
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < TB; ++i)
#pragma unroll
            for (int b = 0; b < EB; ++b) s_part[wave - 1][i * EB + b][lane] = acc[i][b];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < TB; ++i) {
#pragma unroll
        for (int b = 0; b < EB; ++b) {
            v4f v = acc[i][b];
#pragma unroll
            for (int w = 0; w < kWaves - 1; ++w) v += s_part[w][i * EB + b][lane];
            // C layout of the 16x16 MFMA: lane (j, g) holds rows 4g..4g+3 (gate rows, i.e.
            // experts) of column j (token)
            const int t = t0 + 16 * i + j, e = e0 + 16 * b + 4 * g;
            if (t < M && e < E) {
                float* o = logits + (size_t)t * E + e;
                if (e + 3 < E && (E & 3) == 0) {
                    *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (e + q < E) o[q] = v[q];
                }
            }
        }
    }
}

template <int TB, int EB>
long long router_grid(int M, int E) {
    return (long long)((M + 16 * TB - 1) / (16 * TB)) * ((E + 16 * EB - 1) / (16 * EB));
}

template <int TB, int EB>
void router_launch(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                   float* logits, hipStream_t s) {
    hipLaunchKernelGGL((router_kernel<TB, EB>), dim3((unsigned)router_grid<TB, EB>(M, E)),
                       dim3(kWaves * 64), 0, s, x, w_gate, M, H, E, logits);
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                                float* logits, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (router_grid<1, 1>(M, E) > 0x7FFFFFFFLL) return hipErrorInvalidValue;   // one grid
    // the largest tile (fewest bytes per logit) whose grid still covers every CU
    const long long cus = device_info().cu_count;
    if (E > 32 && router_grid<4, 4>(M, E) >= cus) {
        router_launch<4, 4>(x, M, H, w_gate, E, logits, s);
    } else if (E > 32 && router_grid<2, 4>(M, E) >= cus) {
        router_launch<2, 4>(x, M, H, w_gate, E, logits, s);
    } else if (router_grid<4, 1>(M, E) >= cus) {
        router_launch<4, 1>(x, M, H, w_gate, E, logits, s);
    } else if (router_grid<2, 1>(M, E) >= cus) {
        router_launch<2, 1>(x, M, H, w_gate, E, logits, s);
    } else {
        router_launch<1, 1>(x, M, H, w_gate, E, logits, s);
    }
    return hipGetLastError();
}

}  // namespace moe
