// wquant.hip -- 128x128 blockwise E4M3 quantisation of fp32 expert weights ([FMF8] problem
// table: FP8 E4M3 weights with 128x128 quantisation blocks; Baseline item 4 gives the rule
// scale = amax/448, value * (1/scale)).  Weight preparation, off the timed path.
//
// One 256-thread workgroup per block: thread (row group, column quad) reads 16 float4 so that
// each wave load covers 8 rows x 512 contiguous bytes; amax is a wave reduction plus four
// LDS slots; codes go out as 4-byte stores, 8 rows x 128 bytes per wave store.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void wquant_kernel(const float* __restrict__ w, int N, int K,
                                                     uint8_t* __restrict__ w_q,
                                                     float* __restrict__ w_scales) {
    __shared__ float s_max[4];
    const int Nb = N >> 7, Kb = K >> 7;
    const int blk = blockIdx.x;
    const int kb = blk % Kb;
    const int nb = (blk / Kb) % Nb;
    const int e = blk / (Kb * Nb);
    const int tid = threadIdx.x;
    const int c4 = tid & 31;          // column quad inside the block
    const int r0 = tid >> 5;          // first row, then every 8th row

    const size_t base = ((size_t)e * N + (size_t)nb * 128) * K + (size_t)kb * 128 + c4 * 4;
    float4 v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[i] = *reinterpret_cast<const float4*>(w + base + (size_t)(r0 + 8 * i) * K);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                 fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) s_max[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const QScale q = block_scale(amax);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t c =
            e4m3_encode4(v[i].x * q.inv, v[i].y * q.inv, v[i].z * q.inv, v[i].w * q.inv);
        *reinterpret_cast<uint32_t*>(w_q + base + (size_t)(r0 + 8 * i) * K) = c;
    }
    if (tid == 0) w_scales[((size_t)e * Nb + nb) * Kb + kb] = q.scale;
}

}  // namespace

hipError_t launch_quantize_weights(const float* w, int E, int N, int K, uint8_t* w_q,
                                   float* w_scales, hipStream_t s) {
    const size_t blocks = (size_t)E * (N / 128) * (K / 128);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(wquant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K, w_q,
                       w_scales);
    return hipGetLastError();
}

}  // namespace moe
